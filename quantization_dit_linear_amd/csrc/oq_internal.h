// oq_internal.h -- definitions shared by the host side of liborbitquant and
// its HIP kernels (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace oq {

// Raise a kernel's dynamic-LDS limit on the current device, once per device
// (`done` holds one bit per device id; setting the attribute twice from two
// threads is harmless).
inline hipError_t ensure_lds_limit(const void *fn, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

constexpr int kMaxD = 16384;
constexpr int kGroup = 128;  // coordinates per storage-order group
// token lengths d: multiples of kDimStep (a last partial group of 32, 64 or
// 96 coordinates is stored in coordinate order); linear K: multiples of the
// linear's 64-slot K step
constexpr int kDimStep = 32;
constexpr int kLinearKStep = 64;

// Slot size of the bf16 fast rotate kernel for token size d: the Hadamard
// block, at most 1024 coordinates (a block of 2048 or 4096 spans several
// slots), 512 at d = 5120 and 3072 (a batch of two tokens then tiles the
// kernel's compute waves).  The host lays out the kernel's LDS copy of a
// token by slots, so both sides take the size from here.
constexpr __host__ __device__ int fast_slot(int d) {
  const int h = d & -d, cap = (d == 5120 || d == 3072) ? 512 : 1024;
  return h < cap ? h : cap;
}

// Unit-variance decision thresholds of one codebook (fp32, ascending).
struct Thresholds {
  float t[15];
  int count;  // 2^bits - 1
};

// Unit-variance levels of one codebook, as fp16 bit patterns.
struct LevelsF16 {
  uint16_t v[16];
};

// Unit-variance levels of one codebook, fp32 (dequantized outputs).
struct LevelsF32 {
  float v[16];
};

// Device-side rotation plan for one (device, d, seed).
struct DevicePlan {
  int d = 0, h = 0;
  // scatter table for the generic kernel: entry j = pi^-1(j), bit 31 set when
  // the sign applied at that destination is negative.
  int32_t *scatter = nullptr;         // with signs
  int32_t *scatter_nosign = nullptr;  // signs dropped
  // tables of the bf16 fast path: byte offset 2 pi^-1(j) of every source
  // element j inside a token's LDS copy, and per source dword the XOR mask
  // that applies the destination's sign to both bf16 halves.
  uint32_t *fast_scatter = nullptr;
  uint32_t *fast_signs = nullptr;
  uint32_t *fast_nosigns = nullptr;
  // input already in rotation order (x'_i = x_{pi(i)}): identity placement
  int32_t *scatter_id = nullptr;   // generic kernel: j | sign bit of D_j
  uint32_t *fast_signs_id = nullptr;  // fast path: per dword pair, signs of D_j, D_j+1
  int32_t *perm_inv = nullptr;     // pi^-1 (row permutation of oq_permute_rows)
  int pins = 0;  // explicit handles (oq_plan_create) holding this plan
};

struct RotateArgs {
  const void *x;
  int dtype;  // 0 fp32, 1 bf16
  int64_t n_tok;
  int d, h, bits;
  bool signs;
  bool rotated_out;  // fp32 rotated unit vector instead of codes
  bool dequant_out;  // bf16 s * level[code] instead of codes
  bool input_permuted;  // x already in rotation order: D and H only
  LevelsF32 levels;  // unit levels (dequant_out)
  void *out;
  float *norms;
  hipStream_t stream;
};

// Kernel launchers (defined in the .hip files).  Return a hipError_t.
// General kernel.  Up to 4 bits the codebook comes in th and a.levels; at 8
// bits from the device table (layout above).
hipError_t launch_rotate_quantize_generic(const RotateArgs &a, const DevicePlan &p,
                                          const Thresholds &th, const uint32_t *table);
// bf16 fast path; sets *handled = false (and does nothing) for shapes it does
// not cover.  table: the device codebook table of a.bits (layout above).
hipError_t launch_rotate_quantize_fast(const RotateArgs &a, const uint32_t *scat,
                                       const uint32_t *smask, const uint32_t *table,
                                       bool *handled);
// Device codebook table of one (bits, family, d): the fast path's cell grid
// ({tau, base} per cell), then the 2^bits unit levels (fp32), then the
// 2^bits - 1 unit thresholds (fp32), all as 32-bit words.  The grid is 1/8
// of a unit over [-130, 130) up to 4 bits -- every sqrt(d) z of a unit
// vector with d <= 16384 lies inside, so a kernel needs no clamp -- and
// 1/128 over [-5, 5) at 8 bits.
constexpr int kFastHalfUnits = 130;
constexpr int kFastCells = 16 * kFastHalfUnits;
constexpr int kFastCells8 = 1280;
constexpr __host__ __device__ int cells_for_bits(int bits) {
  return bits == 8 ? kFastCells8 : kFastCells;
}
constexpr __host__ __device__ int table_levels_word(int bits) { return 2 * cells_for_bits(bits); }
constexpr __host__ __device__ int table_thresholds_word(int bits) {
  return 2 * cells_for_bits(bits) + (1 << bits);
}

struct LinearArgs {
  const uint8_t *a_codes;
  const float *a_norms;
  int a_bits;
  const uint8_t *w_codes;
  const float *w_norms;
  int w_bits;
  int64_t M, N;
  int K;
  uint16_t *y;
  hipStream_t stream;
};

// Up to 4 bits the levels come as fp16 bit patterns in la / lw; at 8 bits
// as the fp32 unit levels of the device tables ta / tw (layout above).
hipError_t launch_linear(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw,
                         const uint32_t *ta, const uint32_t *tw);

// INT4 weight-only round-to-nearest (AdaLN projections)
hipError_t launch_rtn4_prepare(const void *W, int dtype, int64_t rows, int d, uint8_t *q4,
                               float *scales, hipStream_t stream);
hipError_t launch_rtn4_linear(const void *x, int dtype, int64_t M, const uint8_t *q4,
                              const float *scales, int64_t N, int K, uint16_t *y,
                              hipStream_t stream);

// dst row pi^-1(j) = src row j, i.e. dst[i] = src[pi(i)], rows of row_bytes
hipError_t launch_permute_rows(const void *src, void *dst, int64_t rows, int64_t row_bytes,
                               const int32_t *perm_inv, hipStream_t stream);

}  // namespace oq
