// adaln_rtn4.hip -- INT4 weight-only round-to-nearest for the AdaLN
// modulation projections.
//
// A rotation cannot be folded into a dynamic modulation projection, so its
// weights are kept at INT4 with plain round-to-nearest and its activations
// unquantized (paper.gecl.asia notes, Method item 5; researchpod.app
// transcript).  Per output row n: amax = max_k |W_nk|, scale_n = amax / 7,
// q_nk = rint(W_nk * (7 / amax)) in [-7, 7] (fp32, ties to even), stored
// offset-binary (nibble q + 8), two per byte, the even coordinate in the low
// nibble.  The projection y[m][n] = bf16(scale_n sum_k x_mk q_nk)
// accumulates in fp32 over the exact products x q.  The kernels are bound by
// HBM and latency: the modulation input is a handful of rows (one per
// sample), so the weights are read once.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "oq_internal.h"

namespace oq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_in(const void *x, int dtype, int64_t idx) {
  if (dtype == 1) return __uint_as_float((uint32_t)((const uint16_t *)x)[idx] << 16);
  return ((const float *)x)[idx];
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One workgroup per row (grid-stride); each thread packs 8 coordinates into
// one 32-bit word.
__global__ __launch_bounds__(256) void rtn4_prepare_kernel(const void *__restrict__ W, int dtype,
                                                           int64_t rows, int d,
                                                           uint32_t *__restrict__ q4,
                                                           float *__restrict__ scales) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    float amax = 0.f;
    for (int k = tid; k < d; k += 256) amax = fmaxf(amax, fabsf(load_in(W, dtype, r * d + k)));
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red is reused by the next row
    // the same fp32 operations as the definition: IEEE division, one product,
    // round half to even
    const float inv = amax > 0.f ? __fdiv_rn(7.0f, amax) : 0.f;
    if (tid == 0) scales[r] = __fdiv_rn(amax, 7.0f);
    for (int w8 = tid; w8 < d / 8; w8 += 256) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float t = load_in(W, dtype, r * d + 8 * w8 + e) * inv;
        const int qv = (int)__builtin_rintf(t);
        word |= (uint32_t)(qv + 8) << (4 * e);
      }
      q4[r * (d / 8) + w8] = word;
    }
  }
}

constexpr int kRows = 16;       // output rows per workgroup (16 threads each)
constexpr int kXBytes = 65536;  // LDS for a block of activation rows (fp32)
constexpr int kMaxMB = 8;       // activation rows per block (accumulators per thread)
constexpr int kPad = 36;        // floats per 32-coordinate chunk in LDS: the 16 lanes of a
                                // row read 16 chunks at once, 144 bytes apart, in distinct banks

// y[m][n]: persistent workgroups stage a block of mb <= 8 activation rows in
// LDS (fp32) once, then walk groups of 16 weight rows; 16 threads per row
// stride over 32-coordinate chunks (16 bytes of codes).  Nibbles become
// floats with byte conversions; the offset 8 is removed per value, so the
// fp32 sum runs over the exact products x q.  Each activation block re-reads
// the weights (the modulation input has one row per sample).
__global__ __launch_bounds__(256) void rtn4_linear_kernel(const void *__restrict__ x, int dtype,
                                                          int64_t M, const u32x4 *__restrict__ q4,
                                                          const float *__restrict__ scales,
                                                          int64_t N, int K, int mb,
                                                          uint16_t *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  const int tid = threadIdx.x, r = tid >> 4, j = tid & 15;
  const int chunks = K / 32;
  const int64_t groups = (N + kRows - 1) / kRows;
  for (int64_t m0 = 0; m0 < M; m0 += mb) {
    const int mcount = (int)((M - m0) < mb ? (M - m0) : mb);
    __syncthreads();  // the previous block's reads are done
    // 8 consecutive coordinates per thread and step (K % 32 == 0), four
    // steps' loads issued before their stores
    const int n8 = mcount * K / 8;
    for (int i0 = tid; i0 < n8; i0 += 4 * 256) {
      float v[4][8];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const int i = i0 + 256 * t;
        if (i < n8) {
          const int64_t base = m0 * K + 8 * (int64_t)i;
          if (dtype == 1) {
            const u32x4 w = *(const u32x4 *)((const uint16_t *)x + base);
#pragma unroll
            for (int e = 0; e < 4; e++) {
              v[t][2 * e] = __uint_as_float(w[e] << 16);
              v[t][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
          } else {
            const floatx4 a = *(const floatx4 *)((const float *)x + base);
            const floatx4 b = *(const floatx4 *)((const float *)x + base + 4);
#pragma unroll
            for (int e = 0; e < 4; e++) {
              v[t][e] = a[e];
              v[t][4 + e] = b[e];
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const int i = i0 + 256 * t;
        if (i < n8) {
          // coordinate 8i of the block = row u, chunk c, offset 8 (i % 4)
          floatx4 *d = (floatx4 *)(xs + (i / 4) * kPad + 8 * (i % 4));
          d[0] = floatx4{v[t][0], v[t][1], v[t][2], v[t][3]};
          d[1] = floatx4{v[t][4], v[t][5], v[t][6], v[t][7]};
        }
      }
    }
    __syncthreads();
    for (int64_t g = blockIdx.x; g < groups; g += gridDim.x) {
      const int64_t n = g * kRows + r;
      const u32x4 *qrow = q4 + (n < N ? n : N - 1) * chunks;
      float acc[kMaxMB];
#pragma unroll
      for (int u = 0; u < kMaxMB; u++) acc[u] = 0.f;
      // chunks j, j + 16, ... in batches of 8: all loads of a batch are
      // issued before any of them is used
      for (int c0 = j; c0 < chunks; c0 += 16 * 8) {
        u32x4 wv[8];
#pragma unroll
        for (int t = 0; t < 8; t++) {
          const int c = c0 + 16 * t;
          wv[t] = c < chunks ? qrow[c] : u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        }
#pragma unroll
        for (int t = 0; t < 8; t++) {
          const int c = c0 + 16 * t;
          if (c >= chunks) break;
          float nf[32];  // q = nibble - 8 of coordinates 32c + 8e + h
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint32_t lo = wv[t][e] & 0x0F0F0F0Fu, hi = (wv[t][e] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int b = 0; b < 4; b++) {
              nf[8 * e + 2 * b] = (float)((lo >> (8 * b)) & 0xFFu) - 8.0f;
              nf[8 * e + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu) - 8.0f;
            }
          }
#pragma unroll
          for (int u = 0; u < kMaxMB; u++) {
            if (u < mcount) {
              const floatx4 *xr = (const floatx4 *)(xs + (u * chunks + c) * kPad);
              float s = acc[u];
#pragma unroll
              for (int v = 0; v < 8; v++) {
                const floatx4 xv = xr[v];
                s = fmaf(xv[0], nf[4 * v], s);
                s = fmaf(xv[1], nf[4 * v + 1], s);
                s = fmaf(xv[2], nf[4 * v + 2], s);
                s = fmaf(xv[3], nf[4 * v + 3], s);
              }
              acc[u] = s;
            }
          }
        }
      }
      // reduce the 16 partial sums of each row, one output per (m, n)
      const float sc = scales[n < N ? n : N - 1];
#pragma unroll
      for (int u = 0; u < kMaxMB; u++) {
        float t = acc[u];
        for (int off = 8; off > 0; off >>= 1) t += __shfl_xor(t, off, 16);
        if (j == 0 && n < N && u < mcount)
          y[(m0 + u) * N + n] = f32_to_bf16_rne(t * sc);
      }
    }
  }
}

// One DPP step: v from the lane CTRL selects (rows outside RMASK read 0).
template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, RMASK, 0xF, false));
}

// Sums each of the P partial sums v[i] over the 64 lanes of a wave and
// stores partial i's total to out[i] (LDS), by a transposed reduction:
// swapping the wave's halves (v_permlane32_swap) and adding leaves partial i
// in lanes 0-31 and i + P/2 in lanes 32-63 of P/2 registers; swapping odd
// and even 16-lane rows (v_permlane16_swap) and adding leaves partial
// i + rho P/4 in row rho of P/4 registers; four DPP adds then sum each row.
// 3P/4 swaps and adds and P DPP adds, against 6P DPP adds for P separate
// wave sums.  v is consumed.
template <int P>
__device__ __forceinline__ void wave_sums_to(float (&v)[P], float *out, int lane) {
  static_assert(P % 4 == 0, "P partials in four 16-lane rows");
#pragma unroll
  for (int i = 0; i < P / 2; i++) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + P / 2]), false, false);
    v[i] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
#pragma unroll
  for (int i = 0; i < P / 4; i++) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + P / 4]), false, false);
    v[i] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
#pragma unroll
  for (int i = 0; i < P / 4; i++) {
    float t = v[i];
    t += dpp_f<0xB1, 0xF>(t);   // quad_perm [1,0,3,2]
    t += dpp_f<0x4E, 0xF>(t);   // quad_perm [2,3,0,1]
    t += dpp_f<0x141, 0xF>(t);  // row_half_mirror
    t += dpp_f<0x140, 0xF>(t);  // row_mirror: every lane holds its row's sum
    if ((lane & 15) == 0) out[i + (lane >> 4) * (P / 4)] = t;
  }
}

// Small batches (M <= 4 activation rows, the AdaLN case: one modulation
// row per sample).  Each thread owns one 32-coordinate chunk of K and keeps
// those coordinates of every activation row in registers, so nothing is
// re-read per output row (the general kernel above reads them from LDS for
// every row group: 1.26 GB of LDS reads for 2 x 5120 -> 30720).  A
// workgroup of ceil(K / 2048) waves covers all of K and walks blocks of RB
// output rows: each thread loads its chunk's 16 code bytes of each row (a
// wave reads 1 KB of one row, coalesced), decodes them with byte
// conversions and accumulates the exact fp32 products x q; the RB * MB
// partial sums of a block are reduced over each wave's lanes (wave_sums_to),
// then over the waves through LDS, one barrier per block.
template <int MB>
__global__ __launch_bounds__(512) void rtn4_small_kernel(const void *__restrict__ x, int dtype,
                                                         int M, const u32x4 *__restrict__ q4,
                                                         const float *__restrict__ scales,
                                                         int64_t N, int K,
                                                         uint16_t *__restrict__ y) {
  constexpr int RB = MB == 4 ? 4 : 8;  // output rows per block
  constexpr int P = RB * MB;           // partial sums per block: 8 or 16, p = r MB + m
  __shared__ float red[2][8][P];       // [block parity][wave][partial]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (int)(blockDim.x >> 6);
  const int chunks = K / 32;
  const bool own = tid < chunks;
  float xr[MB][32];
#pragma unroll
  for (int m = 0; m < MB; m++) {
    if (own && m < M) {
      // 16-byte loads of the thread's 32 coordinates (K % 32 == 0)
      if (dtype == 1) {
        const u32x4 *src = (const u32x4 *)((const uint16_t *)x + (int64_t)m * K + 32 * tid);
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const u32x4 a = src[u];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            xr[m][8 * u + 2 * e] = __uint_as_float(a[e] << 16);
            xr[m][8 * u + 2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
          }
        }
      } else {
        const floatx4 *src = (const floatx4 *)((const float *)x + (int64_t)m * K + 32 * tid);
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const floatx4 a = src[u];
#pragma unroll
          for (int e = 0; e < 4; e++) xr[m][4 * u + e] = a[e];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; e++) xr[m][e] = 0.f;
    }
  }
  const int64_t nblk = (N + RB - 1) / RB;
  // codes of the next block are loaded while the current one is decoded
  // the code words of the next block (non-temporal: read once per launch),
  // and the scale of the output row that this thread writes (threads
  // p < RB MB write output p), are loaded while the current block is decoded
  auto load_block = [&](int64_t b, u32x4 (&w)[RB], float &sc) {
#pragma unroll
    for (int r = 0; r < RB; r++) {
      const int64_t n = b * RB + r;
      w[r] = (own && b < nblk && n < N)
                 ? __builtin_nontemporal_load(&q4[n * chunks + tid])
                 : u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
    }
    const int64_t ns = b * RB + tid / MB;
    sc = (tid < P && b < nblk && ns < N) ? scales[ns] : 0.f;
  };
  u32x4 wn[RB];
  float sn;
  load_block(blockIdx.x, wn, sn);
  int par = 0;
  for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x, par ^= 1) {
    const int64_t n0 = b * RB;
    u32x4 w[RB];
#pragma unroll
    for (int r = 0; r < RB; r++) w[r] = wn[r];
    const float scale = sn;
    load_block(b + gridDim.x, wn, sn);
    float v[P];
#pragma unroll
    for (int r = 0; r < RB; r++) {
      float acc[MB];
#pragma unroll
      for (int m = 0; m < MB; m++) acc[m] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const uint32_t lo = w[r][e] & 0x0F0F0F0Fu, hi = (w[r][e] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
          // q = nibble - 8 of coordinates 8e + 2bb (low) and 8e + 2bb + 1
          // (high): one byte permute builds the float 2^23 + nibble (byte bb
          // under the exponent byte 0x4B), one subtraction removes 2^23 + 8
          // (both exact)
          const uint32_t sel = (7u << 24) | (0x0Cu << 16) | (0x0Cu << 8) | (uint32_t)bb;
          const float q0 = __uint_as_float(__builtin_amdgcn_perm(0x4B000000u, lo, sel)) - 8388616.0f;
          const float q1 = __uint_as_float(__builtin_amdgcn_perm(0x4B000000u, hi, sel)) - 8388616.0f;
#pragma unroll
          for (int m = 0; m < MB; m++) {
            acc[m] = fmaf(xr[m][8 * e + 2 * bb], q0, acc[m]);
            acc[m] = fmaf(xr[m][8 * e + 2 * bb + 1], q1, acc[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MB; m++) v[r * MB + m] = acc[m];
    }
    wave_sums_to(v, red[par][wave], lane);
    __syncthreads();  // one barrier per block: red alternates between two buffers
    if (tid < P) {
      float sum = 0.f;
      for (int ww = 0; ww < nw; ww++) sum += red[par][ww][tid];
      const int r = tid / MB, m = tid % MB;
      const int64_t n = n0 + r;
      if (n < N && m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(sum * scale);
    }
  }
}

// bf16 activations (the AdaLN case) on half-precision dot products.  A
// thread scales its 32-coordinate chunk of each activation row by a power of
// two 2^s (largest magnitude into [2^15, 2^16)) and converts it to fp16,
// which is exact when every nonzero bf16 value of the chunk lies within 2^29
// of the largest (fp16 normals hold 11 significant bits, bf16 has 8).  A
// code word's nibbles are split into the even and odd ones (one mask, one
// shift and mask); nibbles j and j + 4 are then two bytes of one of those
// words, and one byte permute puts them under the fp16 high byte 0x64,
// which makes the pair (1024 + n_j, 1024 + n_j+4); one packed fp16
// subtraction of 1032 leaves the exact q = n - 8, and v_dot2c_f32_f16 adds
// the two exact products to an fp32 sum.  The chunk's partial sum is scaled
// back by 2^-s (exact unless the result falls below the fp32 normal range,
// where the fp32 path would round too).  Per 8 nibbles that is 3 + 4 + 4
// instructions and 4 dot products per activation row, against 3 + 16 and 8
// products per row in the fp32 decode.  A workgroup in which any chunk is not exact in fp16
// (a wider range, bf16 subnormals, inf or NaN) decodes in fp32 instead, in
// a loop of its own that re-reads the activations per output row, so the
// fp16 loop holds no registers for it.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int MB>
__global__ __launch_bounds__(512) void rtn4_small_h_kernel(const uint16_t *__restrict__ x, int M,
                                                           const u32x4 *__restrict__ q4,
                                                           const float *__restrict__ scales,
                                                           int64_t N, int K,
                                                           uint16_t *__restrict__ y) {
  constexpr int RB = MB == 4 ? 4 : 8;
  constexpr int P = RB * MB;
  __shared__ float red[2][8][P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (int)(blockDim.x >> 6);
  const int chunks = K / 32;
  const bool own = tid < chunks;
  half2_t xh[MB][16];  // [m][4e + j]: coordinates 8e + j and 8e + j + 4, times 2^s[m]
  int sh[MB];
  bool exact = true;
#pragma unroll
  for (int m = 0; m < MB; m++) {
    uint32_t xb[16];
    if (own && m < M) {
      const u32x4 *src = (const u32x4 *)(x + (int64_t)m * K + 32 * tid);
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const u32x4 a = src[u];
#pragma unroll
        for (int e = 0; e < 4; e++) xb[4 * u + e] = a[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++) xb[i] = 0u;
    }
    // exponent fields of the nonzero values
    int emax = 0, emin = 255;
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const uint32_t b = (xb[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const int ex = (int)((b >> 7) & 0xFFu);
      if (b & 0x7FFFu) {
        emax = ex > emax ? ex : emax;
        emin = ex < emin ? ex : emin;
      }
    }
    if (emin == 255 && emax == 0) emin = emax = 142;  // an all-zero chunk
    exact = exact && emax < 255 && emin > 0 && emax - emin <= 29;
    sh[m] = 142 - emax;  // the largest value lands in [2^15, 2^16)
#pragma unroll
    for (int e = 0; e < 4; e++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int i0 = 8 * e + j, i1 = 8 * e + j + 4;
        const float f0 = __uint_as_float(((xb[i0 >> 1] >> (16 * (i0 & 1))) & 0xFFFFu) << 16);
        const float f1 = __uint_as_float(((xb[i1 >> 1] >> (16 * (i1 & 1))) & 0xFFFFu) << 16);
        // both values are exact in fp16 once scaled, so the rounding mode
        // of the conversion does not matter
        xh[m][4 * e + j] = __builtin_bit_cast(
            half2_t, __builtin_amdgcn_cvt_pkrtz(ldexpf(f0, sh[m]), ldexpf(f1, sh[m])));
      }
  }
  const int64_t nblk = (N + RB - 1) / RB;
  // the code words of the next block (non-temporal: read once per launch),
  // and the scale of the output row that this thread writes (threads
  // p < RB MB write output p), are loaded while the current block is decoded
  auto load_block = [&](int64_t b, u32x4 (&w)[RB], float &sc) {
#pragma unroll
    for (int r = 0; r < RB; r++) {
      const int64_t n = b * RB + r;
      w[r] = (own && b < nblk && n < N)
                 ? __builtin_nontemporal_load(&q4[n * chunks + tid])
                 : u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
    }
    const int64_t ns = b * RB + tid / MB;
    sc = (tid < P && b < nblk && ns < N) ? scales[ns] : 0.f;
  };
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  // the workgroup takes the fp32 decode if any of its chunks is not exact in
  // fp16 (one branch for all its waves, so both loops keep their barriers)
  const bool all_exact = __syncthreads_and(exact ? 1 : 0) != 0;
  auto run = [&](auto fp32_decode) {
    u32x4 wn[RB];
    float sn;
    load_block(blockIdx.x, wn, sn);
    int par = 0;
    for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x, par ^= 1) {
      const int64_t n0 = b * RB;
      u32x4 w[RB];
#pragma unroll
      for (int r = 0; r < RB; r++) w[r] = wn[r];
      const float scale = sn;
      load_block(b + gridDim.x, wn, sn);
      float v[P];
#pragma unroll
      for (int r = 0; r < RB; r++) {
        float acc[MB];
#pragma unroll
        for (int m = 0; m < MB; m++) acc[m] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t lo = w[r][e] & 0x0F0F0F0Fu, hi = (w[r][e] >> 4) & 0x0F0F0F0Fu;
          if constexpr (!decltype(fp32_decode)::value) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
              // nibbles j and j + 4 are bytes k and k + 2 of lo (even j) or
              // hi (odd j), k = j / 2; each goes under the fp16 high byte 0x64
              const uint32_t k = (uint32_t)(j >> 1);
              const uint32_t sel = (4u << 24) | ((k + 2u) << 16) | (4u << 8) | k;
              const uint32_t p = __builtin_amdgcn_perm(0x64646464u, (j & 1) ? hi : lo, sel);
              const half2_t qh = __builtin_bit_cast(half2_t, p) - bias;
#pragma unroll
              for (int m = 0; m < MB; m++)
                acc[m] = __builtin_amdgcn_fdot2(xh[m][4 * e + j], qh, acc[m], false);
            }
          } else {
            // fp32 products, the activations re-read from memory (L1/L2)
#pragma unroll
            for (int m = 0; m < MB; m++) {
              if (own && m < M) {
                const u32x4 a = ((const u32x4 *)(x + (int64_t)m * K + 32 * tid))[e];
#pragma unroll
                for (int bb = 0; bb < 4; bb++) {
                  const uint32_t sel = (7u << 24) | (0x0Cu << 16) | (0x0Cu << 8) | (uint32_t)bb;
                  const float q0 =
                      __uint_as_float(__builtin_amdgcn_perm(0x4B000000u, lo, sel)) - 8388616.0f;
                  const float q1 =
                      __uint_as_float(__builtin_amdgcn_perm(0x4B000000u, hi, sel)) - 8388616.0f;
                  acc[m] = fmaf(__uint_as_float(a[bb] << 16), q0, acc[m]);
                  acc[m] = fmaf(__uint_as_float(a[bb] & 0xFFFF0000u), q1, acc[m]);
                }
              }
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MB; m++)
          v[r * MB + m] = decltype(fp32_decode)::value ? acc[m] : ldexpf(acc[m], -sh[m]);
      }
      wave_sums_to(v, red[par][wave], lane);
      __syncthreads();
      if (tid < P) {
        float sum = 0.f;
        for (int ww = 0; ww < nw; ww++) sum += red[par][ww][tid];
        const int r = tid / MB, m = tid % MB;
        const int64_t n = n0 + r;
        if (n < N && m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(sum * scale);
      }
    }
  };
  if (all_exact)
    run(std::false_type{});
  else
    run(std::true_type{});
}

}  // namespace

hipError_t launch_rtn4_prepare(const void *W, int dtype, int64_t rows, int d, uint8_t *q4,
                               float *scales, hipStream_t stream) {
  const int grid = (int)(rows < 8192 ? rows : 8192);
  hipLaunchKernelGGL(rtn4_prepare_kernel, dim3(grid), dim3(256), 0, stream, W, dtype, rows, d,
                     (uint32_t *)q4, scales);
  return hipGetLastError();
}

hipError_t launch_rtn4_linear(const void *x, int dtype, int64_t M, const uint8_t *q4,
                              const float *scales, int64_t N, int K, uint16_t *y,
                              hipStream_t stream) {
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (M <= 4) {
    // one wave per 64 chunks of 32 coordinates (K <= 16384: at most 8 waves)
    const int chunks = K / 32, threads = 64 * ((chunks + 63) / 64);
    const int rb = M > 2 ? 4 : 8;
    const int64_t nblk = (N + rb - 1) / rb;
    // four workgroups per CU: more waves in flight measured faster than a
    // deeper prefetch queue per wave
    const int64_t want = (int64_t)(cus > 0 ? cus : 256) * 4;
    const unsigned grid = (unsigned)(nblk < want ? nblk : want);
    if (threads > 512) return hipErrorInvalidValue;
    if (dtype == 1) {
      const uint16_t *xb = (const uint16_t *)x;
      if (M == 1)
        hipLaunchKernelGGL(rtn4_small_h_kernel<1>, dim3(grid), dim3(threads), 0, stream, xb,
                           (int)M, (const u32x4 *)q4, scales, N, K, y);
      else if (M == 2)
        hipLaunchKernelGGL(rtn4_small_h_kernel<2>, dim3(grid), dim3(threads), 0, stream, xb,
                           (int)M, (const u32x4 *)q4, scales, N, K, y);
      else
        hipLaunchKernelGGL(rtn4_small_h_kernel<4>, dim3(grid), dim3(threads), 0, stream, xb,
                           (int)M, (const u32x4 *)q4, scales, N, K, y);
      return hipGetLastError();
    }
    if (M == 1)
      hipLaunchKernelGGL(rtn4_small_kernel<1>, dim3(grid), dim3(threads), 0, stream, x, dtype,
                         (int)M, (const u32x4 *)q4, scales, N, K, y);
    else if (M == 2)
      hipLaunchKernelGGL(rtn4_small_kernel<2>, dim3(grid), dim3(threads), 0, stream, x, dtype,
                         (int)M, (const u32x4 *)q4, scales, N, K, y);
    else
      hipLaunchKernelGGL(rtn4_small_kernel<4>, dim3(grid), dim3(threads), 0, stream, x, dtype,
                         (int)M, (const u32x4 *)q4, scales, N, K, y);
    return hipGetLastError();
  }
  int mb = kXBytes / (4 * (K / 32) * kPad);
  if (mb < 1) return hipErrorInvalidValue;
  if (mb > kMaxMB) mb = kMaxMB;
  if (mb > M) mb = (int)M;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit((const void *)rtn4_linear_kernel, kXBytes, lds_set);
  if (e != hipSuccess) return e;
  // as many workgroups as fit two per CU, each with the same number of row
  // groups (no partial last round of groups)
  const int64_t groups = (N + kRows - 1) / kRows;
  const int64_t want = (int64_t)(cus > 0 ? cus : 256) * 2;
  const int64_t per = (groups + want - 1) / want;
  const int64_t grid = (groups + per - 1) / per;
  hipLaunchKernelGGL(rtn4_linear_kernel, dim3((unsigned)grid), dim3(256),
                     (size_t)mb * (K / 32) * kPad * 4,
                     stream, x, dtype, M, (const u32x4 *)q4, scales, N, K, mb, y);
  return hipGetLastError();
}

}  // namespace oq
