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
// accumulates in fp32.  Both kernels are bound by HBM: the modulation input
// is a handful of rows (one per sample), so the weights are read once.
#include <hip/hip_runtime.h>

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
  int mb = kXBytes / (4 * (K / 32) * kPad);
  if (mb < 1) return hipErrorInvalidValue;
  if (mb > kMaxMB) mb = kMaxMB;
  if (mb > M) mb = (int)M;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit((const void *)rtn4_linear_kernel, kXBytes, lds_set);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
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
