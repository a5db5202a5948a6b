// rotate_quantize.hip -- rotate + quantize kernels for gfx950.
//
// Per token x (length d): s = ||x||, y_i = D_i x_{pi(i)}, z = blockwise
// H_h y / (s sqrt(h)), code = #{k : sqrt(d) z >= tau_k} over the unit
// Lloyd-Max thresholds, packed in storage order.  (paper.gecl.asia notes,
// Method items 1, 3, 4; pith.science Supplementary A setup.)
//
// This file holds the general kernel: any dtype, any h, one workgroup per
// token, the token held in LDS as fp32.  Besides packed codes it can write
// the rotated unit vector (fp32) or the dequantized rotated token
// s * c_{code_i} (bf16, fake quantization).  Up to 4 bits the code counts
// the thresholds at or below the value one by one; at 8 bits it is found by
// an 8-step binary search over the 255 thresholds held in LDS.
#include <hip/hip_runtime.h>

#include "oq_internal.h"

namespace oq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_elem(const void *x, int dtype, int64_t idx) {
  if (dtype == 1) {
    uint32_t u = (uint32_t)((const uint16_t *)x)[idx] << 16;
    return __uint_as_float(u);
  }
  return ((const float *)x)[idx];
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t *dst, uint64_t word) {
  if constexpr (BITS == 8) {
    *(uint64_t *)dst = word;
  } else if constexpr (BITS == 4) {
    *(uint32_t *)dst = word;
  } else if constexpr (BITS == 2) {
    *(uint16_t *)dst = (uint16_t)word;
  } else {
    dst[0] = (uint8_t)word;
    dst[1] = (uint8_t)(word >> 8);
    dst[2] = (uint8_t)(word >> 16);
  }
}

// Workgroup sum of one double per thread; every thread gets the total.
__device__ double block_sum(double v, double *scratch) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kThreads / 64; w++) t += scratch[w];
  return t;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Number of unit thresholds at or below u.
template <int BITS>
__device__ __forceinline__ uint32_t code_of(float u, const Thresholds &th, const float *t8) {
  if constexpr (BITS == 8) {
    uint32_t pos = 0;
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1)
      if (u >= t8[pos + step - 1]) pos += step;
    return pos;
  } else {
    uint32_t code = 0;
    for (int k = 0; k < th.count; k++) code += (u >= th.t[k]) ? 1u : 0u;
    return code;
  }
}

template <int BITS>
__device__ __forceinline__ float level_of(uint32_t code, const LevelsF32 &lv, const float *l8) {
  if constexpr (BITS == 8) return l8[code];
  else return lv.v[code];
}

// table (8 bits only): the device codebook table; its levels and thresholds
// are copied into LDS after the token.
template <int BITS>
__global__ __launch_bounds__(kThreads) void rq_generic_kernel(
    const void *__restrict__ x, int dtype, int64_t n_tok, int d, int h,
    const int32_t *__restrict__ scatter, int sign_on, Thresholds th, LevelsF32 lv,
    const uint32_t *__restrict__ table, uint8_t *__restrict__ codes, float *__restrict__ zout,
    uint16_t *__restrict__ dq, float *__restrict__ norms) {
  extern __shared__ float y[];  // d floats, then (8 bits) 256 levels, 256 thresholds
  __shared__ double red[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t row_bytes = (int64_t)d * BITS / 8;
  float *l8 = y + d, *t8 = y + d + 256;
  if constexpr (BITS == 8) {
    l8[tid] = __uint_as_float(table[table_levels_word(8) + tid]);
    if (tid < 255) t8[tid] = __uint_as_float(table[table_thresholds_word(8) + tid]);
    __syncthreads();
  }
  for (int64_t t = blockIdx.x; t < n_tok; t += gridDim.x) {
    // load, sum of squares, scatter with sign: y[pi^-1(j)] = D x_j
    float ss = 0.f;
    for (int j = tid; j < d; j += kThreads) {
      float v = load_elem(x, dtype, t * d + j);
      ss = fmaf(v, v, ss);
      int32_t e = scatter[j];
      y[e & 0x7fffffff] = (e < 0 && sign_on) ? -v : v;
    }
    double total = block_sum((double)ss, red);
    __syncthreads();
    // block Walsh-Hadamard (unnormalised, Sylvester order), radix 2
    for (int len = 1; len < h; len <<= 1) {
      for (int q = tid; q < d / 2; q += kThreads) {
        int i = ((q & ~(len - 1)) << 1) | (q & (len - 1));
        float a = y[i], b = y[i + len];
        y[i] = a + b;
        y[i + len] = a - b;
      }
      __syncthreads();
    }
    const double s = sqrt(total);
    if (tid == 0) norms[t] = (float)s;
    if (zout) {
      const float zs = s > 0.0 ? (float)(1.0 / (s * sqrt((double)h))) : 0.f;
      for (int i = tid; i < d; i += kThreads) zout[t * d + i] = y[i] * zs;
    } else {
      // unit-space value sqrt(d) z_i = y_i sqrt(d/h) / s
      const float us = s > 0.0 ? (float)(sqrt((double)d / (double)h) / s) : 0.f;
      const float fs = (float)(s / sqrt((double)d));  // dequantized value = s * level / sqrt(d)
      // thread q packs 8 consecutive slots into one b-byte word: inside a
      // whole 128-coordinate group (q < full) the slots 8n .. 8n+7 of group
      // G hold coordinates 128G + 32c + 16w + n; in a last, partial group
      // (d mod 128 = 32, 64 or 96) slot i holds coordinate i
      const int full = (d / 128) * 16;
      for (int q = tid; q < d / 8; q += kThreads) {
        const bool grp = q < full;
        const int G = q >> 4, n = q & 15;
        uint64_t word = 0;
#pragma unroll
        for (int w = 0; w < 2; w++)
#pragma unroll
          for (int c = 0; c < 4; c++) {
            const int e = 4 * w + c;  // slot 8q + e (8n + e of group G)
            const int i = grp ? G * 128 + 32 * c + 16 * w + n : 8 * q + e;
            const float u = y[i] * us;
            const uint32_t code = code_of<BITS>(u, th, t8);
            if (dq) dq[t * d + i] = f32_to_bf16_rne(fs * level_of<BITS>(code, lv, l8));
            word |= (uint64_t)code << (BITS * e);
          }
        if (!dq) store_codes<BITS>(codes + t * row_bytes + BITS * q, word);
      }
    }
    __syncthreads();
  }
}

// Row permutation: source row j goes to destination row perm_inv[j], in
// units of V bytes (16 when sizes and pointers allow).
template <typename V>
__global__ __launch_bounds__(256) void permute_rows_kernel(const V *__restrict__ src,
                                                           V *__restrict__ dst, int64_t rows,
                                                           int64_t row_units,
                                                           const int32_t *__restrict__ perm_inv) {
  for (int64_t j = blockIdx.x; j < rows; j += gridDim.x) {
    const V *s = src + j * row_units;
    V *d = dst + (int64_t)perm_inv[j] * row_units;
    for (int64_t u = threadIdx.x; u < row_units; u += blockDim.x) d[u] = s[u];
  }
}

}  // namespace

hipError_t launch_permute_rows(const void *src, void *dst, int64_t rows, int64_t row_bytes,
                               const int32_t *perm_inv, hipStream_t stream) {
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
  const int grid = (int)(rows < 4096 ? rows : 4096);
  if (al % 16 == 0) {
    hipLaunchKernelGGL(permute_rows_kernel<uint4>, dim3(grid), dim3(256), 0, stream,
                       (const uint4 *)src, (uint4 *)dst, rows, row_bytes / 16, perm_inv);
  } else if (al % 4 == 0) {
    hipLaunchKernelGGL(permute_rows_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream,
                       (const uint32_t *)src, (uint32_t *)dst, rows, row_bytes / 4, perm_inv);
  } else if (al % 2 == 0) {
    hipLaunchKernelGGL(permute_rows_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t *)src, (uint16_t *)dst, rows, row_bytes / 2, perm_inv);
  } else {
    hipLaunchKernelGGL(permute_rows_kernel<uint8_t>, dim3(grid), dim3(256), 0, stream,
                       (const uint8_t *)src, (uint8_t *)dst, rows, row_bytes, perm_inv);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_generic_bits(const RotateArgs &a, const int32_t *sc, int sign_on,
                               const Thresholds &th, const uint32_t *table, int grid,
                               uint8_t *codes, float *zout, uint16_t *dq) {
  const size_t lds = sizeof(float) * (a.d + (BITS == 8 ? 512 : 0));
  if (lds > 32768) {
    // tokens above 8192 fp32 need more than the default dynamic-LDS cap (set
    // once per device at the largest token size the path takes)
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = ensure_lds_limit((const void *)rq_generic_kernel<BITS>,
                                    (int)sizeof(float) * (kMaxD + 512), lds_set);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(rq_generic_kernel<BITS>, dim3(grid), dim3(kThreads), lds, a.stream, a.x,
                     a.dtype, a.n_tok, a.d, a.h, sc, sign_on, th, a.levels, table, codes, zout,
                     dq, a.norms);
  return hipGetLastError();
}

hipError_t launch_rotate_quantize_generic(const RotateArgs &a, const DevicePlan &p,
                                          const Thresholds &th, const uint32_t *table) {
  // placement table: pi^-1 with sign bits, or the identity with sign bits
  // when the input is already in rotation order
  const int32_t *sc = a.input_permuted ? p.scatter_id : (a.signs ? p.scatter : p.scatter_nosign);
  const int sign_on = a.signs ? 1 : 0;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t want = (int64_t)(cus > 0 ? cus : 256) * 8;
  const int grid = (int)(a.n_tok < want ? a.n_tok : want);
  uint8_t *codes = (a.rotated_out || a.dequant_out) ? nullptr : (uint8_t *)a.out;
  float *zout = a.rotated_out ? (float *)a.out : nullptr;
  uint16_t *dq = a.dequant_out ? (uint16_t *)a.out : nullptr;
  switch (a.bits) {
    case 2: return launch_generic_bits<2>(a, sc, sign_on, th, table, grid, codes, zout, dq);
    case 3: return launch_generic_bits<3>(a, sc, sign_on, th, table, grid, codes, zout, dq);
    case 4: return launch_generic_bits<4>(a, sc, sign_on, th, table, grid, codes, zout, dq);
    case 8:
      if (!table) return hipErrorInvalidValue;
      return launch_generic_bits<8>(a, sc, sign_on, th, table, grid, codes, zout, dq);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oq
