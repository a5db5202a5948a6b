// linear.hip -- the low-bit linear on gfx950 matrix cores.
//
//   y[m][n] = bf16( s_m r_n / K * sum_k cw[p_nk] ca[q_mk] )
//
// with unit-variance Lloyd-Max levels ca, cw (the sigma = 1/sqrt(K) of both
// codebooks folded into the 1/K of the epilogue).  llmdb.app Mathematical
// Formulation: y = Q_w(W R^-1) Q_a(R x), bias-free.  Both code matrices are
// K-contiguous rows in the same storage order, so the contraction runs over
// storage slots directly.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 output tile; per 64-slot
// K step every thread decodes 32 activation codes and 32 weight codes
// through a 16-entry fp16 lookup table into LDS, then each of the four
// waves multiplies its 64 x 64 quadrant with v_mfma_f32_16x16x32_f16
// (fp32 accumulation).  The epilogue scales by s_m r_n / K and rounds once
// to bf16 (nearest even).
#include <hip/hip_runtime.h>

#include "oq_internal.h"

namespace oq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Decode 32 consecutive codes of BITS bits (little-endian bit string at p,
// 4*BITS bytes, 4-byte aligned) through lut into dst[0..31].
template <int BITS>
__device__ __forceinline__ void decode32(const uint8_t *__restrict__ p,
                                         const _Float16 *__restrict__ lut, _Float16 *dst) {
  uint32_t w[BITS];
#pragma unroll
  for (int i = 0; i < BITS; i++) w[i] = ((const uint32_t *)p)[i];
#pragma unroll
  for (int j = 0; j < 32; j++) {
    const int bit = BITS * j;
    uint32_t v = w[bit >> 5] >> (bit & 31);
    if ((bit & 31) + BITS > 32) v |= w[(bit >> 5) + 1] << (32 - (bit & 31));
    dst[j] = lut[v & ((1u << BITS) - 1u)];
  }
}

template <int BA, int BW>
__global__ __launch_bounds__(256) void linear_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ Wc,
    const float *__restrict__ sw, int64_t M, int64_t N, int K, uint16_t *__restrict__ Y,
    LevelsF16 la, LevelsF16 lw) {
  __shared__ __attribute__((aligned(16))) _Float16 As[BM][LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN][LDK];
  __shared__ _Float16 luta[16], lutw[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  if (tid < 16) {
    luta[tid] = __builtin_bit_cast(_Float16, la.v[tid]);
    lutw[tid] = __builtin_bit_cast(_Float16, lw.v[tid]);
  }
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t arow = (int64_t)K * BA / 8, wrow = (int64_t)K * BW / 8;
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t am = (m0 + lr < M) ? m0 + lr : M - 1;
  const int64_t wnr = (n0 + lr < N) ? n0 + lr : N - 1;
  const uint8_t *pa = A + am * arow + lh * 4 * BA;
  const uint8_t *pw = Wc + wnr * wrow + lh * 4 * BW;

  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    {
      _Float16 tmp[32];
      decode32<BA>(pa + (int64_t)k0 * BA / 8, luta, tmp);
#pragma unroll
      for (int q = 0; q < 4; q++)
        *(half8 *)&As[lr][32 * lh + 8 * q] =
            half8{tmp[8 * q], tmp[8 * q + 1], tmp[8 * q + 2], tmp[8 * q + 3], tmp[8 * q + 4],
                  tmp[8 * q + 5], tmp[8 * q + 6], tmp[8 * q + 7]};
      decode32<BW>(pw + (int64_t)k0 * BW / 8, lutw, tmp);
#pragma unroll
      for (int q = 0; q < 4; q++)
        *(half8 *)&Bs[lr][32 * lh + 8 * q] =
            half8{tmp[8 * q], tmp[8 * q + 1], tmp[8 * q + 2], tmp[8 * q + 3], tmp[8 * q + 4],
                  tmp[8 * q + 5], tmp[8 * q + 6], tmp[8 * q + 7]};
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 32; ks++) {
      half8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        af[i] = *(const half8 *)&As[wm * 64 + 16 * i + (lane & 15)][32 * ks + 8 * (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 4; j++)
        bf[j] = *(const half8 *)&Bs[wn * 64 + 16 * j + (lane & 15)][32 * ks + 8 * (lane >> 4)];
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  const float invk = 1.0f / (float)K;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t col = n0 + wn * 64 + 16 * j + (lane & 15);
      if (col >= N) continue;
      const float rn = sw[col] * invk;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
        if (row < M) Y[row * N + col] = f32_to_bf16_rne(acc[i][j][r] * sa[row] * rn);
      }
    }
}

template <int BA, int BW>
hipError_t launch_ab(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw) {
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  hipLaunchKernelGGL((linear_kernel<BA, BW>), grid, dim3(256), 0, a.stream, a.a_codes, a.a_norms,
                     a.w_codes, a.w_norms, a.M, a.N, a.K, a.y, la, lw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw) {
  if ((a.M + BM - 1) / BM > 65535) return hipErrorInvalidValue;
#define OQ_CASE(x, y) \
  if (a.a_bits == x && a.w_bits == y) return launch_ab<x, y>(a, la, lw);
  OQ_CASE(2, 2) OQ_CASE(2, 3) OQ_CASE(2, 4)
  OQ_CASE(3, 2) OQ_CASE(3, 3) OQ_CASE(3, 4)
  OQ_CASE(4, 2) OQ_CASE(4, 3) OQ_CASE(4, 4)
#undef OQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace oq
