// linear.hip -- the low-bit linear on gfx950 matrix cores.
//
//   y[m][n] = bf16( s_m r_n / K * sum_k cw[p_nk] ca[q_mk] )
//
// with unit-variance Lloyd-Max levels ca, cw (the sigma = 1/sqrt(K) of both
// codebooks folded into the 1/K of the epilogue).  llmdb.app Mathematical
// Formulation: y = Q_w(W R^-1) Q_a(R x), bias-free.  Both code matrices are
// K-contiguous rows in the same storage order, so the contraction runs over
// storage slots directly; any fixed reordering of the slots inside a K step
// applied to both operands leaves the sum unchanged.
//
// Design (one 512-thread workgroup per 256 x 256 output tile):
//   * every thread owns one row of the tile (waves 0-3 the 256 activation
//     rows, waves 4-7 the 256 weight rows) and, per 64-slot K step, turns
//     the row's 64 codes into fp16 levels with v_perm_b32 byte tables (the
//     fp16 low and high bytes of the 2^b levels; no memory lookups);
//   * decoded tiles live in LDS, double buffered, as 8 planes of 256 rows x
//     16 bytes (one plane per 8-slot chunk): the decode stores and the MFMA
//     fragment loads both touch consecutive 16-byte words, so neither has
//     bank conflicts and every offset is an instruction immediate;
//   * each of the 8 waves multiplies a 128 x 64 block with
//     v_mfma_f32_16x16x32_f16 (fp32 accumulation), weight fragment first so
//     every lane ends up with 4 consecutive output columns;
//   * one K step is one branch-free block of 8 chunks; chunk c issues 8
//     MFMAs of step t, loads fragments for chunk c+1, decodes slot chunk c of
//     step t+1 and stores it.  Scheduling fences between chunks keep the
//     decode spread between the MFMAs, so both waves of a SIMD always have
//     VALU work to issue while the matrix core runs; codes are loaded two
//     steps ahead into alternating registers;
//   * epilogue: scale by s_m r_n / K, round once to bf16 (nearest even),
//     8-byte stores;
//   * workgroup -> tile order: contiguous per XCD, grouped along M so tiles
//     resident together share activation rows in L2.
//
// Throughput is bound by the matrix core and the decode's VALU issue
// together (about 3.1 VALU instructions per MFMA at 4 bits); the plain fp16
// library GEMM of the same shape is the practical ceiling for comparison.
#include <hip/hip_runtime.h>

#include "oq_internal.h"

namespace oq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 256, TN = 256, KS = 64;  // tile and K step (slots)
constexpr int PLANE = TM * 16;               // one 8-slot chunk of 256 rows
constexpr int OPB = 8 * PLANE;               // bytes per operand tile (32 KB)
constexpr int STAGEB = 2 * OPB;              // A + B per stage
constexpr int LDS_BYTES = 2 * STAGEB;        // double buffered: 128 KB
constexpr int GROUP_M = 8;

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Byte tables of one codebook for v_perm: lo[j] / hi[j] hold the low / high
// bytes of the fp16 levels 4j .. 4j+3.
struct PermTab {
  uint32_t lo[4], hi[4];
};

// Four codes (one per byte, in the low BITS bits; higher bits ignored) ->
// two dwords of fp16 pairs [F(c0), F(c1)], [F(c2), F(c3)].
template <int BITS>
__device__ __forceinline__ void lut4(uint32_t v, const PermTab &t, uint32_t &o0, uint32_t &o1) {
  uint32_t lo, hi;
  if constexpr (BITS == 4) {
    const uint32_t s = v & 0x07070707u;
    const uint32_t l0 = perm(t.lo[1], t.lo[0], s), l1 = perm(t.lo[3], t.lo[2], s);
    const uint32_t h0 = perm(t.hi[1], t.hi[0], s), h1 = perm(t.hi[3], t.hi[2], s);
    const uint32_t m = ((v >> 1) & 0x04040404u) | 0x03020100u;  // byte i: i, or 4+i if bit 3
    lo = perm(l1, l0, m);
    hi = perm(h1, h0, m);
  } else if constexpr (BITS == 3) {
    const uint32_t s = v & 0x07070707u;
    lo = perm(t.lo[1], t.lo[0], s);
    hi = perm(t.hi[1], t.hi[0], s);
  } else {
    const uint32_t s = v & 0x03030303u;
    lo = perm(t.lo[0], t.lo[0], s);
    hi = perm(t.hi[0], t.hi[0], s);
  }
  o0 = perm(hi, lo, 0x05010400u);
  o1 = perm(hi, lo, 0x07030602u);
}

// Decode slot chunk q (slots 8q .. 8q+7) of one K step, given the step's
// 8*BITS code bytes in w.  The 8 fp16 levels come out in slot order
// 8q + {0,2,4,6,1,3,5,7}, the same for every bit width, so activation and
// weight chunks always line up.
template <int BITS>
__device__ __forceinline__ u32x4 decode_q(const uint32_t *w, const PermTab &t, int q) {
  uint32_t a0, a1, b0, b1;
  if constexpr (BITS == 4) {
    lut4<4>(w[q], t, a0, a1);       // even nibbles: slots 0,2,4,6
    lut4<4>(w[q] >> 4, t, b0, b1);  // odd nibbles: slots 1,3,5,7
  } else if constexpr (BITS == 2) {
    // slots 16p .. 16p+15 in w[p]; byte i of x >> 2r holds slot 4i + r
    const uint32_t x = w[q >> 1];
    const uint32_t v0 = x, v1 = x >> 2, v2 = x >> 4, v3 = x >> 6;
    const uint32_t sel = (q & 1) ? 0x07030602u : 0x05010400u;
    lut4<2>(perm(v2, v0, sel), t, a0, a1);
    lut4<2>(perm(v3, v1, sel), t, b0, b1);
  } else {
    // slots 8q .. 8q+7 occupy bits [24q, 24q+24) of the 192-bit string
    const int bit = 24 * q, wd = bit >> 5, sh = bit & 31;
    uint32_t g = w[wd] >> sh;
    if (sh > 8) g |= w[wd + 1] << (32 - sh);
    const uint32_t ev = (g & 7u) | ((g >> 6) & 7u) << 8 | ((g >> 12) & 7u) << 16 |
                        ((g >> 18) & 7u) << 24;
    const uint32_t od = ((g >> 3) & 7u) | ((g >> 9) & 7u) << 8 | ((g >> 15) & 7u) << 16 |
                        ((g >> 21) & 7u) << 24;
    lut4<3>(ev, t, a0, a1);
    lut4<3>(od, t, b0, b1);
  }
  return u32x4{a0, a1, b0, b1};
}

// Byte offset of (row, chunk) inside one operand tile of the LDS layout.
__device__ __forceinline__ int chunk_off(int row, int chunk) { return chunk * PLANE + row * 16; }

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t *p, uint32_t *w) {
  if constexpr (BITS == 4) {
    const u32x4 a = *(const u32x4 *)p, b = *(const u32x4 *)(p + 16);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else if constexpr (BITS == 2) {
    const u32x4 a = *(const u32x4 *)p;
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a = *(const u32x2 *)p, b = *(const u32x2 *)(p + 8), c = *(const u32x2 *)(p + 16);
    w[0] = a[0]; w[1] = a[1]; w[2] = b[0]; w[3] = b[1]; w[4] = c[0]; w[5] = c[1];
  }
}

// The K loop of one tile for a thread whose row has BITS-bit codes at `prow`
// (activation or weight row; the MFMA work is the same for both roles).
template <int BITS>
__device__ __forceinline__ void k_loop(uint8_t *lds, floatx4 (&acc)[4][8], const uint8_t *prow,
                                       const PermTab &tt, int opoff, int row, int lane, int wm,
                                       int wn, int T) {
  constexpr int RB = 8 * BITS;  // code bytes of one K step
  uint32_t cb0[2 * BITS], cb1[2 * BITS];
  uint8_t *wbase = lds + opoff;
  load_codes<BITS>(prow, cb0);
#pragma unroll
  for (int q = 0; q < 8; q++) *(u32x4 *)(wbase + chunk_off(row, q)) = decode_q<BITS>(cb0, tt, q);
  if (T > 1) load_codes<BITS>(prow + RB, cb1);

  // fragment lanes: rows + (lane & 15), 8-slot chunk (lane >> 4) of each
  // 32-slot half
  const int fr = lane & 15, ch0 = lane >> 4, ch1 = 4 + (lane >> 4);

  // One K step: the MFMAs of step t (stage t&1); when `decode`, also the
  // decode of step t+1 (from `cur`) into stage (t+1)&1 and the load of
  // step t+2's codes into `nb`.
  auto step = [&](int t, const uint32_t *cur, uint32_t *nb, bool decode) {
    __syncthreads();  // stage t&1 complete, stage (t+1)&1 no longer read
    if (decode) {
      const int n2 = (t + 2 < T) ? t + 2 : T - 1;  // past the end: a harmless re-read
      load_codes<BITS>(prow + (int64_t)n2 * RB, nb);
    }
    const uint8_t *sA = lds + (t & 1) * STAGEB;
    const uint8_t *sB = sA + OPB;
    uint8_t *dst = wbase + ((t + 1) & 1) * STAGEB;
    half8 af0[8], bf0[4], af1[8], bf1[4];
#pragma unroll
    for (int j = 0; j < 4; j++) bf0[j] = *(const half8 *)(sB + chunk_off(wn * 64 + 16 * j + fr, ch0));
#pragma unroll
    for (int i = 0; i < 2; i++) af0[i] = *(const half8 *)(sA + chunk_off(wm * 128 + 16 * i + fr, ch0));
#pragma unroll
    for (int c = 0; c < 8; c++) {
      // fragments one chunk ahead: chunk c uses activation blocks 2(c&3),
      // 2(c&3)+1 of half c>>2 against all 4 weight blocks of that half
      if (c < 3) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
          const int i = 2 * (c + 1) + u;
          af0[i] = *(const half8 *)(sA + chunk_off(wm * 128 + 16 * i + fr, ch0));
        }
      } else if (c == 3) {
#pragma unroll
        for (int j = 0; j < 4; j++)
          bf1[j] = *(const half8 *)(sB + chunk_off(wn * 64 + 16 * j + fr, ch1));
#pragma unroll
        for (int i = 0; i < 2; i++)
          af1[i] = *(const half8 *)(sA + chunk_off(wm * 128 + 16 * i + fr, ch1));
      } else if (c < 7) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
          const int i = 2 * (c - 3) + u;
          af1[i] = *(const half8 *)(sA + chunk_off(wm * 128 + 16 * i + fr, ch1));
        }
      }
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int i = 2 * (c & 3) + u;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          if (c < 4)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf0[j], af0[i], acc[j][i], 0, 0, 0);
          else
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf1[j], af1[i], acc[j][i], 0, 0, 0);
        }
      }
      if (decode) *(u32x4 *)(dst + chunk_off(row, c)) = decode_q<BITS>(cur, tt, c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // steps in pairs so the two code buffers alternate without copies
  int t = 0;
  for (; t + 2 < T; t += 2) {
    step(t, cb1, cb0, true);
    step(t + 1, cb0, cb1, true);
  }
  if (t + 1 < T) {
    step(t, cb1, cb0, true);
    t++;
  }
  step(t, cb1, cb0, false);
}

template <int BA, int BW>
__global__ __launch_bounds__(512, 1) void linear_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ Wc,
    const float *__restrict__ sw, int M, int N, int K, uint16_t *__restrict__ Y, PermTab ta,
    PermTab tw, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  // ---- workgroup -> tile (contiguous per XCD, grouped along M)
  const int nbm = (M + TM - 1) / TM, nbn = (N + TN - 1) / TN, total = nbm * nbn;
  int bid = blockIdx.x;
  {
    const int xcd = bid & 7, local = bid >> 3, per = total >> 3, rem = total & 7;
    bid = xcd * per + (xcd < rem ? xcd : rem) + local;
  }
  const int gsz = GROUP_M * nbn, grp = bid / gsz, first_m = grp * GROUP_M;
  const int gm = (nbm - first_m) < GROUP_M ? (nbm - first_m) : GROUP_M;
  const int tm = first_m + (bid % gsz) % gm, tn = (bid % gsz) / gm;
  const int m0 = tm * TM, n0 = tn * TN;

  // ---- the row this thread decodes (rows past the edge repeat the last row)
  const bool is_a = __builtin_amdgcn_readfirstlane(tid) < 256;  // wave-uniform
  const int row = tid & 255;
  const int am = (m0 + row < M) ? m0 + row : M - 1;
  const int wr = (n0 + row < N) ? n0 + row : N - 1;
  const uint8_t *pa = A + (int64_t)am * ((int64_t)K * BA / 8);
  const uint8_t *pw = Wc + (int64_t)wr * ((int64_t)K * BW / 8);
  const int T = K / KS;

  floatx4 acc[4][8];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int i = 0; i < 8; i++) acc[j][i] = floatx4{0.f, 0.f, 0.f, 0.f};

  if constexpr (BA == BW) {
    k_loop<BA>(lds, acc, is_a ? pa : pw, is_a ? ta : tw, is_a ? 0 : OPB, row, lane, wm, wn, T);
  } else {
    // both branches run the same barriers; the branch is wave-uniform
    if (is_a) k_loop<BA>(lds, acc, pa, ta, 0, row, lane, wm, wn, T);
    else k_loop<BW>(lds, acc, pw, tw, OPB, row, lane, wm, wn, T);
  }

  // ---- epilogue: lane holds rows m = .. + (lane & 15), cols n = .. + 4 (lane >> 4) + r
  const float invk = 1.0f / (float)K;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int m = m0 + wm * 128 + 16 * i + (lane & 15);
    if (m >= M) continue;
    const float s = sa[m] * invk;
    uint16_t *yrow = Y + (int64_t)m * N;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int n = n0 + wn * 64 + 16 * j + 4 * (lane >> 4);
      if (vec_store && n + 3 < N) {
        const floatx4 r = *(const floatx4 *)(sw + n);
        const uint32_t lo = f32_to_bf16_rne(acc[j][i][0] * s * r[0]) |
                            (f32_to_bf16_rne(acc[j][i][1] * s * r[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[j][i][2] * s * r[2]) |
                            (f32_to_bf16_rne(acc[j][i][3] * s * r[3]) << 16);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *(u32x2 *)(yrow + n) = u32x2{lo, hi};
      } else {
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (n + r < N) yrow[n + r] = (uint16_t)f32_to_bf16_rne(acc[j][i][r] * s * sw[n + r]);
      }
    }
  }
}

PermTab make_tab(const LevelsF16 &lv) {
  PermTab t{};
  for (int e = 0; e < 16; e++) {
    t.lo[e >> 2] |= (uint32_t)(lv.v[e] & 0xFFu) << (8 * (e & 3));
    t.hi[e >> 2] |= (uint32_t)(lv.v[e] >> 8) << (8 * (e & 3));
  }
  return t;
}

template <int BA, int BW>
hipError_t launch_ab(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)linear_kernel<BA, BW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = ((a.M + TM - 1) / TM) * ((a.N + TN - 1) / TN);
  const int vec = (a.N % 4 == 0) && (((uintptr_t)a.y & 7) == 0) && (((uintptr_t)a.w_norms & 15) == 0);
  hipLaunchKernelGGL((linear_kernel<BA, BW>), dim3((unsigned)tiles), dim3(512), LDS_BYTES,
                     a.stream, a.a_codes, a.a_norms, a.w_codes, a.w_norms, (int)a.M, (int)a.N,
                     a.K, a.y, make_tab(la), make_tab(lw), vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw) {
  if (a.M > (int64_t)1 << 30 || a.N > (int64_t)1 << 30) return hipErrorInvalidValue;
#define OQ_CASE(x, y) \
  if (a.a_bits == x && a.w_bits == y) return launch_ab<x, y>(a, la, lw);
  OQ_CASE(2, 2) OQ_CASE(2, 3) OQ_CASE(2, 4)
  OQ_CASE(3, 2) OQ_CASE(3, 3) OQ_CASE(3, 4)
  OQ_CASE(4, 2) OQ_CASE(4, 3) OQ_CASE(4, 4)
#undef OQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace oq
