// rotate_quantize_fast.hip -- rotate + quantize for bf16 tokens on gfx950.
//
// Same result as the general kernel (rotate_quantize.hip): s = ||x||,
// y_i = D_i x_{pi(i)}, z = blockwise H_h y / (s sqrt(h)), code = number of
// unit Lloyd-Max thresholds at or below sqrt(d) z_i, packed in storage
// order (paper.gecl.asia notes, Method items 1, 3, 4; pith.science
// Supplementary A setup).  This path is built around the VALU budget of an
// HBM-bound kernel (about a dozen lane operations per coordinate):
//
//  * Staging.  A workgroup handles TB tokens per batch.  Each thread owns
//    CPT fixed 8-element chunks of every token: one 16-byte load per chunk,
//    the Rademacher signs applied as an XOR (D moved onto the source index:
//    D_i x_{pi(i)} = (D_{pi^-1(j)} x_j) at j = pi(i)), and every element
//    scattered with ds_write_b16 to its permuted position pi^-1(j) in LDS.
//    The scatter addresses and sign masks stay in registers for the whole
//    kernel.
//  * Norm.  The 8 bf16 of a staged chunk are an MFMA operand as they are:
//    mfma(X, X) accumulates X X^T, whose trace is the sum of squares.
//  * Walsh-Hadamard, stages 0-4.  bf16 values are exact MFMA operands and
//    H_32 is +-1, so v_mfma_f32_16x16x32_bf16 applies the 32-point
//    transform of every 32-element chunk with fp32 accumulation.  The
//    16 rows of one MFMA are 4 chunks of 4 slots (a slot = 1024 consecutive
//    coordinates, or h if smaller), so each lane ends up holding 4 chunks x
//    2 positions of one slot per 128-coordinate group.
//  * Remaining stages (chunk bits) are register butterflies.
//  * Quantize.  A magic-number fma turns v into a cell index of a uniform
//    grid (step 1/8 sigma, narrower than any threshold gap), an LDS table
//    gives the code at the cell's lower edge and the only threshold that can
//    fall inside it; one exact fp32 compare settles the code.
//  * Pack.  A lane's 8 codes per group are exactly 8 consecutive storage
//    slots, so they pack into one b-byte word per lane.
#include <hip/hip_runtime.h>

#include "oq_internal.h"

namespace oq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCells = 2048;                    // grid cells per table copy
constexpr int kCellBytes = 4 * kCells * 2;      // 4 copies (one per output slot lane group), u16
constexpr int kThrBytesPerWave = 4 * 16 * 8;    // 4 slots x 16 entries x {float T, uint base}
constexpr float kMagic = 12582912.0f;           // 1.5 * 2^23

template <int S, int CPT, int TB, int BITS, int W>
__global__ __launch_bounds__(64 * W) void rq_fast_kernel(
    const uint16_t *__restrict__ x, int64_t n_tok, int d, int h, int P,
    const uint32_t *__restrict__ scat, const uint32_t *__restrict__ smask,
    const uint16_t *__restrict__ cells, Thresholds th, uint8_t *__restrict__ codes,
    float *__restrict__ norms) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int G = S / 128;        // 128-coordinate groups per slot
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ybytes = (int64_t)TB * d * 2;
  uint8_t *ybuf = lds;
  uint8_t *ctab = lds + ybytes;
  uint8_t *ttab = ctab + kCellBytes + wave * kThrBytesPerWave;
  float *npart = (float *)(ctab + kCellBytes + W * kThrBytesPerWave);  // [TB][W]

  // cell tables (all 4 copies) into LDS
  for (int i = tid; i < kCellBytes / 16; i += W * 64)
    ((u32x4 *)ctab)[i] = ((const u32x4 *)cells)[i];

  // per-thread staging: chunk c of every token covers x[8*pos, 8*pos+8)
  uint32_t saddr[CPT][8], smk[CPT][4];
  int cpos[CPT];
#pragma unroll
  for (int c = 0; c < CPT; c++) {
    const int pos = tid + c * W * 64;  // chunk index inside a token (d/8 chunks)
    cpos[c] = pos;
#pragma unroll
    for (int e = 0; e < 8; e++) saddr[c][e] = scat[pos * 8 + e];
#pragma unroll
    for (int e = 0; e < 4; e++) smk[c][e] = smask[pos * 4 + e];
  }

  // H_32 operands: lane holds H[k][n] for k = 8(lane>>4)+e, n = lane&15 (+16)
  bf16x8 hb0, hb1;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int k = 8 * (lane >> 4) + e, n = lane & 15;
    hb0[e] = (__builtin_popcount(k & n) & 1) ? (__bf16)-1.0f : (__bf16)1.0f;
    hb1[e] = (__builtin_popcount(k & (n + 16)) & 1) ? (__bf16)-1.0f : (__bf16)1.0f;
  }
  const float root_hd = sqrtf((float)h / (float)d);   // v-space threshold = tau s sqrt(h/d)
  const float inv_delta2 = 16.0f;                       // 2 / (1/8)
  const int WT = TB * P / 4;                            // wave tiles per batch
  const int64_t row_bytes = (int64_t)d * BITS / 8;
  const int64_t nbatch = (n_tok + TB - 1) / TB;

  // register double buffer of the next batch's chunks
  u32x4 stg[TB][CPT];
  auto load_batch = [&](int64_t b) {
#pragma unroll
    for (int tk = 0; tk < TB; tk++) {
      const int64_t t = b * TB + tk;
#pragma unroll
      for (int c = 0; c < CPT; c++)
        stg[tk][c] = (t < n_tok) ? *(const u32x4 *)(x + t * d + 8 * cpos[c]) : u32x4{0, 0, 0, 0};
    }
  };

  int64_t b = blockIdx.x;
  if (b < nbatch) load_batch(b);
  __syncthreads();
  for (; b < nbatch; b += gridDim.x) {
    // ---- stage: norms by Gram MFMA, sign, scatter
#pragma unroll
    for (int tk = 0; tk < TB; tk++) {
      floatx4 gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < CPT; c++) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, stg[tk][c]);
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, xv, gram, 0, 0, 0);
        uint8_t *yb = ybuf + (int64_t)tk * d * 2;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t v = stg[tk][c][e] ^ smk[c][e];
          *(uint16_t *)(yb + saddr[c][2 * e]) = (uint16_t)v;
          *(uint16_t *)(yb + saddr[c][2 * e + 1]) = (uint16_t)(v >> 16);
        }
      }
      // trace of the Gram matrix: diagonal entry r sits in lane 16(r/4)+r, register r%4
      const int r = lane & 15;
      float dg = ((r >> 2) == (lane >> 4)) ? gram[r & 3] : 0.f;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dg += __shfl_xor(dg, off, 64);
      if (lane == 0) npart[tk * W + wave] = dg;
    }
    if (b + gridDim.x < nbatch) load_batch(b + gridDim.x);
    __syncthreads();

    // ---- compute: wave tiles q = wave, wave + W, ...
    for (int q = wave; q < WT; q += W) {
      // output side of this lane: slot so = lane >> 4
      const int so = lane >> 4, sig_o = 4 * q + so;
      const int tko = sig_o / P, jo = sig_o - tko * P;
      float ss = 0.f;
      for (int w = 0; w < W; w++) ss += npart[tko * W + w];
      const float s = sqrtf(ss);
      // thresholds of this slot (v-space): lane writes entry (so, lane & 15)
      {
        const int k = lane & 15;
        const float tv = (k < th.count) ? th.t[k] * s * root_hd : __builtin_inff();
        uint32_t *ent = (uint32_t *)(ttab + 128 * so + 8 * k);
        ent[0] = __float_as_uint(tv);
        ent[1] = (uint32_t)k;
      }
      const float us = (s > 0.f) ? 1.0f / (s * root_hd) : 0.f;  // sqrt(d/h)/s
      const float a2 = us * inv_delta2;
      const float m2 = kMagic + 2.0f * (float)(kCells / 2) + (float)(2 * kCells * so);
      // input side of this lane: row r = lane & 15 -> slot r>>2, chunk (r&3) of each group
      const int si = (lane & 15) >> 2, sig_i = 4 * q + si;
      const int tki = sig_i / P, ji = sig_i - tki * P;
      const uint8_t *ya =
          ybuf + (int64_t)tki * d * 2 + 2 * (ji * S + 32 * (lane & 3) + 8 * (lane >> 4));

      float v[G][2][4];
#pragma unroll
      for (int g = 0; g < G; g++) {
        const bf16x8 a = *(const bf16x8 *)(ya + 256 * g);
        floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hb0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hb1, c1, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          v[g][0][i] = c0[i];
          v[g][1][i] = c1[i];
        }
      }
      // chunk stages: chunk = 4g + i, log2(S/32) bits (this path has h == S)
      constexpr int cbits = (S >= 1024 ? 10 : S >= 512 ? 9 : S >= 256 ? 8 : 7) - 5;
#pragma unroll
      for (int bit = 0; bit < 2; bit++) {
        if (bit < cbits) {
#pragma unroll
          for (int g = 0; g < G; g++)
#pragma unroll
            for (int w = 0; w < 2; w++)
#pragma unroll
              for (int i = 0; i < 4; i++)
                if (!(i & (1 << bit))) {
                  const float p0 = v[g][w][i], p1 = v[g][w][i | (1 << bit)];
                  v[g][w][i] = p0 + p1;
                  v[g][w][i | (1 << bit)] = p0 - p1;
                }
        }
      }
#pragma unroll
      for (int bit = 0; (1 << bit) < G; bit++) {
        if (bit + 2 < cbits) {
#pragma unroll
          for (int g = 0; g < G; g++)
            if (!(g & (1 << bit))) {
#pragma unroll
              for (int w = 0; w < 2; w++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                  const float p0 = v[g][w][i], p1 = v[g | (1 << bit)][w][i];
                  v[g][w][i] = p0 + p1;
                  v[g | (1 << bit)][w][i] = p0 - p1;
                }
            }
        }
      }
      // quantize + pack + store
      const int64_t tok = (b * TB) + tko;
      const bool live = tok < n_tok;
      uint8_t *crow = codes + tok * row_bytes;
      const int n = lane & 15;
#pragma unroll
      for (int g = 0; g < G; g++) {
        uint32_t word = 0;
#pragma unroll
        for (int w = 0; w < 2; w++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float val = v[g][w][i];
            const float tq = __builtin_fmaf(val, a2, m2);
            const uint32_t cell = __float_as_uint(tq) & 0x3FFEu;
            const uint32_t e = *(const uint16_t *)(ctab + cell);
            const uint32_t *ent = (const uint32_t *)(ttab + e);
            const float tv = __uint_as_float(ent[0]);
            const uint32_t code = ent[1] + (val >= tv ? 1u : 0u);
            word |= code << (BITS * (4 * w + i));
          }
        if (live) {
          const int grp = jo * G + g;  // 128-coordinate group inside the token
          uint8_t *dst = crow + 16 * BITS * grp + BITS * n;
          if constexpr (BITS == 4) {
            *(uint32_t *)dst = word;
          } else if constexpr (BITS == 2) {
            *(uint16_t *)dst = (uint16_t)word;
          } else {
            dst[0] = (uint8_t)word;
            dst[1] = (uint8_t)(word >> 8);
            dst[2] = (uint8_t)(word >> 16);
          }
        }
      }
      if (live && n == 0 && jo == 0) norms[tok] = s;
    }
    __syncthreads();
  }
}

}  // namespace

// Kernel configuration for one (d, h): slot size, tokens per batch, waves.
struct FastCfg {
  int S, P, TB, W, CPT;
  size_t lds;
};

bool fast_config(int d, int h, FastCfg &c) {
  if (d % 512 != 0 || h < 128) return false;
  c.S = h < 1024 ? h : 1024;
  if (h > 1024) return false;  // cross-slot stages are not built into this path
  c.P = d / c.S;
  c.TB = 4;
  const int WT = c.TB * c.P / 4;
  const int chunks = d / 512;  // chunks per token per wave of 64 threads
  c.W = 0;
  for (int w = 16; w >= 1; w--)
    if (WT % w == 0 && chunks % w == 0) {
      c.W = w;
      break;
    }
  if (c.W == 0) return false;
  c.CPT = chunks / c.W;
  c.lds = (size_t)c.TB * d * 2 + kCellBytes + (size_t)c.W * kThrBytesPerWave +
          (size_t)c.TB * c.W * 4;
  if (c.lds > 160 * 1024) return false;
  return true;
}

template <int S, int CPT, int BITS, int W>
static hipError_t launch_one(const RotateArgs &a, const FastCfg &c, const uint32_t *scat,
                             const uint32_t *smask, const uint16_t *cells, const Thresholds &th,
                             int grid) {
  auto k = rq_fast_kernel<S, CPT, 4, BITS, W>;
  hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)c.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * W), c.lds, a.stream, (const uint16_t *)a.x,
                     a.n_tok, a.d, a.h, c.P, scat, smask, cells, th, (uint8_t *)a.out, a.norms);
  return hipGetLastError();
}

hipError_t launch_rotate_quantize_fast(const RotateArgs &a, const uint32_t *scat,
                                       const uint32_t *smask, const uint16_t *cells,
                                       const Thresholds &th, bool *handled) {
  *handled = false;
  FastCfg c;
  if (a.dtype != 1 || a.rotated_out || !fast_config(a.d, a.h, c)) return hipSuccess;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per_cu = (int)((160 * 1024) / c.lds) < 1 ? 1 : (int)((160 * 1024) / c.lds);
  const int64_t nb = (a.n_tok + c.TB - 1) / c.TB;
  const int64_t want = (int64_t)(cus > 0 ? cus : 256) * per_cu;
  const int grid = (int)(nb < want ? nb : want);
#define OQ_FAST(S_, CPT_, W_)                                                            \
  if (c.S == S_ && c.CPT == CPT_ && c.W == W_) {                                         \
    *handled = true;                                                                     \
    switch (a.bits) {                                                                    \
      case 2: return launch_one<S_, CPT_, 2, W_>(a, c, scat, smask, cells, th, grid);    \
      case 3: return launch_one<S_, CPT_, 3, W_>(a, c, scat, smask, cells, th, grid);    \
      default: return launch_one<S_, CPT_, 4, W_>(a, c, scat, smask, cells, th, grid);   \
    }                                                                                    \
  }
  OQ_FAST(1024, 2, 3)  // d = 3072, h = 1024
  OQ_FAST(1024, 2, 5)  // d = 5120, h = 1024
  OQ_FAST(512, 3, 9)   // d = 13824, h = 512
  OQ_FAST(1024, 2, 1)  // d = 1024
#undef OQ_FAST
  return hipSuccess;
}

}  // namespace oq
