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
//    CPT fixed 8-element chunks of every token: one 16-byte load per chunk
//    (issued one batch ahead when registers allow), the Rademacher signs
//    applied as an XOR (D moved onto the source index: D_i x_{pi(i)} =
//    (D_{pi^-1(j)} x_j) at j = pi(i)), and every element scattered with
//    ds_write_b16 to its permuted position pi^-1(j) in LDS.  Scatter
//    addresses and sign masks stay in registers for the whole kernel; d is a
//    template parameter so every LDS base folds into instruction offsets.
//    When the input arrives already in rotation order (the producer's output
//    rows were permuted by pi, see oq_permute_rows) the chunk is stored as
//    one 16-byte LDS write after the sign XOR: no scatter at all.
//  * Norm.  The 8 bf16 of a staged chunk are an MFMA operand as they are:
//    mfma(X, X) accumulates X X^T, whose trace is the sum of squares.
//  * Walsh-Hadamard, stages 0-4.  bf16 values are exact MFMA operands and
//    H_32 is +-1, so v_mfma_f32_16x16x32_bf16 applies the 32-point
//    transform of every 32-element chunk with fp32 accumulation.  The 16
//    rows of one MFMA are 4 chunks of 4 slots (a slot = one Hadamard block,
//    h <= 1024 here), so each lane ends up holding 4 chunks x 2 positions
//    of one slot per 128-coordinate group.
//  * Remaining stages (chunk bits) are register butterflies.
//  * Blocks of 2048 or 4096: the transform runs on 1024-element slots as
//    above, and the four slots of a wave tile (one per 16-lane row of the
//    MFMA output) are the 1024-element quarters of one block (or halves of
//    two blocks).  The last one or two butterfly stages pair the rows:
//    v_permlane16_swap / v_permlane32_swap hand each lane its partner's
//    value, and the butterfly leaves the slot bit in the register index and
//    a group bit in the lane, which the store addressing follows.
//  * Quantize.  A magic-number fma turns v into the byte offset of its cell
//    in a uniform grid over sqrt(d) z (narrower than any threshold gap:
//    step 1/8 over [-8, 8) up to 4 bits, 1/128 over [-5, 5) at 8 bits;
//    clamped to the grid, whose ends lie beyond every threshold); one 8-byte
//    LDS read gives the code at the cell's lower edge and the only threshold
//    that can fall inside the cell; one exact fp32 compare of sqrt(d) z with
//    it settles the code.  The table (1 KB, or 10 KB at 8 bits) does not
//    depend on the token, so it is loaded once per workgroup.
//  * Pack.  A lane's 8 codes per group are exactly 8 consecutive storage
//    slots, so they pack into one b-byte word per lane (8 bytes at 8 bits).  (Fake-quantization
//    mode instead stores bf16 s * level[code] at every coordinate.)
#include <hip/hip_runtime.h>

#include "oq_internal.h"

namespace oq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kMagic = 12582912.0f;        // 1.5 * 2^23

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
constexpr int isqrt_ceil(int v) {
  int r = 0;
  while (r * r < v) r++;
  return r;
}
constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

// Cell grid of one token length and bit width, in LDS: {float tau, uint
// base} per 8-byte cell and the fma scale from a unit-space value to bytes.
// Up to 4 bits the kernel takes the window of the device grid that holds
// every possible sqrt(d) z (|sqrt(d) z| <= sqrt(d) for a unit vector, plus
// two units of margin), so no value needs clamping; at 8 bits the grid
// spans [-5, 5) and values beyond are clamped onto its end cells.
template <int D, int BITS>
struct Grid {
  static constexpr bool CLAMP = BITS == 8;
  static constexpr int R = CLAMP ? 0 : isqrt_ceil(D) + 2;           // half-range, units
  static constexpr int CELLS = CLAMP ? kFastCells8 : 16 * R;       // step 1/8 up to 4 bits
  static constexpr int FIRST = CLAMP ? 0 : kFastCells / 2 - 8 * R;  // first device cell
  static constexpr int CELLB = 8 * CELLS;
  static constexpr float PER_UNIT = CLAMP ? 1024.0f : 64.0f;  // 8 / step
  // offset mask: keeps every offset inside the workgroup's LDS even for a NaN
  static constexpr uint32_t MASK = (uint32_t)pow2_ceil(CELLB) - 8u;
  static_assert(CLAMP || R <= kFastHalfUnits, "window inside the device grid");
  static_assert(FIRST % 2 == 0, "16-byte aligned window");
};



constexpr int pick_waves(int wt, int ch, int maxw) {
  int best = 1;
  for (int w = 1; w <= maxw; w++)
    if (wt % w == 0 && ch % w == 0) best = w;
  return best;
}

// Compile-time shape of the kernel for one d and bit width.
template <int D, int BITS>
struct Shape {
  static constexpr int H = D & -D;                    // Hadamard block
  static constexpr int S = H < 1024 ? H : 1024;       // slot: a block, or 1024 of one
  static constexpr int XB = ilog2(H / S);             // butterfly stages across slots
  static constexpr int P = D / S;                     // slots per token
  // tokens per batch: 4, or 2 for long tokens when the slots still tile
  static constexpr int TB = (D * 2 * 4 > 64 * 1024 && (2 * P) % 4 == 0) ? 2 : 4;
  static constexpr int WT = TB * P / 4;               // wave tiles per batch
  static constexpr int CH = D / 512;                  // 8-element chunks per token per 64 threads
  // waves per workgroup: divide both the wave tiles and the staging chunks;
  // with stages across slots at most 2 waves per SIMD (register budget)
  static constexpr int W = pick_waves(WT, CH, XB > 0 ? 8 : 16);
  static constexpr int CPT = CH / W;                  // chunks per thread per token
  static constexpr int G = S / 128;                   // 128-coordinate groups per slot
  static constexpr int CBITS = ilog2(S) - 5;          // chunk bits transformed in registers
  // LDS layout: tables first so their offsets fit instruction immediates
  static constexpr int CT_OFF = 0;                    // cell table, offsets are immediates
  static constexpr int NP_OFF = CT_OFF + Grid<D, BITS>::CELLB;  // [TB][W] partial sums of squares
  static constexpr int LV_OFF = NP_OFF + ((TB * W * 4 + 15) / 16) * 16;  // 2^BITS unit levels
  static constexpr int YB_OFF = LV_OFF + (4 << BITS);
  static constexpr int LDS = YB_OFF + TB * D * 2;
  // d = 5120 (five 5-wave workgroups' worth of tiles, 2 resident at 3
  // waves per SIMD) runs lean instead: no prefetch registers, 4 waves per
  // SIMD, 3 workgroups per CU -- measured 6% faster there and slower at
  // every other size.  d = 4096 (about 175 registers, 2 waves per SIMD)
  // is held to 3 waves per SIMD: a few spilled registers, 7-8% faster;
  // the same at d = 12288 spills about 80 (18% slower without prefetch)
  static constexpr bool LEAN = D == 5120;
  static constexpr int MIN_WAVES_PER_SIMD = LEAN ? 4 : (D == 4096 ? 3 : 1);
  // register budget of the one-batch-ahead prefetch
  static constexpr bool PREFETCH = !LEAN && (TB * CPT * 4) <= (W <= 8 ? 48 : 32);
  static_assert(S <= 1024 && S >= 128, "slot size");
  static_assert(XB <= 2 && (1 << XB) <= G, "at most 4 slots per block");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert((int)Grid<D, BITS>::MASK + 8 <= LDS, "masked offsets stay in the workgroup's LDS");
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// DQ: write bf16 s * level[code] at every coordinate (dq) instead of codes.
// IDENT: the input is already in rotation order (x'_i = x_{pi(i)}); scat is
// unused and smask holds the sign masks of the coordinates in place.
// table: the device codebook table (cell grid, then levels).
template <int D, int BITS, bool DQ, bool IDENT>
__global__ __launch_bounds__((64 * Shape<D, BITS>::W))
__attribute__((amdgpu_waves_per_eu(Shape<D, BITS>::MIN_WAVES_PER_SIMD, 8))) void rq_fast_kernel(
    const uint16_t *__restrict__ x, int64_t n_tok, const uint32_t *__restrict__ scat,
    const uint32_t *__restrict__ smask, const uint32_t *__restrict__ table,
    uint8_t *__restrict__ codes, uint16_t *__restrict__ dq, float *__restrict__ norms) {
  using SH = Shape<D, BITS>;
  using GR = Grid<D, BITS>;
  constexpr int CELLB = GR::CELLB;
  constexpr int S = SH::S, P = SH::P, TB = SH::TB, WT = SH::WT, W = SH::W, CPT = SH::CPT;
  constexpr int G = SH::G;
  // a static array: its base is a compile-time constant, so every table and
  // token-buffer offset below folds into the LDS instructions' immediates
  __shared__ __attribute__((aligned(16))) uint8_t lds[SH::LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float *npart = (float *)(lds + SH::NP_OFF);

  // cell table (and the levels, for fake quantization) into LDS
  for (int i = tid; i < CELLB / 16; i += W * 64)
    ((u32x4 *)(lds + SH::CT_OFF))[i] = ((const u32x4 *)(table + 2 * GR::FIRST))[i];
  if constexpr (DQ) {
    for (int i = tid; i < (1 << BITS); i += W * 64)
      ((uint32_t *)(lds + SH::LV_OFF))[i] = table[table_levels_word(BITS) + i];
  }

  // per-thread staging: chunk c of every token covers x[8*pos, 8*pos+8)
  uint32_t saddr[IDENT ? 1 : CPT][8], smk[CPT][4];
#pragma unroll
  for (int c = 0; c < CPT; c++) {
    const int pos = tid + c * W * 64;
    if constexpr (!IDENT) {
#pragma unroll
      for (int e = 0; e < 8; e++) saddr[c][e] = scat[pos * 8 + e];
    }
#pragma unroll
    for (int e = 0; e < 4; e++) smk[c][e] = smask[pos * 4 + e];
  }
  (void)saddr;

  // H_32 operands: lane holds H[k][n] for k = 8(lane>>4)+e, n = lane&15 (+16)
  bf16x8 hb0, hb1;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int k = 8 * (lane >> 4) + e, n = lane & 15;
    hb0[e] = (__builtin_popcount(k & n) & 1) ? (__bf16)-1.0f : (__bf16)1.0f;
    hb1[e] = (__builtin_popcount(k & (n + 16)) & 1) ? (__bf16)-1.0f : (__bf16)1.0f;
  }
  const float scale_hd = sqrtf((float)SH::H / (float)D);  // v-space threshold = tau s sqrt(h/d)
  constexpr int64_t row_bytes = (int64_t)D * BITS / 8;
  const int64_t nbatch = (n_tok + TB - 1) / TB;

  u32x4 stg[TB][CPT];
  auto load_batch = [&](int64_t b) {
#pragma unroll
    for (int tk = 0; tk < TB; tk++) {
      const int64_t t = b * TB + tk;
#pragma unroll
      for (int c = 0; c < CPT; c++)
        stg[tk][c] = (t < n_tok) ? *(const u32x4 *)(x + t * D + 8 * (tid + c * W * 64))
                                 : u32x4{0, 0, 0, 0};
    }
  };
  if constexpr (SH::PREFETCH) {
    if ((int64_t)blockIdx.x < nbatch) load_batch(blockIdx.x);
  }
  __syncthreads();

  for (int64_t b = blockIdx.x; b < nbatch; b += gridDim.x) {
    // ---- stage: norms by Gram MFMA, sign, scatter
    if constexpr (!SH::PREFETCH) load_batch(b);
#pragma unroll
    for (int tk = 0; tk < TB; tk++) {
      floatx4 gram = {0.f, 0.f, 0.f, 0.f};
      uint8_t *yb = lds + SH::YB_OFF + tk * D * 2;
#pragma unroll
      for (int c = 0; c < CPT; c++) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, stg[tk][c]);
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, xv, gram, 0, 0, 0);
        if constexpr (IDENT) {
          *(u32x4 *)(yb + 16 * (tid + c * W * 64)) =
              u32x4{stg[tk][c][0] ^ smk[c][0], stg[tk][c][1] ^ smk[c][1],
                    stg[tk][c][2] ^ smk[c][2], stg[tk][c][3] ^ smk[c][3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint32_t v = stg[tk][c][e] ^ smk[c][e];
            *(uint16_t *)(yb + saddr[c][2 * e]) = (uint16_t)v;
            *(uint16_t *)(yb + saddr[c][2 * e + 1]) = (uint16_t)(v >> 16);
          }
        }
      }
      // trace of the Gram matrix: diagonal entry r sits in lane 16(r/4)+r,
      // register r%4, so the 16 terms fill the quads of lanes 0-3, 20-23,
      // 40-43 and 60-63.  Two DPP swaps sum each quad, four lane reads
      // gather the quad sums: no LDS traffic (a 64-lane shuffle tree cost
      // 6 LDS permutes per token; d = 5120 ran 13% faster without them)
      const int r = lane & 15;
      float dg = ((r >> 2) == (lane >> 4)) ? gram[r & 3] : 0.f;
      dg += __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, dg), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
      dg += __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, dg), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
      const int dgi = __builtin_bit_cast(int, dg);
      const float q0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 0));
      const float q1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 20));
      const float q2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 40));
      const float q3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 60));
      if (lane == 0) npart[tk * W + wave] = (q0 + q1) + (q2 + q3);
    }
    if constexpr (SH::PREFETCH) {
      if (b + gridDim.x < nbatch) load_batch(b + gridDim.x);
    }
    __syncthreads();

    // ---- compute: wave tiles q = wave, wave + W, ...
    for (int q = wave; q < WT; q += W) {
      // output side: row rl = lane >> 4 of the tile.  Before the stages
      // across slots it holds slot 4q + rl; after them the low XB bits of
      // the slot are register-index bits (group bits, see below) and the low
      // XB bits of rl are group bits.  All slots a lane ends up with belong
      // to one token.
      const int rl = lane >> 4;
      const int sig_o = 4 * q + (rl & ~((1 << SH::XB) - 1));
      const int tko = sig_o / P, jo = sig_o - tko * P;
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; w++) ss += npart[tko * W + w];
      const float s = sqrtf(ss);
      const float us = (s > 0.f) ? 1.0f / (s * scale_hd) : 0.f;  // v -> sqrt(d) z
      const float a8 = us * GR::PER_UNIT;                        // 8 bytes per cell
      constexpr float m8 = kMagic + (float)(CELLB / 2);          // middle cell at u = 0
      // input side: MFMA row r = lane & 15 -> slot r>>2, chunk (r&3) of each group
      const int sig_i = 4 * q + ((lane & 15) >> 2);
      const int tki = sig_i / P, ji = sig_i - tki * P;
      const uint8_t *ya = lds + SH::YB_OFF + tki * D * 2 +
                          2 * (ji * S + 32 * (lane & 3) + 8 * (lane >> 4));

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
      // chunk stages: chunk = 4g + i
#pragma unroll
      for (int bit = 0; bit < SH::CBITS; bit++) {
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
          for (int w = 0; w < 2; w++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int ci = 4 * g + i, pi = ci ^ (1 << bit);
              if (ci < pi) {
                const float p0 = v[g][w][i], p1 = v[pi >> 2][w][pi & 3];
                v[g][w][i] = p0 + p1;
                v[pi >> 2][w][pi & 3] = p0 - p1;
              }
            }
      }
      // stages across the tile's slots: slot bit x pairs lane rows r, r ^ (1 << x)
#pragma unroll
      for (int x = 0; x < SH::XB; x++) {
#pragma unroll
        for (int g = 0; g < G; g++) {
          if (g & (1 << x)) continue;
          const int g2 = g | (1 << x);
#pragma unroll
          for (int w = 0; w < 2; w++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const uint32_t a = __float_as_uint(v[g][w][i]), c = __float_as_uint(v[g2][w][i]);
              // row pairs: this lane receives its partner's copy of the same
              // register; rows with bit x clear keep register g, the others g2
              const auto sw = (x == 0) ? __builtin_amdgcn_permlane16_swap(a, c, false, false)
                                       : __builtin_amdgcn_permlane32_swap(a, c, false, false);
              const float lo = __uint_as_float(sw[0]), hi = __uint_as_float(sw[1]);
              v[g][w][i] = lo + hi;   // slot bit x = 0
              v[g2][w][i] = lo - hi;  // slot bit x = 1
            }
        }
      }
      // quantize + pack + store.  Register group g holds slot jo + (g & m)
      // and group (g & ~m) | (rl & m) of that slot, m = 2^XB - 1.
      constexpr int XM = (1 << SH::XB) - 1;
      const int64_t tok = b * TB + tko;
      if ((lane & 15) == 0 && (rl & XM) == 0 && jo == 0 && tok < n_tok) norms[tok] = s;
      uint8_t *dst0 = codes + tok * row_bytes + 16 * BITS * (jo * G + (rl & XM)) + BITS * (lane & 15);
      // fake quantization: coordinate of register (g, w, i) is
      // (jo + (g & XM)) S + ((g & ~XM) | (rl & XM)) 128 + 32 i + 16 w + (lane & 15)
      uint16_t *dq0 = dq + tok * D + jo * S + (rl & XM) * 128 + (lane & 15);
      const float fs = s * (1.0f / __builtin_sqrtf((float)D));  // s / sqrt(d)
#pragma unroll
      for (int g = 0; g < G; g++) {
        uint32_t word = 0, word1 = 0;  // word1: codes 4-7 at 8 bits
#pragma unroll
        for (int w = 0; w < 2; w++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float val = v[g][w][i];
            // byte offset 8 floor(u / step + C/2 + 1/16) of the cell (u clamped
            // to the grid at 8 bits); the integer sits in the low mantissa bits
            const float fq = __builtin_fmaf(val, a8, m8);
            const float tq = GR::CLAMP ? __builtin_amdgcn_fmed3f(fq, kMagic, kMagic + (float)(CELLB - 1))
                                       : fq;
            const uint32_t off = __float_as_uint(tq) & GR::MASK;
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 ent = *(const u32x2 *)(lds + SH::CT_OFF + off);  // {tau, base}
            const uint32_t code = ent[1] + (val * us >= __uint_as_float(ent[0]) ? 1u : 0u);
            if constexpr (DQ) {
              // (code masked: a u outside the window -- only from a norm
              // that underflowed -- reads an arbitrary entry)
              const float lvv = *(const float *)(lds + SH::LV_OFF + 4 * (code & ((1u << BITS) - 1)));
              if (tok < n_tok)
                dq0[(g & XM) * S + (g & ~XM) * 128 + 32 * i + 16 * w] = f32_to_bf16_rne(fs * lvv);
            }
            if constexpr (BITS == 8) {
              if (w == 0) word |= code << (8 * i);
              else word1 |= code << (8 * i);
            } else {
              word |= code << (BITS * (4 * w + i));
            }
          }
        if (!DQ && tok < n_tok) {
          uint8_t *dst = dst0 + 16 * BITS * ((g & XM) * G + (g & ~XM));
          if constexpr (BITS == 8) {
            typedef uint32_t u32x2s __attribute__((ext_vector_type(2)));
            *(u32x2s *)dst = u32x2s{word, word1};
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
      }
    }
    __syncthreads();
  }
}

template <int D, int BITS>
hipError_t launch_one(const RotateArgs &a, const uint32_t *scat, const uint32_t *smask,
                      const uint32_t *table) {
  using SH = Shape<D, BITS>;
  auto k = a.dequant_out ? (a.input_permuted ? rq_fast_kernel<D, BITS, true, true>
                                             : rq_fast_kernel<D, BITS, true, false>)
                         : (a.input_permuted ? rq_fast_kernel<D, BITS, false, true>
                                             : rq_fast_kernel<D, BITS, false, false>);
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // persistent workgroups: exactly as many as can be resident at once
  // (registers and LDS decide), each looping over batches, so no second
  // partial round of workgroups and each pays its table set-up once
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * SH::W, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int64_t nb = (a.n_tok + SH::TB - 1) / SH::TB;
  const int64_t want = (int64_t)(cus > 0 ? cus : 256) * per_cu;
  const int grid = (int)(nb < want ? nb : want);
  uint8_t *codes = a.dequant_out ? nullptr : (uint8_t *)a.out;
  uint16_t *dq = a.dequant_out ? (uint16_t *)a.out : nullptr;
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * SH::W), 0, a.stream, (const uint16_t *)a.x,
                     a.n_tok, scat, smask, table, codes, dq, a.norms);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const RotateArgs &a, const uint32_t *scat, const uint32_t *smask,
                    const uint32_t *table) {
  switch (a.bits) {
    case 2: return launch_one<D, 2>(a, scat, smask, table);
    case 3: return launch_one<D, 3>(a, scat, smask, table);
    case 8: return launch_one<D, 8>(a, scat, smask, table);
    default: return launch_one<D, 4>(a, scat, smask, table);
  }
}

}  // namespace

hipError_t launch_rotate_quantize_fast(const RotateArgs &a, const uint32_t *scat,
                                       const uint32_t *smask, const uint32_t *table,
                                       bool *handled) {
  *handled = false;
  if (a.dtype != 1 || a.rotated_out) return hipSuccess;
  *handled = true;
  switch (a.d) {
    case 1024: return launch_d<1024>(a, scat, smask, table);
    case 2048: return launch_d<2048>(a, scat, smask, table);
    case 3072: return launch_d<3072>(a, scat, smask, table);
    case 4096: return launch_d<4096>(a, scat, smask, table);
    case 5120: return launch_d<5120>(a, scat, smask, table);
    case 12288: return launch_d<12288>(a, scat, smask, table);
    case 13824: return launch_d<13824>(a, scat, smask, table);
    default: break;
  }
  *handled = false;
  return hipSuccess;
}

}  // namespace oq
