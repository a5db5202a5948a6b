// rotate_quantize_fast.hip -- rotate + quantize for bf16 tokens on gfx950.
//
// Same result as the general kernel (rotate_quantize.hip): s = ||x||,
// y_i = D_i x_{pi(i)}, z = blockwise H_h y / (s sqrt(h)), code = number of
// unit Lloyd-Max thresholds at or below sqrt(d) z_i, packed in storage
// order (paper.gecl.asia notes, Method items 1, 3, 4; pith.science
// Supplementary A setup).  This path is built around the VALU budget of an
// HBM-bound kernel (about a dozen lane operations per coordinate):
//
//  * Roles.  A workgroup handles TB tokens per batch.  At d = 3072, 5120
//    and 13824 its waves have fixed roles: staging waves load and scatter
//    batch b+1 into one of two token buffers while compute waves transform
//    and quantize batch b from the other, so the LDS-bound scatter and the
//    VALU-bound transform run at the same time; elsewhere every wave stages
//    and then computes, with one token buffer.  A wave tile is 4 slots; at
//    d = 13824 (27 slots per token, one token per batch) the last tile
//    holds 3, and its fourth row works on a copy that is never stored.
//  * Staging.  Each staging thread owns CPT fixed 8-element chunks of every
//    token: one 16-byte load per chunk (issued one batch ahead when
//    registers allow), the Rademacher signs
//    applied as an XOR (D moved onto the source index: D_i x_{pi(i)} =
//    (D_{pi^-1(j)} x_j) at j = pi(i)), and every element scattered with
//    ds_write_b16 to its permuted position pi^-1(j) in LDS.  Scatter
//    addresses and sign masks stay in registers for the whole kernel; d is a
//    template parameter so every LDS base folds into instruction offsets.
//    When the input arrives already in rotation order (the producer's output
//    rows were permuted by pi, see oq_permute_rows) the chunk is stored as
//    one 16-byte LDS write after the sign XOR: no scatter at all.
//  * Norm.  The 8 bf16 of a staged chunk are an MFMA operand as they are:
//    mfma(X, X) accumulates X X^T, whose trace is the sum of squares.  With
//    split roles (d = 3072, 5120) the last staging wave to deliver its
//    partials of a batch (an LDS arrival counter; no wave waits) sums them
//    in wave order and finishes the norms before the batch's barrier.
//  * Walsh-Hadamard, stages 0-4.  bf16 values are exact MFMA operands and
//    H_32 is +-1, so v_mfma_f32_16x16x32_bf16 applies the 32-point
//    transform of every 32-element chunk with fp32 accumulation.  The 16
//    rows of one MFMA are 4 chunks of 4 slots (a slot = one Hadamard block
//    of at most 1024 coordinates, 512 at d = 3072 and 5120), so each lane
//    ends up holding 4 chunks x 2 positions of one slot per 128-coordinate
//    group.  The lowest group bit is usually transformed there too (two
//    accumulated k-blocks with the signs of H_2).
//  * Remaining stages (chunk bits) are register butterflies.
//  * Blocks larger than a slot (2048 or 4096, and the 1024 blocks of the
//    512-slot sizes): the four slots of a wave tile (one per 16-lane row of
//    the MFMA output) are the quarters of one block (or halves of two
//    blocks).  The last one or two butterfly stages pair the rows:
//    v_permlane16_swap / v_permlane32_swap hand each lane its partner's
//    value, and the butterfly leaves the slot bit in the register index and
//    a group bit in the lane, which the store addressing follows.  A 4096
//    block (4 slots of 1024, 64 values per lane) is split over two waves:
//    each produces the half of the groups with one value of the top group
//    bit, whose H_2 the matrix cores apply by accumulating both input
//    halves with its signs, so a wave holds 32 values per lane.
//  * Quantize.  A magic-number fma turns v into the byte offset of its cell
//    in a uniform grid over sqrt(d) z (narrower than any threshold gap:
//    step 1/8 up to 4 bits, over +-(ceil(sqrt(d)) + 2) units, which holds
//    every value a unit vector can take, so nothing is clamped; step 1/128
//    over [-5, 5) at 8 bits, values beyond clamped onto the end cells, which
//    lie beyond every threshold); one 8-byte LDS read gives the code at the
//    cell's lower edge and the only threshold that can fall inside the cell;
//    one exact fp32 compare of sqrt(d) z with it settles the code.  The
//    table window (4-15 KB, or 10 KB at 8 bits) does not depend on the
//    token, so it is loaded once per workgroup.
//  * Pack.  A lane's 8 codes per group are exactly 8 consecutive storage
//    slots, so they pack into one b-byte word per lane (8 bytes at 8 bits).  (Fake-quantization
//    mode instead stores bf16 s * level[code] at every coordinate, and the
//    rotated-value mode the fp32 unit vector z itself, both in coordinate
//    order.)
#include <hip/hip_runtime.h>

#include "oq_internal.h"


namespace oq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kMagic = 12582912.0f;        // 1.5 * 2^23

// compile-time half index of a split wave tile
template <int V>
struct Half {
  static constexpr int value = V;
};

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



// Per token size d, measured on MI355X (32760 x 5120, 9216 x 12288, 65536 x
// 3072, 16384 x 4096 tokens):
//  * mfma_group_bits: group bits of a slot (coordinate bits 7 .. 7+MB-1)
//    transformed on the matrix cores together with the five in-chunk bits:
//    the MFMA then applies a 2^(5+MB)-point Hadamard (the H_32 operand and
//    the +-1 signs of H_(2^MB) over 2^MB accumulated k-blocks), 2^(2MB+1)
//    MFMAs per 16 x 2^(5+MB) block instead of MB register butterfly stages.
//    One bit: 8-10% faster at d = 5120 (and at 12288 with one wave per
//    4096 block; equal there with the split tiles), equal at 1024, 3072 and
//    13824, 12% slower at 4096 (6-8% with the split tiles: more MFMA chains
//    than the register stages they replace); two or three bits were slower
//    everywhere.
//  * d = 5120 runs 512-coordinate slots (one permlane stage joins the two
//    halves of each 1024 block) so that a batch of two tokens still tiles
//    the five waves: half the staging registers, which leaves room for the
//    one-batch-ahead prefetch at 4 waves per SIMD (5% faster than four
//    tokens of 1024-coordinate slots without prefetch).
constexpr int mfma_group_bits(int d) { return (d == 2048 || d == 4096) ? 0 : 1; }
// Staging waves per workgroup (0: every wave stages and computes in turn).
// With staging waves, W compute waves transform and quantize batch b from
// one token buffer while the staging waves load batch b+2 and scatter
// batch b+1 into the other, one barrier per batch: the LDS-bound scatter
// and the VALU-bound transform run at the same time on different waves
// instead of one after the other.  d = 5120: 130 -> 96 us for 32760 tokens
// (two workgroups of 5 + 5 waves per CU, 70 registers); d = 3072 (512
// slots, two tokens per batch, 3 + 3 waves, four workgroups per CU): 3-6%
// faster, already close to the device's copy rate at 65536 tokens.  d =
// 13824 (27 slots of 512 per token): one token per batch in 7 wave tiles,
// the last holding 3 slots (the slots transform alone, so the missing one
// is a copy whose results are never stored), 7 + 9 waves, two workgroups
// per CU at 64 registers: 334 -> 223 us for 32760 tokens (four tokens per
// batch, the tile-aligned shape, left room for one 112 KB token buffer
// only).  d = 12288 keeps one role per wave (below).
constexpr int staging_waves(int d) { return d == 5120 ? 5 : (d == 3072 ? 3 : (d == 13824 ? 9 : 0)); }
// Compute waves per wave tile: 2 where the wave tile is a whole 4096 block
// (h = 4096: 4 slots of 1024).  Each of the two takes the half of the
// output groups with one value of the top group bit; the matrix cores
// apply that bit's H_2 too (its two input halves accumulated with signs),
// so a wave holds 32 values per lane instead of 64.  d = 12288 (two tokens
// per batch): 12 waves that each stage and compute, three per SIMD at 140
// registers, 91 -> 76-81 us for 9216 tokens (one wave per tile at 197
// registers left 1.5 waves per SIMD; split roles, 6 + 6 waves with one
// token per batch, spilled at the 80 registers two workgroups per CU
// allow and ran 13% slower than one wave per tile).  d = 4096: 114
// registers instead of 168 with spills, 2-4% faster for 16384 tokens.
constexpr int tile_split(int d) { return (d == 12288 || d == 4096) ? 2 : 1; }

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
  static constexpr int S = fast_slot(D);              // slot: a block, or 1024 (512) of one
  static constexpr int XB = ilog2(H / S);             // butterfly stages across slots
  static constexpr int P = D / S;                     // slots per token
  // tokens per batch: 4, or 2 for long tokens when the slots still tile;
  // 1 at d = 13824, whose 27 slots leave the last wave tile partial
  static constexpr int TB = D == 13824 ? 1
                            : ((D * 2 * 4 > 64 * 1024 || staging_waves(D)) && (2 * P) % 4 == 0) ? 2 : 4;
  static constexpr int NSLOT = TB * P;                // slots per batch
  static constexpr int GS = tile_split(D);            // compute waves per 4-slot tile
  static constexpr int WT = (NSLOT + 3) / 4 * GS;     // wave tiles per batch (the last may be partial)
  static constexpr int CH = D / 512;                  // 8-element chunks per token per 64 threads
  // waves per workgroup: divide both the wave tiles and the staging chunks;
  // with stages across slots on unsplit tiles at most 2 waves per SIMD
  // (register budget); with staging waves, one compute wave per tile
  static constexpr int W =
      staging_waves(D) ? WT : pick_waves(WT, CH, (XB > 0 && tile_split(D) == 1) ? 8 : 16);
  static constexpr int CPT = CH / W;                  // chunks per thread per token
  // split roles: W compute waves and WS staging waves (loads, norm partials,
  // scatter into the other of two token buffers)
  static constexpr int WS = staging_waves(D);
  static constexpr bool SPLIT = WS > 0;
  static constexpr int WTOT = W + WS;
  static constexpr int WSTG = SPLIT ? WS : W;          // waves that stage
  static constexpr int CPTS = CH / WSTG;               // staged chunks per thread per token
  static constexpr int NBUF = SPLIT ? 2 : 1;
  // with split roles the staging waves also finish each token's norm
  // (d = 5120: 1.5-3% faster; 3072 equal), except at d = 13824, whose
  // 64-register budget the finishing code overflows (3 spilled, 1% slower)
  static constexpr bool FIN = SPLIT && D != 13824;
  static constexpr int G = S / 128;                   // 128-coordinate groups per slot
  static constexpr int GW = G / GS;                   // groups of a slot one wave holds
  static constexpr int CBITS = ilog2(S) - 5;          // chunk bits (above the 32-element chunk)
  // group bits (coordinate bits 7 .. 7+MB-1) transformed on the matrix cores
  // together with the five in-chunk bits; the other chunk bits are register
  // butterflies
  static constexpr int MB = mfma_group_bits(D) < ilog2(G) ? mfma_group_bits(D) : ilog2(G);
  // a slot takes SP elements of LDS: 8 of padding shift the next slot by one
  // 16-byte bank group, so the 16 operand rows of an MFMA (4 slots x 4
  // chunks) fall on 16 different bank groups
  static constexpr int SP = S + 8;
  static constexpr int TOKB = P * SP * 2;             // bytes per token in LDS
  // LDS layout: tables first so their offsets fit instruction immediates
  static constexpr int CT_OFF = 0;                    // cell table, offsets are immediates
  static constexpr int NP_OFF = CT_OFF + Grid<D, BITS>::CELLB;  // [NBUF][TB][WSTG] sums of squares
  // FIN: [NBUF][TB] finished {s, 1/(s sqrt(h/d))} per token, and [NBUF]
  // arrival counters of the staging waves
  static constexpr int FN_OFF = NP_OFF + ((NBUF * TB * WSTG * 4 + 15) / 16) * 16;
  static constexpr int CN_OFF = FN_OFF + ((NBUF * TB * 8 + 15) / 16) * 16;
  static constexpr int LV_OFF = CN_OFF + 16;  // unit levels
  static constexpr int YB_OFF = LV_OFF + (4 << BITS);
  static constexpr int LDS = YB_OFF + NBUF * TB * TOKB;
  // register target (waves per SIMD): 5 with staging waves (about 70
  // registers); 8 at d = 13824 (64 registers, so two 16-wave workgroups
  // share a CU: 3% faster than one); with split tiles 3 at d = 12288 (one
  // 12-wave workgroup per CU) and 4 at d = 4096 (two 8-wave workgroups)
  static constexpr int MIN_WAVES_PER_SIMD =
      D == 13824 ? 8 : D == 12288 ? 3 : SPLIT ? 5 : (D == 4096 ? 4 : 1);
  // register budget of the one-batch-ahead prefetch
  static constexpr bool PREFETCH = SPLIT || (TB * CPT * 4) <= (W <= 8 ? 48 : 32);
  static_assert(S <= 1024 && S >= 128, "slot size");
  static_assert(XB <= 2 && (1 << XB) <= GW, "at most 4 slots per block, held by one wave");
  static_assert(GS == 1 || (GS == 2 && (1 << MB) <= GW), "a split tile keeps the low group bits");
  static_assert(NSLOT % 4 == 0 || XB == 0, "a partial last tile needs slots that transform alone");
  static_assert(CH % WSTG == 0, "every staging thread owns whole chunks");
  static_assert(!SPLIT || W == WT, "one compute wave per wave tile");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert((int)Grid<D, BITS>::MASK + 8 <= LDS, "masked offsets stay in the workgroup's LDS");
};

typedef float floatx2 __attribute__((ext_vector_type(2)));

// s = sqrt(ss) and us = 1 / (s sqrt(h/d)) (v -> sqrt(d) z) by the hardware
// square root and reciprocal (1 ulp each; a sum of squares below 2^-64 is
// scaled by 2^64 first, away from the range where the square root loses
// accuracy): a few instructions instead of the correctly rounded
// sequences, and the codes only move inside the decision windows that
// rounding of the transform already leaves
__device__ __forceinline__ floatx2 token_norm(float ss, float scale_hd) {
  const bool tiny = ss < 0x1p-64f;
  const float s = __builtin_amdgcn_sqrtf(tiny ? ss * 0x1p64f : ss) * (tiny ? 0x1p-32f : 1.0f);
  return floatx2{s, (s > 0.f) ? __builtin_amdgcn_rcpf(s * scale_hd) : 0.f};
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// What the kernel writes besides the norms.
enum OutMode { kCodes = 0, kDequant = 1, kRotated = 2 };

// MODE: kCodes packs codes; kDequant writes bf16 s * level[code] at every
// coordinate (dq); kRotated writes the fp32 unit vector z = H_h y / (s
// sqrt(h)) at every coordinate (zout) and skips the quantizer.
// IDENT: the input is already in rotation order (x'_i = x_{pi(i)}); scat is
// unused and smask holds the sign masks of the coordinates in place.
// table: the device codebook table (cell grid, then levels).
template <int D, int BITS, int MODE, bool IDENT>
__global__ __launch_bounds__((64 * Shape<D, BITS>::WTOT))
__attribute__((amdgpu_waves_per_eu(Shape<D, BITS>::MIN_WAVES_PER_SIMD, 8))) void rq_fast_kernel(
    const uint16_t *__restrict__ x, int64_t n_tok, const uint32_t *__restrict__ scat,
    const uint32_t *__restrict__ smask, const uint32_t *__restrict__ table,
    uint8_t *__restrict__ codes, uint16_t *__restrict__ dq, float *__restrict__ zout,
    float *__restrict__ norms) {
  using SH = Shape<D, BITS>;
  using GR = Grid<D, BITS>;
  constexpr bool DQ = MODE == kDequant, ZO = MODE == kRotated;
  constexpr int CELLB = GR::CELLB;
  constexpr int S = SH::S, P = SH::P, TB = SH::TB, WT = SH::WT, W = SH::W, CPT = SH::CPTS;
  constexpr int WSTG = SH::WSTG, WTOT = SH::WTOT;
  constexpr int G = SH::G, GW = SH::GW;
  // a static array: its base is a compile-time constant, so every table and
  // token-buffer offset below folds into the LDS instructions' immediates
  __shared__ __attribute__((aligned(16))) uint8_t lds[SH::LDS];
  const int tid0 = threadIdx.x, lane = tid0 & 63, wave = tid0 >> 6;
  const bool stager = !SH::SPLIT || wave >= W;    // this wave stages
  const int swave = SH::SPLIT ? wave - W : wave;   // index among the staging waves
  const int tid = swave * 64 + lane;               // staging thread index
  float *npart = (float *)(lds + SH::NP_OFF);
  floatx2 *fin = (floatx2 *)(lds + SH::FN_OFF);
  uint32_t *arrived = (uint32_t *)(lds + SH::CN_OFF);
  if constexpr (SH::FIN) {
    // zeroed before any staging wave counts (the barrier runs in every wave)
    if (tid0 < SH::NBUF) arrived[tid0] = 0;
    __syncthreads();
  }

  // cell table (and the levels, for fake quantization) into LDS
  if constexpr (!ZO) {
    for (int i = tid0; i < CELLB / 16; i += WTOT * 64)
      ((u32x4 *)(lds + SH::CT_OFF))[i] = ((const u32x4 *)(table + 2 * GR::FIRST))[i];
  }
  if constexpr (DQ) {
    for (int i = tid0; i < (1 << BITS); i += WTOT * 64)
      ((uint32_t *)(lds + SH::LV_OFF))[i] = table[table_levels_word(BITS) + i];
  }

  // per-thread staging: chunk c of every token covers x[8*pos, 8*pos+8)
  uint32_t saddr[IDENT ? 1 : CPT][8], smk[CPT][4];
#pragma unroll
  for (int c = 0; c < CPT; c++) {
    const int pos = (stager ? tid : 0) + c * WSTG * 64;
    if constexpr (!IDENT) {
#pragma unroll
      for (int e = 0; e < 8; e++) saddr[c][e] = scat[pos * 8 + e];
    }
#pragma unroll
    for (int e = 0; e < 4; e++) smk[c][e] = smask[pos * 4 + e];
  }
  (void)saddr;

  // H_32 operands: lane holds H[k][n] for k = 8(lane>>4)+e, n = lane&15 (+16)
  // (nhb: the same negated, for the -1 entries of H_(2^MB))
  bf16x8 hb0, hb1, nhb0, nhb1;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int k = 8 * (lane >> 4) + e, n = lane & 15;
    const bool n0 = __builtin_popcount(k & n) & 1, n1 = __builtin_popcount(k & (n + 16)) & 1;
    hb0[e] = n0 ? (__bf16)-1.0f : (__bf16)1.0f;
    hb1[e] = n1 ? (__bf16)-1.0f : (__bf16)1.0f;
    nhb0[e] = n0 ? (__bf16)1.0f : (__bf16)-1.0f;
    nhb1[e] = n1 ? (__bf16)1.0f : (__bf16)-1.0f;
  }
  const float scale_hd = sqrtf((float)SH::H / (float)D);  // v-space threshold = tau s sqrt(h/d)
  constexpr int64_t row_bytes = (int64_t)D * BITS / 8;
  const int64_t nbatch = (n_tok + TB - 1) / TB;

  // the lane's diagonal Gram register as one-hot weights (all zero off
  // the diagonal lanes), made once: selecting the term is then a product
  // and three multiply-adds of exact zeros and ones, no compares per token
  float dsel[4];
  {
    const int r = lane & 15;
    const bool on_diag = (r >> 2) == (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; i++) dsel[i] = (on_diag && (r & 3) == i) ? 1.f : 0.f;
  }
  u32x4 stg[TB][CPT];
  // non-temporal loads: every token is read once, so its lines need not
  // displace what the caches hold -- in a layer the output the previous
  // kernel has just written (a linear's 1 GB at 32760 x 15360), whose
  // write-back the displacement would otherwise pull into this kernel's
  // time (32760 x 5120 after such a linear: 102.6 -> 91.3 us)
  auto load_batch = [&](int64_t b) {
    if (b * TB + TB <= n_tok) {
      // a whole batch (every batch but possibly the last): no per-token
      // bounds checks (1-2% at 32760 x 5120)
#pragma unroll
      for (int tk = 0; tk < TB; tk++) {
        const int64_t t = b * TB + tk;
#pragma unroll
        for (int c = 0; c < CPT; c++)
          stg[tk][c] = __builtin_nontemporal_load(
              (const u32x4 *)(x + t * D + 8 * (tid + c * WSTG * 64)));
      }
      return;
    }
#pragma unroll
    for (int tk = 0; tk < TB; tk++) {
      const int64_t t = b * TB + tk;
#pragma unroll
      for (int c = 0; c < CPT; c++)
        stg[tk][c] = (t < n_tok) ? __builtin_nontemporal_load(
                                       (const u32x4 *)(x + t * D + 8 * (tid + c * WSTG * 64)))
                                 : u32x4{0, 0, 0, 0};
    }
  };
  // staging of the batch held in stg into token buffer nb: norms by Gram
  // MFMA, signs, scatter
  auto stage_batch = [&](int nb) {
#pragma unroll
    for (int tk = 0; tk < TB; tk++) {
      floatx4 gram = {0.f, 0.f, 0.f, 0.f};
      uint8_t *yb = lds + SH::YB_OFF + (nb * TB + tk) * SH::TOKB;
#pragma unroll
      for (int c = 0; c < CPT; c++) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, stg[tk][c]);
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, xv, gram, 0, 0, 0);
        if constexpr (IDENT) {
          // chunk pos of the token: slot pos / (S/8), 16 bytes of padding per slot
          const int pos = tid + c * WSTG * 64;
          *(u32x4 *)(yb + 16 * (pos + pos / (S / 8))) =
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
      float dg = gram[0] * dsel[0] + gram[1] * dsel[1] + gram[2] * dsel[2] + gram[3] * dsel[3];
      dg += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, dg), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
      dg += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, dg), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
      const int dgi = __builtin_bit_cast(int, dg);
      const float q0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 0));
      const float q1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 20));
      const float q2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 40));
      const float q3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(dgi, 60));
      if (lane == 0) npart[(nb * TB + tk) * WSTG + swave] = (q0 + q1) + (q2 + q3);
    }
    if constexpr (SH::FIN) {
      // the last staging wave to deliver its partials of this buffer sums
      // them (in wave order, whichever wave it is) and finishes every
      // token's norm before the batch's barrier, so the compute waves read
      // one value per token; nothing waits here
      uint32_t prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(arrived + nb, 1u, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev % WSTG == WSTG - 1 && lane < TB) {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < WSTG; w++) ss += npart[(nb * TB + lane) * WSTG + w];
        fin[nb * TB + lane] = token_norm(ss, scale_hd);
      }
    }
  };
  if constexpr (SH::SPLIT) {
    if (stager) {
      // staging waves: their own loop (its registers are not live in the
      // compute waves' loop): batch b+1 into the other buffer while the
      // compute waves work on batch b, one barrier per batch
      if ((int64_t)blockIdx.x < nbatch) {
        load_batch(blockIdx.x);
        stage_batch(0);
        if ((int64_t)(blockIdx.x + gridDim.x) < nbatch) load_batch(blockIdx.x + gridDim.x);
      }
      __syncthreads();
      // two batches per iteration, so the token buffer (and with it every
      // scatter address offset) is a compile-time constant: the offsets go
      // into the LDS stores' immediate field instead of one add per element
      const int64_t g = gridDim.x;
      for (int64_t b = blockIdx.x; b < nbatch; b += 2 * g) {
        if (b + g < nbatch) {
          stage_batch(1);
          if (b + 2 * g < nbatch) load_batch(b + 2 * g);
        }
        __syncthreads();
        if (b + g >= nbatch) break;
        if (b + 2 * g < nbatch) {
          stage_batch(0);
          if (b + 3 * g < nbatch) load_batch(b + 3 * g);
        }
        __syncthreads();
      }
      return;
    }
  } else if constexpr (SH::PREFETCH) {
    if ((int64_t)blockIdx.x < nbatch) load_batch(blockIdx.x);
  }
  __syncthreads();

  int it = 0;
  for (int64_t b = blockIdx.x; b < nbatch; b += gridDim.x, it++) {
    const int cur = SH::SPLIT ? (it & 1) : 0;
    if constexpr (!SH::SPLIT) {
      if constexpr (!SH::PREFETCH) load_batch(b);
      stage_batch(0);
      if constexpr (SH::PREFETCH) {
        if (b + gridDim.x < nbatch) load_batch(b + gridDim.x);
      }
      __syncthreads();
    }

    // ---- compute: wave tiles q = wave, wave + W, ...; wave tile q is half
    // hh of 4-slot tile qt when a tile is split over two waves
    for (int q = wave; q < WT; q += W) {
      const int qt = q / SH::GS;
      const int hh = SH::GS == 1 ? 0 : __builtin_amdgcn_readfirstlane(q % SH::GS);
      // output side: row rl = lane >> 4 of the tile.  Before the stages
      // across slots it holds slot 4q + rl; after them the low XB bits of
      // the slot are register-index bits (group bits, see below) and the low
      // XB bits of rl are group bits.  All slots a lane ends up with belong
      // to one token.
      const int rl = lane >> 4;
      // rows past the batch's last slot (a partial last tile; only without
      // stages across slots) compute on a copy of that slot and store nothing
      const int sig_r = 4 * qt + (rl & ~((1 << SH::XB) - 1));
      const bool row_ok = SH::NSLOT % 4 == 0 || sig_r < SH::NSLOT;
      const int sig_o = row_ok ? sig_r : SH::NSLOT - 1;
      const int tko = sig_o / P, jo = sig_o - tko * P;
      floatx2 nrm;
      if constexpr (SH::FIN) {
        nrm = fin[cur * TB + tko];  // finished by the staging waves
      } else {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < WSTG; w++) ss += npart[(cur * TB + tko) * WSTG + w];
        nrm = token_norm(ss, scale_hd);
      }
      const float s = nrm[0], us = nrm[1];  // us: v -> sqrt(d) z
      const float a8 = us * GR::PER_UNIT;                        // 8 bytes per cell
      constexpr float m8 = kMagic + (float)(CELLB / 2);          // middle cell at u = 0
      // input side: MFMA row r = lane & 15 -> slot r>>2, chunk (r&3) of each group
      const int sig_i = min(4 * qt + ((lane & 15) >> 2), SH::NSLOT - 1);
      const int tki = sig_i / P, ji = sig_i - tki * P;
      const uint8_t *ya = lds + SH::YB_OFF + (cur * TB + tki) * SH::TOKB +
                          2 * (ji * SH::SP + 32 * (lane & 3) + 8 * (lane >> 4));

      // Matrix cores: MFMA row r = (slot r>>2, chunk (r&3) of a group), k =
      // the 32 elements of the chunk.  Accumulating the k-blocks of GA
      // consecutive groups with the signs of H_GA applies the Hadamard over
      // the in-chunk bits and the low MB group bits at once (the Sylvester
      // matrix is a Kronecker product over the coordinate bits, so its
      // factors can be applied in any order and any grouping).  Output
      // block b of group block gb lands in register group gb GA + b.  With
      // a split tile the top group bit joins them: the wave of half hh
      // accumulates both halves a1 of the slot's groups with the sign of
      // H_2[hh][a1], and its register group g is group hh GW + g.
      constexpr int GA = 1 << SH::MB, GB = GW / GA, GS = SH::GS;
      float v[GW][2][4];
      auto transform = [&](auto half) {
        constexpr int HH = decltype(half)::value;
#pragma unroll
        for (int gb = 0; gb < GB; gb++) {
          floatx4 acc[GA][2];
#pragma unroll
          for (int b = 0; b < GA; b++) acc[b][0] = acc[b][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int a1 = 0; a1 < GS; a1++)
#pragma unroll
            for (int a = 0; a < GA; a++) {
              const bf16x8 av = *(const bf16x8 *)(ya + 256 * (a1 * GW + gb * GA + a));
#pragma unroll
              for (int b = 0; b < GA; b++) {
                const bool neg = (__builtin_popcount(a & b) & 1) ^ (a1 & HH);
                acc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, neg ? nhb0 : hb0, acc[b][0],
                                                                    0, 0, 0);
                acc[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, neg ? nhb1 : hb1, acc[b][1],
                                                                    0, 0, 0);
              }
            }
#pragma unroll
          for (int b = 0; b < GA; b++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              v[gb * GA + b][0][i] = acc[b][0][i];
              v[gb * GA + b][1][i] = acc[b][1][i];
            }
        }
      };
      if (hh == 0) transform(Half<0>{});
      else if constexpr (GS == 2) transform(Half<1>{});
      // butterfly (scaling comes later: an fma(p0, us, -p1 us) would turn an
      // exact cancellation p0 = p1 into a rounding residue of either sign,
      // and an exact zero sits on a decision threshold)
      auto bfly = [](float &x0, float &x1, float p0, float p1) {
        x0 = p0 + p1;
        x1 = p0 - p1;
      };
      // register stages over the chunk bits the matrix cores did not take:
      // chunk = 4g + i, bits 0-1 are i, bits 2.. are g
      constexpr int NCB = SH::CBITS - SH::MB - (GS - 1);  // register chunk stages
#pragma unroll
      for (int st = 0; st < NCB; st++) {
        const int bit = st < 2 ? st : st + SH::MB;
#pragma unroll
        for (int g = 0; g < GW; g++)
#pragma unroll
          for (int w = 0; w < 2; w++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int ci = 4 * g + i, pi = ci ^ (1 << bit);
              if (ci < pi)
                bfly(v[g][w][i], v[pi >> 2][w][pi & 3], v[g][w][i], v[pi >> 2][w][pi & 3]);
            }
      }
      // stages across the tile's slots: slot bit x pairs lane rows r, r ^ (1 << x)
#pragma unroll
      for (int x = 0; x < SH::XB; x++) {
#pragma unroll
        for (int g = 0; g < GW; g++) {
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
              // slot bit x = 0 / 1
              bfly(v[g][w][i], v[g2][w][i], __uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
        }
      }
      // quantize + pack + store.  Register group g holds slot jo + (g & m)
      // and group hh GW + (g & ~m) | (rl & m) of that slot, m = 2^XB - 1.
      constexpr int XM = (1 << SH::XB) - 1;
      // tok_end: stores happen for tok < tok_end (n_tok, or 0 for rows past
      // the batch's last slot)
      const int64_t tok = b * TB + tko, tok_end = row_ok ? n_tok : 0;
      if ((lane & 15) == 0 && (rl & XM) == 0 && jo == 0 && hh == 0 && tok < tok_end) norms[tok] = s;
      const int gh = hh * GW;  // first group of this wave's half
      uint8_t *dst0 =
          codes + tok * row_bytes + 16 * BITS * (jo * G + gh + (rl & XM)) + BITS * (lane & 15);
      // fake quantization: coordinate of register (g, w, i) is
      // (jo + (g & XM)) S + (gh + (g & ~XM) | (rl & XM)) 128 + 32 i + 16 w + (lane & 15)
      uint16_t *dq0 = dq + tok * D + jo * S + (gh + (rl & XM)) * 128 + (lane & 15);
      const float fs = s * (1.0f / __builtin_sqrtf((float)D));  // s / sqrt(d)
      if constexpr (ZO) {
        // rotated values: z = v us / sqrt(d), same coordinates as above
        const float rsd = us / __builtin_sqrtf((float)D);
        float *z0 = zout + tok * D + jo * S + (gh + (rl & XM)) * 128 + (lane & 15);
        if (tok < tok_end) {
#pragma unroll
          for (int g = 0; g < GW; g++)
#pragma unroll
            for (int w = 0; w < 2; w++)
#pragma unroll
              for (int i = 0; i < 4; i++)
                z0[(g & XM) * S + (g & ~XM) * 128 + 32 * i + 16 * w] = v[g][w][i] * rsd;
        }
        continue;  // wave-uniform: no codes in this mode
      }
#pragma unroll
      for (int g = 0; g < GW; g++) {
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
              if (tok < tok_end)
                dq0[(g & XM) * S + (g & ~XM) * 128 + 32 * i + 16 * w] = f32_to_bf16_rne(fs * lvv);
            }
            if constexpr (BITS == 8) {
              if (w == 0) word |= code << (8 * i);
              else word1 |= code << (8 * i);
            } else {
              word |= code << (BITS * (4 * w + i));
            }
          }
        if (!DQ && tok < tok_end) {
          // non-temporal, like the token loads: the codes of a step (84 MB
          // at 32760 x 5120) need not displace other lines on their way to
          // HBM; the linear that reads them next was measured no slower
          // (32760 x 5120: 90.3 -> 88.3 us; 9216 x 3072: 20.5 -> 19.2 us)
          uint8_t *dst = dst0 + 16 * BITS * ((g & XM) * G + (g & ~XM));
          if constexpr (BITS == 8) {
            typedef uint32_t u32x2s __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2s{word, word1}, (u32x2s *)dst);
          } else if constexpr (BITS == 4) {
            __builtin_nontemporal_store(word, (uint32_t *)dst);
          } else if constexpr (BITS == 2) {
            __builtin_nontemporal_store((uint16_t)word, (uint16_t *)dst);
          } else {
            __builtin_nontemporal_store((uint8_t)word, dst);
            __builtin_nontemporal_store((uint8_t)(word >> 8), dst + 1);
            __builtin_nontemporal_store((uint8_t)(word >> 16), dst + 2);
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int D, int BITS, int MODE>
hipError_t launch_one(const RotateArgs &a, const uint32_t *scat, const uint32_t *smask,
                      const uint32_t *table) {
  using SH = Shape<D, BITS>;
  auto k = a.input_permuted ? rq_fast_kernel<D, BITS, MODE, true>
                            : rq_fast_kernel<D, BITS, MODE, false>;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // persistent workgroups: exactly as many as can be resident at once
  // (registers and LDS decide), each looping over batches, so no second
  // partial round of workgroups and each pays its table set-up once
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * SH::WTOT, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int64_t nb = (a.n_tok + SH::TB - 1) / SH::TB;
  const int64_t want = (int64_t)(cus > 0 ? cus : 256) * per_cu;
  const int grid = (int)(nb < want ? nb : want);
  uint8_t *codes = MODE == kCodes ? (uint8_t *)a.out : nullptr;
  uint16_t *dq = MODE == kDequant ? (uint16_t *)a.out : nullptr;
  float *zout = MODE == kRotated ? (float *)a.out : nullptr;
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * SH::WTOT), 0, a.stream, (const uint16_t *)a.x,
                     a.n_tok, scat, smask, table, codes, dq, zout, a.norms);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_mode(const RotateArgs &a, const uint32_t *scat, const uint32_t *smask,
                       const uint32_t *table) {
  return a.dequant_out ? launch_one<D, BITS, kDequant>(a, scat, smask, table)
                       : launch_one<D, BITS, kCodes>(a, scat, smask, table);
}

template <int D>
hipError_t launch_d(const RotateArgs &a, const uint32_t *scat, const uint32_t *smask,
                    const uint32_t *table) {
  // rotated values do not depend on the bit width: one instantiation
  if (a.rotated_out) return launch_one<D, 4, kRotated>(a, scat, smask, table);
  switch (a.bits) {
    case 2: return launch_mode<D, 2>(a, scat, smask, table);
    case 3: return launch_mode<D, 3>(a, scat, smask, table);
    case 8: return launch_mode<D, 8>(a, scat, smask, table);
    default: return launch_mode<D, 4>(a, scat, smask, table);
  }
}

}  // namespace

hipError_t launch_rotate_quantize_fast(const RotateArgs &a, const uint32_t *scat,
                                       const uint32_t *smask, const uint32_t *table,
                                       bool *handled) {
  *handled = false;
  if (a.dtype != 1) return hipSuccess;
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
