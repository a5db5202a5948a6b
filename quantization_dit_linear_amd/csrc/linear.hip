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
//     the row's 64 codes into fp16 levels.  With 4-bit codes on both sides
//     an LDS table maps each code byte (two slots) straight to the fp16
//     pair, four 32-bit LDS reads per 8 slots and about one VALU instruction
//     per MFMA (32 lane-interleaved copies of the table keep the random
//     lookups from piling onto a few banks); 4-bit activations use the same
//     table against weights of another width, regrouped into the slot order
//     of the weights' decode (two byte permutes per 8 slots); every other
//     row uses v_perm_b32 byte tables (the fp16 low and high bytes of the
//     2^b levels; no memory lookups);
//   * decoded tiles live in LDS, double buffered, as 8 planes of 256 rows x
//     16 bytes (one plane per 8-slot chunk): the decode stores and the MFMA
//     fragment loads both touch consecutive 16-byte words, so neither has
//     bank conflicts and every offset is an instruction immediate (the
//     per-lane bases are kept opaque to the compiler so it cannot fold them
//     into one register per fragment);
//   * each of the 8 waves multiplies a 128 x 64 block with
//     v_mfma_f32_16x16x32_f16 (fp32 accumulation), weight fragment first so
//     every lane ends up with 4 consecutive output columns;
//   * one K step is one branch-free block of 8 chunks; chunk c issues 8
//     MFMAs of step t, loads fragments for chunk c+1, decodes slot chunk c of
//     step t+1 and stores it.  Scheduling fences between chunks keep the
//     decode spread between the MFMAs, so both waves of a SIMD always have
//     other work to issue while the matrix core runs; codes are loaded two
//     steps ahead into alternating registers;
//   * epilogue: scale by s_m r_n / K (the tile's norms were loaded at tile
//     start and pass through LDS), round once to bf16 with the hardware's
//     round to nearest even; each wave stages its bf16 block in its own LDS
//     region (XOR-swizzled 128-byte rows) and stores whole rows in 16-byte
//     pieces;
//   * persistent workgroups (one per CU); workgroup -> tile order is
//     contiguous per XCD and grouped along M, so tiles resident together
//     share activation rows in L2, and a tile's stores drain while the next
//     tile starts;
//   * a sparse last round (at most a quarter of the CUs' worth of tiles)
//     would leave one CU per tile running a whole K loop alone; those tiles
//     run first instead, as 128 x 128 sub-tiles cut into K ranges that fill
//     every CU, with their fp32 partial sums parked in output rows that the
//     full rounds overwrite afterwards, and a small kernel sums them.
//
// Throughput: 45-50% of the fp16 matrix-core peak at these shapes (45-47%
// at 9216 x 9216 x 3072, on par with the plain fp16 library GEMM of that
// shape, which does no decoding; 46-50% with 32760 tokens, 0.81-0.87 of
// it there); the K loop's LDS traffic (fragment loads, table lookups,
// decoded stores) and barriers take most of the rest.
//
// 8-bit codes (W8A8) take the same path except for the decode: 256 levels do
// not fit byte-permute tables, so each workgroup first converts the fp32
// unit levels to an fp16 table at the start of LDS (32 interleaved copies,
// as for the 4-bit pairs; activation and weight codes of one linear share
// K, bit width and codebook family, so they share the table) and a code
// becomes one LDS read; these reads run one chunk ahead of their stores.
// The decoded tiles follow the table.
#include <hip/hip_runtime.h>

#include <cstring>

#include "oq_internal.h"

namespace oq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int KS = 64;      // K step (slots)
constexpr int GROUP_M = 8;  // tile rows per group of the tile order
constexpr int BIG = 256;    // main tile edge

// Tile shape: TT x TT output tile, WM x WN waves, one decoded row per thread.
template <int TT, int WM, int WN, int LUTC_, int WGS_>
struct Tile {
  static constexpr int T = TT;
  static constexpr int LUTC = LUTC_;              // interleaved copies of an LDS code table
  static constexpr int WGS = WGS_;                // workgroups meant to share a CU
  static constexpr int THREADS = 2 * TT;          // TT activation + TT weight rows
  static constexpr int IB = TT / WM / 16;         // 16-row activation blocks per wave
  static constexpr int JB = TT / WN / 16;         // 16-row weight blocks per wave
  static constexpr int PLANE = TT * 16;           // one 8-slot chunk of TT rows
  static constexpr int OPB = 8 * PLANE;           // bytes per operand tile
  static constexpr int STAGEB = 2 * OPB;          // A + B per stage
  static constexpr int LDS = 2 * STAGEB;          // double buffered
  static_assert(WM * WN * 64 == THREADS, "one wave per 64 rows");
  static_assert(IB % 4 == 0 && JB >= 1, "4 chunks per K half");
};
// 256 x 256: 128 x 64 per wave, 128 KB of tiles + a 32 KB table fill the
// CU.  128 x 128: 64 x 64 per wave (one wave per SIMD per workgroup), 64 KB
// of tiles + a 16 KB table, so two workgroups share a CU.
using BigTile = Tile<256, 2, 4, 32, 1>;
using SmallTile = Tile<128, 2, 2, 16, 2>;

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
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

// LDS code tables (4 bits on both sides, and 8 bits): 256 32-bit entries,
// stored as C interleaved copies (entry e of copy c at word C e + c) and
// read by lane l from copy l mod C, so the random lookups of a wave spread
// over the banks instead of piling onto a few (C = 32 for 256 x 256 tiles:
// 2-4% faster than 16, and 32 KB with the two 64 KB tile stages fills the
// CU's 160 KB exactly).  `lut` below already points at the lane's copy.
template <int C>
__device__ __forceinline__ uint32_t lut_at(const uint32_t *lut, uint32_t e) {
  return lut[e * C];
}

// 8 bits: slots 8q .. 8q+7 are bytes 0-3 of w[2q] and w[2q+1]; each code
// reads its fp16 level (low half of the entry), and the levels come out in
// the same slot order as above.
template <int C>
__device__ __forceinline__ uint32_t lut_pair8(const uint32_t *lut, uint32_t v, int sh0, int sh1) {
  return perm(lut_at<C>(lut, (v >> sh1) & 0xFFu), lut_at<C>(lut, (v >> sh0) & 0xFFu),
              0x05040100u);
}

template <int C>
__device__ __forceinline__ u32x4 decode_q8(const uint32_t *w, const uint32_t *lut, int q) {
  const uint32_t w0 = w[2 * q], w1 = w[2 * q + 1];
  return u32x4{lut_pair8<C>(lut, w0, 0, 16), lut_pair8<C>(lut, w1, 0, 16),
               lut_pair8<C>(lut, w0, 8, 24), lut_pair8<C>(lut, w1, 8, 24)};
}

// 4 bits on both sides: one code byte holds slots 2k and 2k+1, and the
// table maps the byte straight to the fp16 pair [F(lo), F(hi)], so slots
// 8q .. 8q+7 (word w[q]) come out in natural order with four 32-bit reads
// and no byte permutes.
template <int C>
__device__ __forceinline__ u32x4 decode_pair4(const uint32_t *w, const uint32_t *lut, int q) {
  const uint32_t v = w[q];
  return u32x4{lut_at<C>(lut, v & 0xFFu), lut_at<C>(lut, (v >> 8) & 0xFFu),
               lut_at<C>(lut, (v >> 16) & 0xFFu), lut_at<C>(lut, v >> 24)};
}

// The same pair-table decode with the levels regrouped into the slot order
// of the byte-permute decoder (8q + {0,2,4,6,1,3,5,7}), for 4-bit
// activations against weights of another width: low halves of the pairs
// (even slots) first, then the high halves (odd slots).
template <int C>
__device__ __forceinline__ u32x4 decode_pair4_ilv(const uint32_t *w, const uint32_t *lut, int q) {
  const uint32_t v = w[q];
  const uint32_t p0 = lut_at<C>(lut, v & 0xFFu), p1 = lut_at<C>(lut, (v >> 8) & 0xFFu);
  const uint32_t p2 = lut_at<C>(lut, (v >> 16) & 0xFFu), p3 = lut_at<C>(lut, v >> 24);
  return u32x4{perm(p1, p0, 0x05040100u), perm(p3, p2, 0x05040100u),
               perm(p1, p0, 0x07060302u), perm(p3, p2, 0x07060302u)};
}

// The decode of one role: byte-permute tables (2-4 bits) or an LDS table
// (4 bits on both sides: pairs; 8 bits: levels).
struct Decoder {
  PermTab t;
  const uint32_t *lut;
};

template <int BITS, int PAIR, int C>
__device__ __forceinline__ u32x4 decode_chunk(const uint32_t *w, const Decoder &dc, int q) {
  if constexpr (BITS == 8) return decode_q8<C>(w, dc.lut, q);
  else if constexpr (PAIR == 2) return decode_pair4_ilv<C>(w, dc.lut, q);
  else if constexpr (PAIR == 1) return decode_pair4<C>(w, dc.lut, q);
  else return decode_q<BITS>(w, dc.t, q);
}

// Byte offset of (row, chunk) inside one operand tile of the LDS layout.
template <class TL>
__device__ __forceinline__ int chunk_off(int row, int chunk) { return chunk * TL::PLANE + row * 16; }

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t *p, uint32_t *w) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const u32x4 a = *(const u32x4 *)(p + 16 * v);
      w[4 * v] = a[0]; w[4 * v + 1] = a[1]; w[4 * v + 2] = a[2]; w[4 * v + 3] = a[3];
    }
  } else if constexpr (BITS == 4) {
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
template <class TL, int BITS, int PAIR>
__device__ __forceinline__ void k_loop(uint8_t *lds, floatx4 (&acc)[TL::JB][TL::IB],
                                       const uint8_t *prow, const Decoder &tt, int opoff, int row,
                                       int lane, int wm, int wn, int T) {
  constexpr int RB = 8 * BITS;           // code bytes of one K step
  constexpr int IB = TL::IB, JB = TL::JB;
  constexpr int IPC = IB / 4;            // activation blocks per chunk
  // 8 bits: one 64-byte code buffer, refilled 16 bytes at a time as soon as
  // a pair of chunks has been decoded from it (registers are too tight for
  // two), still about three quarters of a step ahead of use
  constexpr bool REFILL = BITS == 8;
  // 8 bits: the decode (eight table reads per chunk) runs one chunk ahead;
  // at 4+4 bits (four reads) that measured no better than decoding in place
  constexpr bool PIPE = BITS == 8;
  uint32_t cb0[2 * BITS], cb1[REFILL ? 1 : 2 * BITS];
  uint8_t *wbase = lds + opoff;
  load_codes<BITS>(prow, cb0);
#pragma unroll
  for (int q = 0; q < 8; q++)
    *(u32x4 *)(wbase + chunk_off<TL>(row, q)) = decode_chunk<BITS, PAIR, TL::LUTC>(cb0, tt, q);
  if (T > 1) load_codes<BITS>(prow + RB, REFILL ? cb0 : cb1);

  // fragment lanes: rows + (lane & 15), 8-slot chunk (lane >> 4) of each
  // 32-slot half.  The per-lane byte offsets are made opaque to the
  // compiler (an empty asm), so it cannot rewrite base + constant as a
  // bitwise or and every fragment and chunk offset below stays an
  // instruction immediate: a few address registers instead of one per
  // fragment.
  const int fr = lane & 15, ch0 = lane >> 4;
  uint32_t aoff = chunk_off<TL>(wm * (16 * IB) + fr, ch0);
  uint32_t boff = TL::OPB + chunk_off<TL>(wn * (16 * JB) + fr, ch0);
  uint32_t woff = opoff + row * 16;
  asm volatile("" : "+v"(aoff), "+v"(boff), "+v"(woff));
  constexpr int H1 = 4 * TL::PLANE;  // chunk ch0 + 4: the second 32-slot half

  // One K step: the MFMAs of step t (stage t&1); when `decode`, also the
  // decode of step t+1 (from `cur`) into stage (t+1)&1 and the load of
  // step t+2's codes into `nb`.
  auto step = [&](int t, uint32_t *cur, uint32_t *nb, bool decode) {
    __syncthreads();  // stage t&1 complete, stage (t+1)&1 no longer read
    const int n2 = (t + 2 < T) ? t + 2 : T - 1;  // past the end: a harmless re-read
    if (decode && !REFILL) load_codes<BITS>(prow + (int64_t)n2 * RB, nb);
    const uint8_t *stg = lds + (t & 1) * TL::STAGEB;
    const uint8_t *sA = stg + aoff, *sB = stg + boff;
    uint8_t *dst = lds + ((t + 1) & 1) * TL::STAGEB + woff;
    half8 af0[IB], bf0[JB], af1[IB], bf1[JB];
    // pipelined decodes: chunk c's lookups are issued in chunk c-1, so
    // eight MFMAs cover their latency before the store
    u32x4 pend = {0u, 0u, 0u, 0u};
    if (PIPE && decode) pend = decode_chunk<BITS, PAIR, TL::LUTC>(cur, tt, 0);
#pragma unroll
    for (int j = 0; j < JB; j++) bf0[j] = *(const half8 *)(sB + 256 * j);
#pragma unroll
    for (int u = 0; u < IPC; u++) af0[u] = *(const half8 *)(sA + 256 * u);
#pragma unroll
    for (int c = 0; c < 8; c++) {
      // chunk c: activation blocks IPC*(c&3) .. of K half c>>2 against all
      // weight blocks of that half; fragments are loaded one chunk ahead
      if (c < 3) {
#pragma unroll
        for (int u = 0; u < IPC; u++) {
          const int i = IPC * (c + 1) + u;
          af0[i] = *(const half8 *)(sA + 256 * i);
        }
      } else if (c == 3) {
#pragma unroll
        for (int j = 0; j < JB; j++) bf1[j] = *(const half8 *)(sB + H1 + 256 * j);
#pragma unroll
        for (int u = 0; u < IPC; u++) af1[u] = *(const half8 *)(sA + H1 + 256 * u);
      } else if (c < 7) {
#pragma unroll
        for (int u = 0; u < IPC; u++) {
          const int i = IPC * (c - 3) + u;
          af1[i] = *(const half8 *)(sA + H1 + 256 * i);
        }
      }
#pragma unroll
      for (int u = 0; u < IPC; u++) {
        const int i = IPC * (c & 3) + u;
#pragma unroll
        for (int j = 0; j < JB; j++) {
          if (c < 4)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf0[j], af0[i], acc[j][i], 0, 0, 0);
          else
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf1[j], af1[i], acc[j][i], 0, 0, 0);
        }
      }
      if (decode) {
        if constexpr (PIPE) {
          u32x4 nxt = pend;
          if (c < 7) nxt = decode_chunk<BITS, PAIR, TL::LUTC>(cur, tt, c + 1);
          *(u32x4 *)(dst + c * TL::PLANE) = pend;
          pend = nxt;
        } else {
          *(u32x4 *)(dst + c * TL::PLANE) = decode_chunk<BITS, PAIR, TL::LUTC>(cur, tt, c);
        }
      }
      if constexpr (REFILL) {
        if (decode && (c & 1)) {  // words 2c-2 .. 2c+1 are free: step t+2's bytes 8c-8 ..
          const u32x4 v = *(const u32x4 *)(prow + (int64_t)n2 * RB + 8 * (c - 1));
          cur[2 * c - 2] = v[0]; cur[2 * c - 1] = v[1]; cur[2 * c] = v[2]; cur[2 * c + 1] = v[3];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // steps in pairs so the two code buffers alternate without copies
  uint32_t *b0 = REFILL ? cb0 : cb1, *b1 = cb0;
  int t = 0;
  for (; t + 2 < T; t += 2) {
    step(t, b0, b1, true);
    step(t + 1, b1, b0, true);
  }
  if (t + 1 < T) {
    step(t, b0, b1, true);
    t++;
  }
  step(t, b0, b1, false);
}

// Group-major tile order: index g -> 256 x 256 tile (tm, tn), GROUP_M tile
// rows per group, column-major inside a group.
__host__ __device__ __forceinline__ void big_tile_of(int g, int nbm, int nbn, int &tm, int &tn) {
  const int gsz = GROUP_M * nbn, grp = g / gsz, first_m = grp * GROUP_M;
  const int gm = (nbm - first_m) < GROUP_M ? (nbm - first_m) : GROUP_M;
  tm = first_m + (g % gsz) % gm;
  tn = (g % gsz) / gm;
}

// One workgroup per output tile.  TL = BigTile: `count` tiles of the
// group-major order from index `first` (block ids spread so each XCD takes a
// contiguous run).  TL = SmallTile: each 256 x 256 tile from index `first`
// on is split into four 128 x 128 tiles, one workgroup each; with
// splits > 1 each of those is further cut into `splits` contiguous K ranges
// (piece v: sub-tile v mod 4 count, range v div 4 count), and a piece
// writes its raw fp32 accumulators, in fragment order, to part + 128^2 v
// instead of the epilogue (tail_reduce_kernel finishes the tile).
// lv8 (8 bits only): fp32 unit levels of the shared codebook.
template <class TL, int BA, int BW>
__global__ __launch_bounds__(TL::THREADS, TL::WGS) void linear_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ Wc,
    const float *__restrict__ sw, int M, int N, int K, uint16_t *__restrict__ Y, PermTab ta,
    PermTab tw, const float *__restrict__ lv8, int vec_store, int first, int count, int splits,
    float *__restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_base[];
  static_assert(BA != 8 || BW == 8, "8-bit codes on both sides");
  constexpr bool PAIR = BA == 4 && BW == 4;
  // 4-bit activations always decode through the pair table (with other
  // weight widths the weight rows keep the byte permutes)
  constexpr bool TAB_A = BA == 4;
  constexpr int LUTB = 256 * TL::LUTC * 4;                       // table bytes
  uint8_t *lds = lds_base + ((BA == 8 || TAB_A) ? LUTB : 0);  // decoded tiles
  constexpr int TT = TL::T, IB = TL::IB, JB = TL::JB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn_count = TT / (16 * JB);
  const int wm = wave / wn_count, wn = wave % wn_count;

  const int nbm = (M + BIG - 1) / BIG, nbn = (N + BIG - 1) / BIG;
  const bool is_a = __builtin_amdgcn_readfirstlane(tid) < TT;  // wave-uniform
  const int row = tid % TT;
  const int T = K / KS;

  Decoder da{ta, nullptr}, dw{tw, nullptr};
  if constexpr (BA == 8 || TAB_A) {
    // the shared table, TL::LUTC interleaved copies: 8 bits, the fp16 levels
    // (round to nearest even, as on the host); 4+4 bits, the fp16 pairs of
    // every code byte, from the byte-permute tables
    uint32_t *lut = (uint32_t *)lds_base;
    for (int i = tid; i < 256 * TL::LUTC; i += TL::THREADS) {
      const int b = i / TL::LUTC;
      uint32_t e;
      if constexpr (BA == 8) {
        e = __builtin_bit_cast(uint16_t, (_Float16)lv8[b]);
      } else {
        const int e0 = b & 15, e1 = b >> 4;
        const uint32_t f0 = ((ta.lo[e0 >> 2] >> (8 * (e0 & 3))) & 0xFFu) |
                            (((ta.hi[e0 >> 2] >> (8 * (e0 & 3))) & 0xFFu) << 8);
        const uint32_t f1 = ((ta.lo[e1 >> 2] >> (8 * (e1 & 3))) & 0xFFu) |
                            (((ta.hi[e1 >> 2] >> (8 * (e1 & 3))) & 0xFFu) << 8);
        e = f0 | (f1 << 16);
      }
      lut[i] = e;
    }
    __syncthreads();
    da.lut = lut + (lane & (TL::LUTC - 1));
    dw.lut = da.lut;
  }

  // ---- tiles: TL = BigTile is persistent (one workgroup per CU, each
  // walking its XCD's contiguous run of tiles, so a tile's output stores
  // drain while the next tile computes); TL = SmallTile takes one tile
  const int nv = (TT == BIG) ? count : 4 * count * splits;
  for (int v = blockIdx.x; v < nv; v += gridDim.x) {
    int m0, n0;
    int kb = 0, ke = T;  // K steps of this piece
    float *pdst = nullptr;
    if constexpr (TT == BIG) {
      const int xcd = v & 7, local = v >> 3, per = count >> 3, rem = count & 7;
      int tm, tn;
      big_tile_of(first + xcd * per + (xcd < rem ? xcd : rem) + local, nbm, nbn, tm, tn);
      m0 = tm * BIG;
      n0 = tn * BIG;
    } else {
      int tm, tn;
      const int nsub = 4 * count, u = v % nsub, s = v / nsub;
      big_tile_of(first + (u >> 2), nbm, nbn, tm, tn);
      const int sub = u & 3;
      m0 = tm * BIG + (sub >> 1) * TT;
      n0 = tn * BIG + (sub & 1) * TT;
      if (splits > 1) {
        kb = s * T / splits;
        ke = (s + 1) * T / splits;
        pdst = part + (int64_t)v * (TT * TT);
      }
    }

    // the row this thread decodes (rows past the edge repeat the last row)
    const int am = (m0 + row < M) ? m0 + row : M - 1;
    const int wr = (n0 + row < N) ? n0 + row : N - 1;
    const uint8_t *pa = A + (int64_t)am * ((int64_t)K * BA / 8) + kb * (8 * BA);
    const uint8_t *pw = Wc + (int64_t)wr * ((int64_t)K * BW / 8) + kb * (8 * BW);
    // this row's norm, loaded now and used after the K loop (latency hidden)
    const float nrm = pdst ? 0.f : (is_a ? sa[am] : sw[wr]);

    floatx4 acc[JB][IB];
#pragma unroll
    for (int j = 0; j < JB; j++)
#pragma unroll
      for (int i = 0; i < IB; i++) acc[j][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // the previous tile's last step may still read stage 0

    if constexpr (BA == BW) {
      k_loop<TL, BA, PAIR>(lds, acc, is_a ? pa : pw, is_a ? da : dw, is_a ? 0 : TL::OPB, row,
                           lane, wm, wn, ke - kb);
    } else {
      // both branches run the same barriers; the branch is wave-uniform
      if (is_a) k_loop<TL, BA, TAB_A ? 2 : 0>(lds, acc, pa, da, 0, row, lane, wm, wn, ke - kb);
      else k_loop<TL, BW, 0>(lds, acc, pw, dw, TL::OPB, row, lane, wm, wn, ke - kb);
    }

    if (pdst) {
      // K-range piece: raw accumulators, one 16-byte fragment per lane and
      // (wave, j, i), consecutive lanes adjacent (fully coalesced)
#pragma unroll
      for (int j = 0; j < JB; j++)
#pragma unroll
        for (int i = 0; i < IB; i++)
          *(floatx4 *)(pdst + 4 * (((wave * JB + j) * IB + i) * 64 + lane)) = acc[j][i];
      continue;  // uniform across the workgroup
    }

    // ---- epilogue.  The tile's norms go through LDS into registers
    // (activation rows, then weight rows, in the pipeline stage the last K
    // step left idle); bf16 rounding is the hardware's round to nearest
    // even.  Each wave stages its own (16 IB) x (16 JB) bf16 block in a
    // region of the (now idle) decoded-tile buffers -- rows of 32 JB bytes
    // (128: one cache line), 8-byte column chunks XOR-swizzled by an even
    // row mask so neither the fragment-shaped writes nor the row reads
    // conflict -- and writes it out as 16-byte row pieces: whole cache lines
    // instead of 16 rows x 32 bytes per store instruction, and no
    // workgroup barrier between staging and stores (measured 0.5-1% faster
    // at K = 3072, 6% at K = 128, than staging the whole tile).
    float *nl = (float *)(lds + ((ke - kb) & 1) * TL::STAGEB);
    nl[is_a ? row : TT + row] = nrm;
    __syncthreads();  // norms visible; every wave is past its last MFMA read of the tiles
    const float invk = 1.0f / (float)K;
    float sn[IB];
    floatx4 rn[JB];
#pragma unroll
    for (int i = 0; i < IB; i++) sn[i] = nl[wm * (16 * IB) + 16 * i + (lane & 15)] * invk;
#pragma unroll
    for (int j = 0; j < JB; j++)
      rn[j] = *(const floatx4 *)(nl + TT + wn * (16 * JB) + 16 * j + 4 * (lane >> 4));
    __syncthreads();  // every norm read before the staging regions overwrite them
    constexpr int WR = 16 * IB, WCB = 32 * JB, WCH = WCB / 8;  // rows, row bytes, chunks
    static_assert((TL::THREADS / 64) * WR * WCB <= 2 * TL::STAGEB, "regions fit the idle stages");
    uint8_t *reg = lds + wave * (WR * WCB);
    auto swz = [](int r) { return (2 * r) & (WCH - 2); };
#pragma unroll
    for (int i = 0; i < IB; i++) {
      const int rr = 16 * i + (lane & 15);
      const float s = sn[i];
#pragma unroll
      for (int j = 0; j < JB; j++) {
        const int ch = 4 * j + (lane >> 4);
        const floatx4 r = rn[j];
        const bf16x2 p0 = {(__bf16)(acc[j][i][0] * s * r[0]), (__bf16)(acc[j][i][1] * s * r[1])};
        const bf16x2 p1 = {(__bf16)(acc[j][i][2] * s * r[2]), (__bf16)(acc[j][i][3] * s * r[3])};
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *(u32x2 *)(reg + WCB * rr + 8 * (ch ^ swz(rr))) =
            u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
      }
    }
    // the row reads take values other lanes of this wave wrote: wait for
    // the wave's LDS writes (lgkmcnt(0)); no other wave touches the region
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    constexpr int PPR = WCB / 16, RPI = 64 / PPR;  // 16-byte pieces per row, rows per pass
    const int k = lane % PPR;
#pragma unroll 4
    for (int rr = lane / PPR; rr < WR; rr += RPI) {
      const int m = m0 + wm * WR + rr, n = n0 + wn * (16 * JB) + 8 * k;
      const u32x4 v = *(const u32x4 *)(reg + WCB * rr + 8 * ((2 * k) ^ swz(rr)));
      if (m >= M || n >= N) continue;
      uint16_t *yp = Y + (int64_t)m * N + n;
      if (vec_store && n + 7 < N) {
        // non-temporal: the output is not read again by this kernel, and
        // lines that stay dirty in the caches are written back later, in
        // whatever runs next (the following rotate+quantize at 32760 x 5120
        // measured 91.3 -> 88.4 us; this kernel equal or 0.3% faster)
        __builtin_nontemporal_store(v, (u32x4 *)yp);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
          if (n + e < N) yp[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// Finishes the tiles cut into K-range pieces: for every fragment of every
// 128 x 128 sub-tile, the sum of its `splits` partial accumulators (in
// range order), scaled and rounded exactly as the tile epilogue does, one
// 8-byte store of 4 bf16 outputs.  Requires N % 8 == 0 and a 16-byte
// aligned y (the launcher checks).
__global__ __launch_bounds__(256) void tail_reduce_kernel(
    const float *__restrict__ part, int splits, int count, int first, int M, int N, int K,
    const float *__restrict__ sa, const float *__restrict__ sw, uint16_t *__restrict__ Y) {
  using TL = SmallTile;
  constexpr int IB = TL::IB, JB = TL::JB, FR = TL::THREADS * TL::IB * TL::JB;  // per sub-tile
  const int nsub = 4 * count;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)nsub * FR) return;
  const int u = (int)(g / FR), f = (int)(g % FR);
  const int lane = f & 63, i = (f >> 6) % IB, j = (f >> 6) / IB % JB, wave = (f >> 6) / (IB * JB);
  const int wn_count = TL::T / (16 * JB), wm = wave / wn_count, wn = wave % wn_count;
  const int nbm = (M + BIG - 1) / BIG, nbn = (N + BIG - 1) / BIG;
  int tm, tn;
  big_tile_of(first + (u >> 2), nbm, nbn, tm, tn);
  const int m = tm * BIG + ((u & 3) >> 1) * TL::T + wm * (16 * IB) + 16 * i + (lane & 15);
  const int n = tn * BIG + (u & 1) * TL::T + wn * (16 * JB) + 16 * j + 4 * (lane >> 4);
  if (m >= M || n >= N) return;
  floatx4 acc = *(const floatx4 *)(part + 4 * (int64_t)g);
  for (int s = 1; s < splits; s++) acc += *(const floatx4 *)(part + 4 * ((int64_t)s * nsub * FR + g));
  const float sc = sa[m] * (1.0f / (float)K);
  const floatx4 r = {sw[n], sw[n + 1], sw[n + 2], sw[n + 3]};
  const bf16x2 p0 = {(__bf16)(acc[0] * sc * r[0]), (__bf16)(acc[1] * sc * r[1])};
  const bf16x2 p1 = {(__bf16)(acc[2] * sc * r[2]), (__bf16)(acc[3] * sc * r[3])};
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(
      u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)},
      (u32x2 *)(Y + (int64_t)m * N + n));  // output, as in the tile epilogue
}

PermTab make_tab(const LevelsF16 &lv) {
  PermTab t{};
  for (int e = 0; e < 16; e++) {
    t.lo[e >> 2] |= (uint32_t)(lv.v[e] & 0xFFu) << (8 * (e & 3));
    t.hi[e >> 2] |= (uint32_t)(lv.v[e] >> 8) << (8 * (e & 3));
  }
  return t;
}

template <class TL, int BA, int BW>
hipError_t launch_tiles(const LinearArgs &a, const PermTab &ta, const PermTab &tw,
                        const float *lv8, int vec, int first, int count, unsigned grid,
                        int splits = 1, float *part = nullptr) {
  constexpr int lds = TL::LDS + ((BA == 8 || BA == 4) ? 256 * TL::LUTC * 4 : 0);
  static_assert(lds * TL::WGS <= 160 * 1024, "LDS of one CU");
  static std::atomic<uint64_t> lds_set{0};  // per instantiation and device
  hipError_t e = ensure_lds_limit((const void *)linear_kernel<TL, BA, BW>, lds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((linear_kernel<TL, BA, BW>), dim3(grid), dim3(TL::THREADS), lds, a.stream,
                     a.a_codes, a.a_norms, a.w_codes, a.w_norms, (int)a.M, (int)a.N, a.K, a.y, ta,
                     tw, lv8, vec, first, count, splits, part);
  return hipGetLastError();
}

// Tiles of 256 x 256, one workgroup per CU at a time.  A problem too small
// to fill half of the CUs runs as 128 x 128 tiles instead (four times the
// workgroups, two per CU; 10-15% faster there than 256 x 256 tiles on part
// of the CUs).  A large problem whose last round would leave at most half
// of the CUs busy (R leftover tiles, each alone on its CU for a whole K
// loop) runs those R tiles first as 128 x 128 sub-tiles, each cut into
// S = 2 CUs / 4R K ranges (when that is 2 or more) so that every CU takes
// two pieces (two 128 x 128 workgroups share a CU); the pieces'
// fp32 partial sums go to rows of y that belong to the full rounds (they
// are overwritten later in stream order, so no extra memory is needed),
// tail_reduce_kernel sums them into the R tiles, and then the full rounds
// run as before.  Tails of more than half of the CUs stay whole 256 x 256
// tiles.
template <int BA, int BW>
hipError_t launch_ab(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw,
                     const float *lv8) {
  const PermTab ta = make_tab(la), tw = make_tab(lw);
  const int vec = (a.N % 8 == 0) && (((uintptr_t)a.y & 15) == 0);
  const int nbm = (int)((a.M + BIG - 1) / BIG), nbn = (int)((a.N + BIG - 1) / BIG);
  const int64_t tiles = (int64_t)nbm * nbn;
  if (tiles > (int64_t)(INT32_MAX / 4)) return hipErrorInvalidValue;
  int cus = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (cus <= 0) cus = 256;
  }
  if (4 * tiles <= SmallTile::WGS * cus)
    return launch_tiles<SmallTile, BA, BW>(a, ta, tw, lv8, vec, 0, (int)tiles,
                                           (unsigned)(4 * tiles));
  const int64_t rounds = tiles / cus, rem = tiles % cus;
  if (rounds == 0 || rem == 0 || 4 * rem > SmallTile::WGS * cus)
    // persistent: at most one workgroup per CU (a multiple of 8 keeps each
    // workgroup on one XCD's run of tiles)
    return launch_tiles<BigTile, BA, BW>(a, ta, tw, lv8, vec, 0, (int)tiles,
                                         (unsigned)(tiles < cus ? tiles : cus));

  const int first = (int)(rounds * cus), R = (int)rem, T = a.K / KS;
  int S = SmallTile::WGS * cus / (4 * R);  // pieces fill every CU's 128 x 128 slots
  if (S > T / 3) S = T / 3;  // at least three K steps per piece
  if (S > 1 && !vec) S = 1;
  if (S > 1) {
    // scratch: y rows above the highest leftover tile row, all full-round tiles
    int top = nbm;
    for (int g = first; g < (int)tiles; g++) {
      int tm, tn;
      big_tile_of(g, nbm, nbn, tm, tn);
      if (tm < top) top = tm;
    }
    const int64_t need = (int64_t)S * 4 * R * SmallTile::T * SmallTile::T * 4;
    if (need > (int64_t)top * BIG * a.N * 2) S = 1;
  }
  if (S < 1) S = 1;
  float *part = S > 1 ? (float *)a.y : nullptr;
  hipError_t e = launch_tiles<SmallTile, BA, BW>(a, ta, tw, lv8, vec, first, R,
                                                 (unsigned)(4 * R * S), S, part);
  if (e != hipSuccess) return e;
  if (S > 1) {
    const int64_t work = (int64_t)4 * R * SmallTile::THREADS * SmallTile::IB * SmallTile::JB;
    hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0,
                       a.stream, part, S, R, first, (int)a.M, (int)a.N, a.K, a.a_norms, a.w_norms,
                       a.y);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_tiles<BigTile, BA, BW>(a, ta, tw, lv8, vec, 0, first, (unsigned)cus);
}

}  // namespace

hipError_t launch_linear(const LinearArgs &a, const LevelsF16 &la, const LevelsF16 &lw,
                         const uint32_t *ta, const uint32_t *tw) {
  if (a.M > (int64_t)1 << 30 || a.N > (int64_t)1 << 30) return hipErrorInvalidValue;
  if (a.a_bits == 8 && a.w_bits == 8) {
    // one codebook for both operands: same K, bit width and family
    if (!ta || ta != tw) return hipErrorInvalidValue;
    return launch_ab<8, 8>(a, la, lw, (const float *)(ta + table_levels_word(8)));
  }
  // 4 bits on both sides: one pair table serves both operands
  if (a.a_bits == 4 && a.w_bits == 4 && std::memcmp(la.v, lw.v, sizeof(la.v)) != 0)
    return hipErrorInvalidValue;
#define OQ_CASE(x, y) \
  if (a.a_bits == x && a.w_bits == y) return launch_ab<x, y>(a, la, lw, nullptr);
  OQ_CASE(2, 2) OQ_CASE(2, 3) OQ_CASE(2, 4)
  OQ_CASE(3, 2) OQ_CASE(3, 3) OQ_CASE(3, 4)
  OQ_CASE(4, 2) OQ_CASE(4, 3) OQ_CASE(4, 4)
#undef OQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace oq
