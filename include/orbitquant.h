/*
 * orbitquant.h -- C ABI of liborbitquant.so, the MI355X (gfx950) library for
 * OrbitQuant's online quantized-linear path.
 *
 * The method (sources: the paper's abstract as reprinted on hotpaper.ai and
 * pith.science; paper.gecl.asia close-reading notes, section Method;
 * llmdb.app summary, section Mathematical Formulation; pith.science
 * Figure 2 caption and Supplementary A setup):
 *   - every activation token x (length d) keeps its L2 norm s = ||x|| apart
 *     and only its direction u = x / s is quantized;
 *   - u is rotated by RPBH: a seeded random permutation Pi, Rademacher signs
 *     D, then an orthonormal Walsh-Hadamard transform on each of the
 *     k = d / h blocks, h = the largest power of two dividing d;
 *   - each rotated coordinate is replaced by the nearest level of the
 *     Lloyd-Max codebook C_{d,b} for N(0, 1/d) (b = 2..4 bits, or 8: the
 *     pages' bit range runs from W2A4 up to W8A8, llmdb.app summary);
 *   - weights are prepared offline as the rows of W Pi^T, i.e. each row w_i
 *     goes through the same rotation and quantizer, with row norm r_i;
 *   - the linear is y[m][n] = s_m r_n sum_k C_{K,bw}[p_nk] C_{K,ba}[q_mk]
 *     (no bias; the rotation cancels inside the product).
 *
 * Conventions shared by every entry point
 *   - Return value: OQ_OK (0) or a negative OQ_E* status; oq_strerror()
 *     describes it.  Nothing throws across this boundary.
 *   - Arguments are validated on the host before any HIP call is made; a
 *     rejected call has no side effect.
 *   - Device pointers are caller-owned device memory (e.g. from PyTorch).
 *     The library never frees them.  Work is enqueued on `stream` (a
 *     hipStream_t passed as void*; NULL = the null stream) and is
 *     asynchronous: results are valid once the stream has reached them.
 *   - The library owns only its rotation-plan tables (a few tens of KB per
 *     (device, d, seed)) and codebook tables (decision grid, levels and
 *     thresholds: about 1 KB per (device, bits, family), 11 KB at 8 bits,
 *     per d for the sphere family); they live until oq_release_plans() or
 *     unload.
 *   - The rotation seed and flags of a layer's weights and of its
 *     activations must be the same; the library cannot check this.
 *   - Code layout ("storage order"): inside each whole group of 128
 *     consecutive rotated coordinates, coordinate 32c + p (c < 4, p < 32)
 *     is stored at slot 8 (p mod 16) + 4 (p div 16) + c; the coordinates
 *     of a last, partial group (d mod 128 = 32, 64 or 96 of them) are
 *     stored at their own index; slot t of a row holds the code
 *     in bits [b t, b t + b) of the row's bytes, little-endian bit order.
 *     A row of d codes therefore takes d*b/8 bytes.  Codes are level
 *     indices 0..2^b-1 in ascending level order.
 *     At 8 bits this is plain byte addressing: byte slot(i) holds code i.
 *   - Limits: d a multiple of 32, 32 <= d <= 16384 (so h = d & -d >= 32);
 *     the linear's K a multiple of 64 (whole 64-slot K steps); bits in
 *     {2, 3, 4, 8} (1..8 for oq_codebook; the exact-sphere family 1..4 and 8).
 *     Zero rows are valid (a zero token gets norm 0 and every code
 *     2^(b-1)).  NaN/Inf inputs give unspecified codes and no error.
 */
#ifndef ORBITQUANT_H
#define ORBITQUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define OQ_OK 0
#define OQ_EINVAL (-1)        /* bad argument (null/misaligned pointer, negative size, ...) */
#define OQ_EUNSUPPORTED (-2)  /* valid but not supported (d, bits, bit pair) */
#define OQ_ENOMEM (-3)        /* the library could not allocate its plan tables */
#define OQ_EDEVICE (-4)       /* a HIP call or kernel launch failed */

/* input element types */
#define OQ_F32 0   /* IEEE fp32 */
#define OQ_BF16 1  /* bfloat16, 16-bit patterns */

/* flags */
#define OQ_ROT_NO_SIGNS (1u << 0)     /* rotation without the Rademacher signs D (Pi then H only) */
#define OQ_OUT_F32_ROTATED (1u << 1)  /* oq_rotate_quantize writes the rotated unit vector z
                                         (fp32 [n_tok][d], coordinate order) instead of codes */
#define OQ_OUT_BF16_DEQUANT (1u << 2) /* oq_rotate_quantize writes the dequantized rotated token
                                         s * c_{code_i} (bf16 [n_tok][d], coordinate order, round
                                         to nearest even) instead of codes: fake quantization */
#define OQ_CODEBOOK_SPHERE (1u << 4)  /* Lloyd-Max for the exact marginal of one coordinate of
                                         a uniform point on S^{d-1} instead of its Gaussian limit
                                         N(0, 1/d); activations, weights and oq_linear_ex must
                                         all use the same family */
#define OQ_ROT_INPUT_PERMUTED (1u << 3) /* the input rows are already in rotation order,
                                           x'_i = x_{pi(i)} (see oq_permute_rows); only D and
                                           H are applied.  Same outputs as the unpermuted rows
                                           without this flag */

/* Text for a status code.  Never NULL; the string is static. */
const char *oq_strerror(int status);

/* Library ABI version (major * 100 + minor). */
int oq_version(void);

/* Lloyd-Max codebook C_{d,bits} for the dimension marginal N(0, 1/d)
 * (paper.gecl.asia notes, Core Idea and Method item 3; pith.science
 * Figure 2 caption).  Host only, synchronous.
 *   levels:     caller buffer of 2^bits floats, ascending, sigma = 1/sqrt(d)
 *   thresholds: caller buffer of 2^bits - 1 floats, the midpoints of
 *               adjacent levels (decision boundaries)
 * bits in 1..8, d >= 1.  Errors: OQ_EINVAL (null buffer, d < 1),
 * OQ_EUNSUPPORTED (bits).  The solver is Max's shooting method; at 8 bits
 * its levels lie within about 1e-9 (unit scale) of the fixed point. */
int oq_codebook(int d, int bits, float *levels, float *thresholds);

/* oq_codebook with a codebook family (flags 0 or OQ_CODEBOOK_SPHERE).  The
 * sphere family is the Lloyd-Max quantizer of the density
 * c_d (1 - t^2)^((d-3)/2) of one coordinate of a uniform point on S^{d-1}
 * (pith.science: the referee's minor comment 1 asks for this closed-form
 * marginal), defined for the dimensions the kernels take (d % 32 == 0,
 * d <= 16384) and bits 1..4 and 8 (else OQ_EUNSUPPORTED).  It differs from
 * the Gaussian one by 0.8% of a level at d = 256 and 0.015% at d = 13824
 * (4 bits).  Up to 4 bits the solver is Max's shooting method; at 8 bits
 * Newton's method on the Lloyd-Max conditions from the Gaussian codebook
 * (the conditions fix the 8-bit levels to about 1e-7 of the unit scale in
 * double precision). */
int oq_codebook_ex(int d, int bits, uint32_t flags, float *levels, float *thresholds);

/* Bytes of a packed code matrix: rows * d * bits / 8 (-1 on bad input). */
int64_t oq_codes_bytes(int64_t rows, int d, int bits);

/* Online activation path (paper.gecl.asia notes, Method items 1 and 4;
 * pith.science Supplementary A setup; llmdb.app Implementation Details):
 * for each of the n_tok rows of x, s = ||x||_2, z = RPBH(x / s), and each
 * coordinate of z is quantized to the nearest level of C_{d,bits} (ties to
 * the upper level).
 *   x:      device, [n_tok][d] row-major, dtype OQ_F32 or OQ_BF16, 16-byte
 *           aligned
 *   seed:   rotation seed (selects Pi and D)
 *   flags:  OQ_ROT_NO_SIGNS, OQ_ROT_INPUT_PERMUTED, OQ_CODEBOOK_SPHERE, and at
 *           most one of OQ_OUT_F32_ROTATED, OQ_OUT_BF16_DEQUANT
 *   out:    device; packed codes uint8 [n_tok][d*bits/8] (storage order,
 *           16-byte aligned), or with OQ_OUT_F32_ROTATED fp32 [n_tok][d], or
 *           with OQ_OUT_BF16_DEQUANT bf16 [n_tok][d]: coordinate i holds
 *           s * C_{d,bits}[code_i], the token's reconstruction in the rotated
 *           basis.  A bf16 GEMM of two such matrices (activations and weight
 *           rows, same seed) is the fake-quantized product the pages evaluate
 *           (paper.gecl.asia notes, Dataset/Evaluation; llmdb.app
 *           Implementation Details), equal to oq_linear up to operand rounding
 *   norms:  device fp32 [n_tok], receives s (4-byte aligned)
 * n_tok = 0 is a no-op that succeeds (the pointers may then be NULL).
 * Errors: OQ_EINVAL, OQ_EUNSUPPORTED, OQ_ENOMEM, OQ_EDEVICE. */
int oq_rotate_quantize(const void *x, int dtype, int64_t n_tok, int d, uint64_t seed,
                       uint32_t flags, int bits, void *out, float *norms, void *stream);

/* Offline weight preparation (hotpaper.ai abstract: the same quantizer on
 * the weight rows, rotation absorbed into the weights; paper.gecl.asia
 * notes, Method item 2: W Pi^T): row i of W [n_out][d_in] becomes the
 * packed codes of RPBH(w_i / r_i) under C_{d_in,bits} plus r_i = ||w_i||.
 * Same layout, limits and errors as oq_rotate_quantize (w_codes
 * [n_out][d_in*bits/8], row_norms [n_out]); OQ_OUT_F32_ROTATED and
 * OQ_OUT_BF16_DEQUANT are rejected here (oq_rotate_quantize on the weight
 * rows gives the same outputs). */
int oq_prepare_weights(const void *W, int dtype, int64_t n_out, int d_in, uint64_t seed,
                       uint32_t flags, int bits, uint8_t *w_codes, float *row_norms,
                       void *stream);

/* Low-bit linear (llmdb.app Mathematical Formulation, y = Q_w(W R^-1)
 * Q_a(R x), no bias):
 *   y[m][n] = bf16( s_m r_n sum_k C_{K,w_bits}[p_nk] C_{K,a_bits}[q_mk] )
 * with both code matrices in storage order (the sum runs over the same
 * permuted coordinates on both sides).  Accumulation is fp32 over fp16
 * copies of the unit-variance levels; the output is rounded once to bf16
 * (round to nearest even).
 *   a_codes [M][K*a_bits/8], a_norms [M], w_codes [N][K*w_bits/8],
 *   w_norms [N]: device, as produced by oq_rotate_quantize /
 *   oq_prepare_weights with the same seed, flags and K
 *   y: device bf16 bit patterns, [M][N] row-major, 2-byte aligned; a y
 *      that shares a byte with any of the four inputs is rejected
 *      (OQ_EINVAL).  Until the call completes on the stream, y
 *      may hold intermediate values (a sparse last round of output tiles
 *      parks fp32 partial sums in y's first rows, which are then
 *      overwritten), so nothing may read it concurrently.
 * a_bits, w_bits in {2, 3, 4}, any pair, or both 8 (W8A8: the codes are
 * decoded through an fp16 table of the 256 levels; a pair with only one
 * side at 8 bits is OQ_EUNSUPPORTED).  K % 64 == 0, K <= 16384 (a K with a
 * last partial group of 32 or 96 coordinates is OQ_EUNSUPPORTED here, though
 * such rows can be rotated and prepared).  M and N up to 2^30
 * (OQ_EUNSUPPORTED beyond).  M = 0 or N = 0 is a no-op that succeeds (the pointers may then
 * be NULL).  Errors:
 * OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE. */
int oq_linear(const uint8_t *a_codes, const float *a_norms, int a_bits,
              const uint8_t *w_codes, const float *w_norms, int w_bits,
              int64_t M, int64_t N, int K, uint16_t *y, void *stream);

/* oq_linear with a codebook family for both operands (flags 0 or
 * OQ_CODEBOOK_SPHERE; the codes must come from rotate/prepare calls with
 * the same family).  Same layout, limits and errors; flags outside the
 * family bit give OQ_EINVAL.  W8A8 takes either family. */
int oq_linear_ex(const uint8_t *a_codes, const float *a_norms, int a_bits,
                 const uint8_t *w_codes, const float *w_norms, int w_bits,
                 int64_t M, int64_t N, int K, uint32_t flags, uint16_t *y, void *stream);

/* Free every cached rotation plan and codebook table on every device (the
 * caller must ensure that no enqueued work still uses them, e.g. by
 * synchronising first, and that no other thread is inside a library call
 * meanwhile).  Handles from oq_plan_create stay valid to destroy
 * but name no tables any more. */
int oq_release_plans(void);

/* INT4 weight-only round-to-nearest for the AdaLN modulation projections
 * (paper.gecl.asia notes, Method item 5: a rotation cannot be folded into a
 * dynamic modulation, so those weights get INT4 RTN and the activations
 * stay unquantized; researchpod.app transcript).  Per output row n:
 * amax = max_k |W_nk|, scale_n = amax / 7, q_nk = rint(W_nk * (7 / amax)) in
 * [-7, 7], the decisions taken in fp32 (IEEE division and product, ties to
 * even); a zero row gives q = 0, scale 0.
 *   W:      device, fp32 or bf16 [n_out][d_in] (4-byte aligned)
 *   q4:     device uint8 [n_out][d_in/2] (16-byte aligned): nibble q + 8,
 *           coordinate 2i in the low nibble of byte i
 *   scales: device fp32 [n_out]
 *   d_in % 32 == 0, d_in <= 16384 (else OQ_EUNSUPPORTED); n_out = 0 no-op.
 * Errors: OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE. */
int oq_rtn4_prepare_weights(const void *W, int dtype, int64_t n_out, int d_in, uint8_t *q4,
                            float *scales, void *stream);

/* The AdaLN projection with those weights:
 *   y[m][n] = bf16( scale_n sum_k x_mk q_nk )
 * fp32 accumulation (exact products), one bf16 rounding (nearest even), no
 * bias.  x: device fp32 or bf16 [M][K] (16-byte aligned); y: bf16 [M][N].
 * Sized for modulation inputs (one row per sample): weights are read once
 * per block of 8 rows.  K % 32 == 0, K <= 16384; M = 0 or N = 0 no-op.
 * Errors: OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE. */
int oq_rtn4_linear(const void *x, int dtype, int64_t M, const uint8_t *q4, const float *scales,
                   int64_t N, int K, uint16_t *y, void *stream);

/* Permute rows by the rotation permutation pi of (d = rows, seed):
 * dst row i = src row pi(i), rows of row_bytes bytes each (any dtype).
 * Folds pi into a producer: permuting the output rows of the layer that
 * feeds the activations (and its bias), with an elementwise function such
 * as GELU between, makes the activations arrive in rotation order, and
 * oq_rotate_quantize with OQ_ROT_INPUT_PERMUTED then skips the permutation
 * (paper.gecl.asia notes, Limitations: rotation and norm cost at run time).
 * The signs D cannot be folded through a nonlinearity and stay in the call.
 *   src, dst: device, caller-owned, distinct (no in-place), [rows][row_bytes]
 *   rows:     the permutation length d: 32 <= d <= 16384, d % 32 == 0
 *   row_bytes >= 1
 * rows = 0 is rejected (there is no plan of length 0).
 * Errors: OQ_EINVAL (null or equal pointers, row_bytes < 1), OQ_EUNSUPPORTED
 * (rows), OQ_ENOMEM, OQ_EDEVICE. */
int oq_permute_rows(const void *src, void *dst, int64_t rows, int64_t row_bytes, uint64_t seed,
                    void *stream);

/* Optional explicit plan ownership.  The compute calls build the rotation
 * plan of (current device, d, seed) -- the permutation Pi and the signs D
 * (pith.science Supplementary A setup) as device tables -- on first use and
 * cache it.  oq_plan_create builds it now (no first-call latency) and pins
 * it; oq_plan_destroy drops the pin and frees the tables when no other
 * handle pins them (the caller must ensure that no enqueued work still
 * uses them and that no other thread's call on the same (d, seed) is in
 * progress).  A later compute call with the same (d, seed) rebuilds the plan.
 *   d:     32 <= d <= 16384, d % 32 == 0   (else OQ_EUNSUPPORTED)
 *   flags: 0 or OQ_ROT_NO_SIGNS (one plan serves both sign modes)
 *   plan:  receives an opaque handle (NULL on error)
 * Errors: OQ_EINVAL (null out pointer, bad flags, d <= 0, or a handle not
 * made by oq_plan_create), OQ_EUNSUPPORTED, OQ_ENOMEM, OQ_EDEVICE. */
int oq_plan_create(int d, uint64_t seed, uint32_t flags, void **plan);
int oq_plan_destroy(void *plan);

#ifdef __cplusplus
}
#endif
#endif /* ORBITQUANT_H */
