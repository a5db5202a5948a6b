/*
 * oq_oracle.c -- plain fp64 CPU oracle for the OrbitQuant online
 * quantized-linear path.  TEST INFRASTRUCTURE ONLY: the test-suite, the
 * smoke check and the benchmark's CPU-baseline leg are the only callers.
 * The product library never links, loads or calls this file, and this file
 * shares no code, header, table or constant generator with it.
 *
 * Every step is written the slow, obvious way, in double precision, in the
 * order the method states it.  Sources (page title; section / figure):
 *
 *  - "OrbitQuant: Data-Agnostic Quantization for Image and Video Diffusion
 *    Transformers" (paper.gecl.asia close-reading notes), section Method,
 *    items 1-4: keep the per-token L2 norm, quantize only the unit
 *    direction; fold the rotation into the weight rows (W Pi^T) and apply
 *    Pi x online; Lloyd-Max codebook on the dimension marginal
 *    f_d ~ N(0, 1/d); RPBH = random permutation then block Hadamard.
 *  - hotpaper.ai page, abstract: the same quantizer is applied to the weight
 *    rows offline.
 *  - pith.science page, Figure 2 caption: f_d ~ N(0,1/d) and one codebook
 *    C_{d,b} per dimension and bit width; Supplementary A (proof-sketch
 *    setup): d = k h, y = P_pi x, z^(j) = H_h D_j y^(j), (H_h)_{li} =
 *    +-1/sqrt(h), D_j Rademacher.
 *  - llmdb.app page, section Mathematical Formulation: y_hat =
 *    Q_w(W R^-1) Q_a(R x), no bias.
 *
 * Readings where the pages are silent (each one is listed with its reason
 * in the design notes):
 *  - RNG: SplitMix64 (Vigna's published reference generator).  Pi is a
 *    Durstenfeld shuffle driven by it, j = floor(r * (i+1) / 2^64); the d
 *    Rademacher signs are drawn next from the same stream, sign = top bit.
 *  - Hadamard in Sylvester natural order, H[a][b] = (-1)^popcount(a & b).
 *  - Gather convention y_i = s_i * u_{pi(i)}.
 *  - Ties go to the upper level: code = #{k : z >= tau_k}; -0 counts as 0.
 *  - Codes are stored in a tile-interleaved slot order inside every whole
 *    group of 128 coordinates (a last, partial group of 32, 64 or 96 in
 *    coordinate order), then packed as a little-endian bitstream.
 *  - Parity pins for each function are in the oracle test files.  The
 *    permutation itself has no value printed on any page: it is pinned only
 *    through the SplitMix64 published outputs and the bijection property.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oq_oracle.h"

/* ------------------------------------------------------------------ RNG -- */

/* SplitMix64: state advances by the golden-ratio gamma, output is the
 * state passed through two xor-shift-multiply rounds and a final xor-shift
 * (Vigna's public-domain splitmix64.c). */
uint64_t oqo_splitmix64_next(uint64_t *state)
{
    uint64_t z;
    *state += 0x9E3779B97F4A7C15ULL;
    z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* ----------------------------------------------------------- plan (Pi, D) -- */

int oqo_block_size(int d)
{
    /* largest power of two that divides d */
    int h = 1;
    while (d % (2 * h) == 0) h *= 2;
    return h;
}

/* Random permutation Pi (Durstenfeld shuffle) and Rademacher signs D, both
 * drawn from one SplitMix64 stream seeded with `seed`. */
void oqo_plan(int d, uint64_t seed, int32_t *perm, int8_t *sign)
{
    uint64_t state = seed;
    for (int i = 0; i < d; i++) perm[i] = i;
    for (int i = d - 1; i >= 1; i--) {
        uint64_t r = oqo_splitmix64_next(&state);
        /* j = floor(r * (i+1) / 2^64), the high word of a 128-bit product */
        unsigned __int128 prod = (unsigned __int128)r * (unsigned __int128)(uint64_t)(i + 1);
        int j = (int)(uint64_t)(prod >> 64);
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    for (int i = 0; i < d; i++) {
        uint64_t r = oqo_splitmix64_next(&state);
        sign[i] = (r >> 63) ? -1 : +1;
    }
}

/* ------------------------------------------------------------- codebook -- */

static double std_pdf(double t)
{
    if (isinf(t)) return 0.0;
    return exp(-0.5 * t * t) / sqrt(2.0 * M_PI);
}

/* P(a <= X < b) for X ~ N(0,1), written with erfc on the side where it does
 * not cancel. */
static double std_mass(double a, double b)
{
    if (a >= 0.0) /* both in the upper half: Q(a) - Q(b) */
        return 0.5 * erfc(a / sqrt(2.0)) - 0.5 * erfc(b / sqrt(2.0));
    if (b <= 0.0) /* both in the lower half: Phi(b) - Phi(a) */
        return 0.5 * erfc(-b / sqrt(2.0)) - 0.5 * erfc(-a / sqrt(2.0));
    return 1.0 - 0.5 * erfc(-a / sqrt(2.0)) - 0.5 * erfc(b / sqrt(2.0));
}

/* Lloyd-Max quantizer for N(0,1) with L = 2^bits levels (Lloyd 1982; Max
 * 1960), by Lloyd's alternation: thresholds are the midpoints of adjacent
 * levels, and each level is the conditional mean of its cell,
 *     c_k = (pdf(t_k) - pdf(t_{k+1})) / P(t_k <= X < t_{k+1}).
 * Stops when no level moves by more than 1e-15 (or after max_iter).
 * From 5 bits on the alternation converges too slowly to reach that (its
 * slowest mode contracts by about 1 - O(1/L^2) per sweep), so a short
 * alternation is followed by Newton's method on the same two conditions
 * (lloyd_max_newton).  Writes L unit-variance levels and L-1 thresholds;
 * returns iterations. */
static int lloyd_max_newton(int L, double *levels);

/* Both densities (N(0,1) and the sphere marginal) are even, so their
 * Lloyd-Max quantizers are symmetric, c_{L-1-k} = -c_k, with the middle
 * threshold at 0.  Newton's method on the conditions (5-8 bits) breaks
 * that only by rounding (about 1e-13); this restores it, so a zero token
 * takes code L/2 whatever the bit width. */
static void symmetrize(int L, double *c)
{
    for (int k = 0; k < L / 2; k++) {
        const double m = 0.5 * (c[L - 1 - k] - c[k]);
        c[k] = -m;
        c[L - 1 - k] = m;
    }
}

int oqo_codebook_unit(int bits, double *levels, double *thresholds)
{
    const int L = 1 << bits;
    double t[256 + 1];
    int it;
    if (bits < 1 || bits > 8) return -1;
    for (int k = 0; k < L; k++) /* evenly spread start inside (-2, 2) */
        levels[k] = -2.0 + 4.0 * (k + 0.5) / L;
    const int max_iter = bits <= 4 ? 200000 : 2000;
    for (it = 1; it <= max_iter; it++) {
        double move = 0.0;
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int k = 1; k < L; k++) t[k] = 0.5 * (levels[k - 1] + levels[k]);
        for (int k = 0; k < L; k++) {
            double c = (std_pdf(t[k]) - std_pdf(t[k + 1])) / std_mass(t[k], t[k + 1]);
            double dm = fabs(c - levels[k]);
            if (dm > move) move = dm;
            levels[k] = c;
        }
        if (move < 1e-15) break;
    }
    if (bits > 4) it += lloyd_max_newton(L, levels);
    symmetrize(L, levels);
    for (int k = 1; k < L; k++) thresholds[k - 1] = 0.5 * (levels[k - 1] + levels[k]);
    return it;
}

/* Newton's method on the Lloyd-Max conditions F_k(c) = c_k - mu(t_k, t_{k+1})
 * = 0, t_k = (c_{k-1} + c_k) / 2, with mu(a, b) the mean of N(0,1) on
 * [a, b).  Its partial derivatives are
 *     d mu / d a = pdf(a) (mu - a) / m,   d mu / d b = pdf(b) (b - mu) / m
 * (m the cell mass), so the Jacobian is tridiagonal and each step is one
 * Thomas-algorithm solve.  Converges quadratically until the steps reach
 * the rounding noise of F (amplified by the Jacobian's small eigenvalue,
 * about 1e-12 at 8 bits); stops there: after a step below 1e-14, or once a
 * step no longer shrinks to under half the previous one.  Returns the
 * number of steps. */
static int lloyd_max_newton(int L, double *c)
{
    double t[256 + 1], lo[256], di[256], up[256], rhs[256];
    double prev = INFINITY;
    int it;
    for (it = 1; it <= 100; it++) {
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int k = 1; k < L; k++) t[k] = 0.5 * (c[k - 1] + c[k]);
        for (int k = 0; k < L; k++) {
            const double a = t[k], b = t[k + 1];
            const double m = std_mass(a, b);
            const double mu = (std_pdf(a) - std_pdf(b)) / m;
            const double da = isinf(a) ? 0.0 : std_pdf(a) * (mu - a) / m;
            const double db = isinf(b) ? 0.0 : std_pdf(b) * (b - mu) / m;
            lo[k] = -0.5 * da;
            up[k] = -0.5 * db;
            di[k] = 1.0 - 0.5 * da - 0.5 * db;
            rhs[k] = -(c[k] - mu);
        }
        /* Thomas algorithm: forward elimination, back substitution */
        for (int k = 1; k < L; k++) {
            const double f = lo[k] / di[k - 1];
            di[k] -= f * up[k - 1];
            rhs[k] -= f * rhs[k - 1];
        }
        rhs[L - 1] /= di[L - 1];
        for (int k = L - 2; k >= 0; k--) rhs[k] = (rhs[k] - up[k] * rhs[k + 1]) / di[k];
        double move = 0.0;
        for (int k = 0; k < L; k++) {
            c[k] += rhs[k];
            if (fabs(rhs[k]) > move) move = fabs(rhs[k]);
        }
        if (move < 1e-14 || (it >= 3 && move > 0.5 * prev)) break;
        prev = move;
    }
    return it;
}

/* The codebook C_{d,b} for the dimension marginal N(0, 1/d): the unit
 * codebook scaled by sigma = 1/sqrt(d). */
int oqo_codebook(int d, int bits, double *levels, double *thresholds)
{
    const int L = 1 << bits;
    const double sigma = 1.0 / sqrt((double)d);
    int it = oqo_codebook_unit(bits, levels, thresholds);
    for (int k = 0; k < L; k++) levels[k] *= sigma;
    for (int k = 0; k < L - 1; k++) thresholds[k] *= sigma;
    return it;
}

/* Mean squared error of the unit quantizer, E[(X - Q(X))^2], by the closed
 * form  sum_k [ m_k (1 + c_k^2) - 2 c_k (pdf(a)-pdf(b)) + (a pdf(a) - b pdf(b)) ]
 * where m_k is the cell mass. */
double oqo_codebook_mse(int bits, const double *levels, const double *thresholds)
{
    const int L = 1 << bits;
    double s = 0.0;
    for (int k = 0; k < L; k++) {
        double a = (k == 0) ? -INFINITY : thresholds[k - 1];
        double b = (k == L - 1) ? INFINITY : thresholds[k];
        double m = std_mass(a, b);
        double pa = std_pdf(a), pb = std_pdf(b);
        double apa = isinf(a) ? 0.0 : a * pa;
        double bpb = isinf(b) ? 0.0 : b * pb;
        /* E[X^2 1_cell] = m + a pdf(a) - b pdf(b);  E[X 1_cell] = pdf(a) - pdf(b) */
        s += (m + apa - bpb) - 2.0 * levels[k] * (pa - pb) + levels[k] * levels[k] * m;
    }
    return s;
}

/* ------------------------------------------- exact sphere marginal -- */

/* Regularized incomplete beta I_x(a, b) by its continued fraction
 * (DLMF 8.17.22), evaluated with the modified Lentz method, on the side of
 * the symmetry I_x(a,b) = 1 - I_{1-x}(b,a) where it converges quickly.
 * `upper` asks for 1 - I_x(a,b) without cancellation. */
static double betacf(double a, double b, double x)
{
    const double tiny = 1e-300;
    double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
    if (fabs(dd) < tiny) dd = tiny;
    dd = 1.0 / dd;
    double h = dd;
    for (int m = 1; m <= 100000; m++) {
        double num = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
        dd = 1.0 + num * dd; if (fabs(dd) < tiny) dd = tiny;
        c = 1.0 + num / c;   if (fabs(c) < tiny) c = tiny;
        dd = 1.0 / dd; h *= dd * c;
        num = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
        dd = 1.0 + num * dd; if (fabs(dd) < tiny) dd = tiny;
        c = 1.0 + num / c;   if (fabs(c) < tiny) c = tiny;
        dd = 1.0 / dd;
        const double del = dd * c;
        h *= del;
        if (fabs(del - 1.0) < 1e-16) break;
    }
    return h;
}

static double ibeta(double a, double b, double x, int upper)
{
    if (x <= 0.0) return upper ? 1.0 : 0.0;
    if (x >= 1.0) return upper ? 0.0 : 1.0;
    const double lfront = lgamma(a + b) - lgamma(a) - lgamma(b) + a * log(x) + b * log1p(-x);
    if (x < (a + 1.0) / (a + b + 2.0)) {
        const double v = exp(lfront) * betacf(a, b, x) / a;
        return upper ? 1.0 - v : v;
    }
    const double w = exp(lfront) * betacf(b, a, 1.0 - x) / b; /* = 1 - I_x(a,b) */
    return upper ? w : 1.0 - w;
}

/* Mass of [a, b] under the marginal of one coordinate T of a uniform point
 * on the unit sphere S^{d-1}: T^2 ~ Beta(1/2, (d-1)/2), symmetric about 0.
 * Tail masses use the upper incomplete beta (no cancellation). */
static double sphere_tail(double t, int d) /* P(T >= t) for t >= 0 */
{
    return 0.5 * ibeta(0.5, 0.5 * (d - 1), t * t, 1);
}

static double sphere_mass(double a, double b, int d)
{
    if (a >= 0.0) return sphere_tail(a, d) - sphere_tail(b, d);
    if (b <= 0.0) return sphere_tail(-b, d) - sphere_tail(-a, d);
    return 1.0 - sphere_tail(-a, d) - sphere_tail(b, d);
}

/* E[T 1{a <= T < b}] in closed form: the density is
 * c_d (1 - t^2)^((d-3)/2), c_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)), and
 * t (1 - t^2)^((d-3)/2) integrates to -(1 - t^2)^((d-1)/2) / (d - 1). */
static double sphere_moment(double a, double b, int d)
{
    const double lc = lgamma(0.5 * d) - 0.5 * log(M_PI) - lgamma(0.5 * (d - 1));
    const double pa = (a <= -1.0 || a >= 1.0) ? 0.0 : exp(0.5 * (d - 1) * log1p(-a * a));
    const double pb = (b <= -1.0 || b >= 1.0) ? 0.0 : exp(0.5 * (d - 1) * log1p(-b * b));
    return exp(lc) * (pa - pb) / (d - 1);
}

/* Density of T: c_d (1 - t^2)^((d-3)/2) on (-1, 1). */
static double sphere_pdf(double t, int d)
{
    if (t <= -1.0 || t >= 1.0) return 0.0;
    const double lc = lgamma(0.5 * d) - 0.5 * log(M_PI) - lgamma(0.5 * (d - 1));
    return exp(lc + 0.5 * (d - 3) * log1p(-t * t));
}

/* Newton's method on the Lloyd-Max conditions for the sphere marginal: the
 * same conditions, Jacobian and stopping rule as lloyd_max_newton (there
 * for N(0,1)), with f_d's density, cell masses and first moments, the
 * outer cells ending at -1 and 1 (fixed ends: no derivative), and steps
 * measured in units of sigma = 1/sqrt(d).  Returns the number of steps. */
static int sphere_newton(int d, int L, double *c)
{
    double t[256 + 1], lo[256], di[256], up[256], rhs[256];
    const double unit = sqrt((double)d);
    double prev = INFINITY;
    int it;
    for (it = 1; it <= 100; it++) {
        t[0] = -1.0;
        t[L] = 1.0;
        for (int k = 1; k < L; k++) t[k] = 0.5 * (c[k - 1] + c[k]);
        for (int k = 0; k < L; k++) {
            const double a = t[k], b = t[k + 1];
            const double m = sphere_mass(a, b, d);
            const double mu = sphere_moment(a, b, d) / m;
            const double da = (k == 0) ? 0.0 : sphere_pdf(a, d) * (mu - a) / m;
            const double db = (k == L - 1) ? 0.0 : sphere_pdf(b, d) * (b - mu) / m;
            lo[k] = -0.5 * da;
            up[k] = -0.5 * db;
            di[k] = 1.0 - 0.5 * da - 0.5 * db;
            rhs[k] = -(c[k] - mu);
        }
        for (int k = 1; k < L; k++) {
            const double f = lo[k] / di[k - 1];
            di[k] -= f * up[k - 1];
            rhs[k] -= f * rhs[k - 1];
        }
        rhs[L - 1] /= di[L - 1];
        for (int k = L - 2; k >= 0; k--) rhs[k] = (rhs[k] - up[k] * rhs[k + 1]) / di[k];
        double move = 0.0;
        for (int k = 0; k < L; k++) {
            c[k] += rhs[k];
            if (fabs(rhs[k]) * unit > move) move = fabs(rhs[k]) * unit;
        }
        if (move < 1e-14 || (it >= 3 && move > 0.5 * prev)) break;
        prev = move;
    }
    return it;
}

/* Lloyd-Max quantizer for the exact marginal of one coordinate of a uniform
 * point on S^{d-1} (pith.science: the referee's minor comment 1 asks for
 * this closed-form marginal; the Figure 2 caption uses its Gaussian limit
 * N(0, 1/d)): Lloyd's alternation as for the Gaussian, with the cell masses
 * and first moments of f_d, started from the Gaussian codebook scaled by
 * sigma; from 5 bits on (8 bits: the top of the llmdb.app bit range) a
 * short alternation is followed by Newton's method (sphere_newton), as for
 * the Gaussian.  Writes levels and thresholds in units of z (the sigma =
 * 1/sqrt(d) scale is built in).  d >= 3. */
int oqo_codebook_sphere(int d, int bits, double *levels, double *thresholds)
{
    if (d < 3 || bits < 1 || bits > 8) return -1;
    const int L = 1 << bits;
    double t[257];
    double ul[256], ut[255];
    oqo_codebook_unit(bits, ul, ut); /* a start near the fixed point */
    for (int k = 0; k < L; k++) levels[k] = ul[k] / sqrt((double)d);
    for (int k = 0; k < L; k++) { /* keep the start inside (-1, 1) */
        if (levels[k] <= -1.0) levels[k] = -1.0 + (k + 0.5) / L;
        if (levels[k] >= 1.0) levels[k] = 1.0 - (L - k - 0.5) / L;
    }
    const int max_iter = bits <= 4 ? 400000 : 200;
    int it;
    for (it = 1; it <= max_iter; it++) {
        double move = 0.0;
        t[0] = -1.0;
        t[L] = 1.0;
        for (int k = 1; k < L; k++) t[k] = 0.5 * (levels[k - 1] + levels[k]);
        for (int k = 0; k < L; k++) {
            const double c = sphere_moment(t[k], t[k + 1], d) / sphere_mass(t[k], t[k + 1], d);
            const double dm = fabs(c - levels[k]) * sqrt((double)d);
            if (dm > move) move = dm;
            levels[k] = c;
        }
        if (move < 1e-13) break; /* the incomplete beta is good to about 1e-15 */
    }
    if (bits > 4) it += sphere_newton(d, L, levels);
    symmetrize(L, levels);
    for (int k = 1; k < L; k++) thresholds[k - 1] = 0.5 * (levels[k - 1] + levels[k]);
    return it;
}

/* P(a <= T < b) for the sphere marginal (exported for the pins). */
double oqo_sphere_mass(double a, double b, int d) { return sphere_mass(a, b, d); }

/* ------------------------------------------------------------- rotation -- */

/* In-place unnormalised Walsh-Hadamard transform of length h (power of
 * two), Sylvester natural order: out[a] = sum_b (-1)^popcount(a&b) in[b]. */
void oqo_fwht(double *v, int h)
{
    for (int len = 1; len < h; len *= 2)
        for (int i = 0; i < h; i += 2 * len)
            for (int j = i; j < i + len; j++) {
                double a = v[j], b = v[j + len];
                v[j] = a + b;
                v[j + len] = a - b;
            }
}

/* One entry of the Sylvester Hadamard matrix (+-1, unnormalised). */
int oqo_hadamard_entry(int a, int b)
{
    return (__builtin_popcount((unsigned)(a & b)) & 1) ? -1 : 1;
}

/* Rotate one token: s = ||x||, y_i = D_i x_{pi(i)}, and
 * z^(j) = H_h y^(j) / (s sqrt(h)) for each of the k = d/h blocks (z = 0
 * when s = 0): the rotation of u = x / s, normalised last.  Writes z
 * (length d) and the norm. */
void oqo_rotate_token(const double *x, int d, const int32_t *perm, const int8_t *sign,
                      int use_signs, double *z, double *norm)
{
    const int h = oqo_block_size(d);
    double ss = 0.0;
    for (int i = 0; i < d; i++) ss += x[i] * x[i];
    const double s = sqrt(ss);
    *norm = s;
    /* the rotation is linear, so it runs on x itself and the division by
     * s sqrt(h) comes last: the transform of bf16 or fp32 inputs is then
     * exact in double precision, and a coordinate that cancels exactly is
     * an exact zero (which the tie rule sends to the upper level) instead of
     * a rounding residue of either sign */
    for (int i = 0; i < d; i++) {
        const double v = x[perm[i]];
        z[i] = (use_signs && sign[i] < 0) ? -v : v;
    }
    const double den = s * sqrt((double)h);
    for (int j = 0; j < d / h; j++) {
        oqo_fwht(z + (size_t)j * h, h);
        for (int i = 0; i < h; i++)
            z[(size_t)j * h + i] = (s > 0.0) ? z[(size_t)j * h + i] / den : 0.0;
    }
}

/* ------------------------------------------------------- quantize, pack -- */

/* Nearest level of the codebook, ties to the upper level:
 * code = #{k : z >= t_k} over the L-1 ascending thresholds. */
int oqo_quantize_one(double z, const double *thresholds, int L)
{
    int code = 0;
    for (int k = 0; k < L - 1; k++)
        if (z >= thresholds[k]) code++;
    return code;
}

/* Storage slot of coordinate i of a row of d coordinates: inside each
 * whole group of 128 coordinates, coordinate 128G + 32c + p (c < 4,
 * p < 32) goes to slot 128G + 8 (p mod 16) + 4 floor(p / 16) + c; the
 * coordinates of a last, partial group (the d mod 128 = 32, 64 or 96 after
 * the whole groups) keep their own index. */
int64_t oqo_slot_of(int64_t i, int d)
{
    if (i >= (int64_t)(d / 128) * 128) return i;
    int64_t G = i / 128, r = i % 128;
    int64_t c = r / 32, p = r % 32;
    return 128 * G + 8 * (p % 16) + 4 * (p / 16) + c;
}

/* Pack one row: code of coordinate i goes to bits [b*slot(i), b*slot(i)+b)
 * of the row's byte string, little-endian bit order. */
void oqo_pack_row(const uint8_t *codes, int d, int bits, uint8_t *out)
{
    memset(out, 0, (size_t)d * bits / 8);
    for (int i = 0; i < d; i++) {
        int64_t bitpos = (int64_t)bits * oqo_slot_of(i, d);
        for (int t = 0; t < bits; t++)
            if ((codes[i] >> t) & 1)
                out[(bitpos + t) / 8] |= (uint8_t)(1u << ((bitpos + t) % 8));
    }
}

void oqo_unpack_row(const uint8_t *packed, int d, int bits, uint8_t *codes)
{
    for (int i = 0; i < d; i++) {
        int64_t bitpos = (int64_t)bits * oqo_slot_of(i, d);
        int c = 0;
        for (int t = 0; t < bits; t++)
            if ((packed[(bitpos + t) / 8] >> ((bitpos + t) % 8)) & 1) c |= 1 << t;
        codes[i] = (uint8_t)c;
    }
}

/* ------------------------------------------------------------- drivers -- */

static double load_elem(const void *x, int dtype, size_t idx)
{
    if (dtype == OQO_F32) return (double)((const float *)x)[idx];
    /* bf16: the 16 stored bits are the top half of an fp32 */
    uint32_t u = (uint32_t)((const uint16_t *)x)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Rotate and quantize `rows` rows of x (row-major, d columns).  codes may be
 * NULL (then only z / norms); z may be NULL.  Rows run in parallel. */
/* The codebook of a family: 0 = Lloyd-Max for N(0, 1/d), 1 = Lloyd-Max for
 * the exact sphere marginal of dimension d. */
static int family_codebook(int family, int d, int bits, double *lv, double *th)
{
    return family ? oqo_codebook_sphere(d, bits, lv, th) : oqo_codebook(d, bits, lv, th);
}

int oqo_rotate_quantize_ex(const void *x, int dtype, int64_t rows, int d, uint64_t seed,
                           int use_signs, int bits, int family, uint8_t *codes, double *norms,
                           double *z)
{
    if (d <= 0 || d % 32 != 0 || bits < 1 || bits > 8) return -1;
    const int L = 1 << bits;
    int32_t *perm = malloc(sizeof(int32_t) * d);
    int8_t *sign = malloc(d);
    double lv[256], th[256];
    oqo_plan(d, seed, perm, sign);
    family_codebook(family, d, bits, lv, th);
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * d);
        double *zr = malloc(sizeof(double) * d);
        uint8_t *cr = malloc(d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; r++) {
            double nrm;
            for (int i = 0; i < d; i++) xr[i] = load_elem(x, dtype, (size_t)r * d + i);
            oqo_rotate_token(xr, d, perm, sign, use_signs, zr, &nrm);
            if (norms) norms[r] = nrm;
            if (z) memcpy(z + (size_t)r * d, zr, sizeof(double) * d);
            if (codes) {
                for (int i = 0; i < d; i++) cr[i] = (uint8_t)oqo_quantize_one(zr[i], th, L);
                oqo_pack_row(cr, d, bits, codes + (size_t)r * d * bits / 8);
            }
        }
        free(xr);
        free(zr);
        free(cr);
    }
    free(perm);
    free(sign);
    return 0;
}

int oqo_rotate_quantize(const void *x, int dtype, int64_t rows, int d, uint64_t seed,
                        int use_signs, int bits, uint8_t *codes, double *norms, double *z)
{
    return oqo_rotate_quantize_ex(x, dtype, rows, d, seed, use_signs, bits, 0, codes, norms, z);
}

/* The low-bit linear, in fp64:
 *   y[m][n] = s_m r_n sum_k C_{K,bw}[p_nk] C_{K,ba}[q_mk]
 * with sigma-scaled levels.  Only the rows listed in `rows` (indices into
 * the activation rows) are computed; y is [nrows][N]. */
int oqo_linear_ex(const uint8_t *a_codes, const double *a_norms, int ba,
                  const uint8_t *w_codes, const double *w_norms, int bw, int family,
                  int64_t N, int K, const int64_t *rows, int64_t nrows, double *y)
{
    if (K <= 0 || K % 32 != 0) return -1;
    double la[256], ta[256], lw[256], tw[256];
    family_codebook(family, K, ba, la, ta);
    family_codebook(family, K, bw, lw, tw);
    double *wd = malloc(sizeof(double) * (size_t)N * K);
#pragma omp parallel
    {
        uint8_t *c = malloc(K);
        double *ad = malloc(sizeof(double) * K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            oqo_unpack_row(w_codes + (size_t)n * K * bw / 8, K, bw, c);
            for (int k = 0; k < K; k++) wd[(size_t)n * K + k] = lw[c[k]];
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; i++) {
            int64_t m = rows[i];
            oqo_unpack_row(a_codes + (size_t)m * K * ba / 8, K, ba, c);
            for (int k = 0; k < K; k++) ad[k] = la[c[k]];
            for (int64_t n = 0; n < N; n++) {
                double acc = 0.0;
                const double *wr = wd + (size_t)n * K;
                for (int k = 0; k < K; k++) acc += wr[k] * ad[k];
                y[(size_t)i * N + n] = a_norms[m] * w_norms[n] * acc;
            }
        }
        free(c);
        free(ad);
    }
    free(wd);
    return 0;
}

/* Fake quantization, the evaluation path of the pages (paper.gecl.asia
 * notes, Dataset/Evaluation; llmdb.app Implementation Details): every
 * coordinate of the rotated unit token is replaced by its codebook level
 * and scaled back by the norm, out[r][i] = s_r * C_{d,bits}[code(z_ri)], in
 * coordinate order (no packing).  fp64. */
int oqo_fake_quantize(const void *x, int dtype, int64_t rows, int d, uint64_t seed,
                      int use_signs, int bits, double *out, double *norms)
{
    if (d <= 0 || d % 32 != 0 || bits < 1 || bits > 8) return -1;
    const int L = 1 << bits;
    int32_t *perm = malloc(sizeof(int32_t) * d);
    int8_t *sign = malloc(d);
    double lv[256], th[256];
    oqo_plan(d, seed, perm, sign);
    oqo_codebook(d, bits, lv, th);
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * d);
        double *zr = malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; r++) {
            double nrm;
            for (int i = 0; i < d; i++) xr[i] = load_elem(x, dtype, (size_t)r * d + i);
            oqo_rotate_token(xr, d, perm, sign, use_signs, zr, &nrm);
            if (norms) norms[r] = nrm;
            for (int i = 0; i < d; i++)
                out[(size_t)r * d + i] = nrm * lv[oqo_quantize_one(zr[i], th, L)];
        }
        free(xr);
        free(zr);
    }
    free(perm);
    free(sign);
    return 0;
}

/* INT4 weight-only round-to-nearest of the AdaLN modulation projections
 * (paper.gecl.asia notes, Method item 5: no rotation can be folded into a
 * dynamic modulation, so those weights get INT4 RTN only; researchpod.app
 * transcript).  Per output row: amax = max |w|, scale = amax / 7,
 * q = rint(w * (7 / amax)) in [-7, 7].  These are integer decisions made in
 * floating point, so they are taken in fp32 (IEEE division and product,
 * ties to even) exactly as the library takes them; amax = 0 gives q = 0 and
 * scale 0. */
int oqo_rtn4_quantize(const void *W, int dtype, int64_t rows, int d, int8_t *q, float *scales)
{
    if (d <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float amax = 0.0f;
        for (int k = 0; k < d; k++) {
            const float w = (float)load_elem(W, dtype, (size_t)r * d + k);
            const float a = fabsf(w);
            if (a > amax) amax = a;
        }
        const float inv = amax > 0.0f ? 7.0f / amax : 0.0f;
        scales[r] = amax / 7.0f;
        for (int k = 0; k < d; k++) {
            const float w = (float)load_elem(W, dtype, (size_t)r * d + k);
            const float t = w * inv;
            q[(size_t)r * d + k] = (int8_t)rintf(t);
        }
    }
    return 0;
}

/* y[m][n] = scale_n sum_k x_mk q_nk in fp64 (the AdaLN projection with
 * INT4 RTN weights; activations unquantized). */
int oqo_rtn4_linear(const void *x, int dtype, int64_t M, const int8_t *q, const float *scales,
                    int64_t N, int K, double *y)
{
    if (K <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int k = 0; k < K; k++)
                acc += load_elem(x, dtype, (size_t)m * K + k) * (double)q[(size_t)n * K + k];
            y[(size_t)m * N + n] = acc * (double)scales[n];
        }
    }
    return 0;
}

int oqo_linear(const uint8_t *a_codes, const double *a_norms, int ba,
               const uint8_t *w_codes, const double *w_norms, int bw,
               int64_t N, int K, const int64_t *rows, int64_t nrows, double *y)
{
    return oqo_linear_ex(a_codes, a_norms, ba, w_codes, w_norms, bw, 0, N, K, rows, nrows, y);
}

/* Threads an OpenMP region of this oracle uses (for reporting). */
int oqo_num_threads(void) { return omp_get_max_threads(); }

/* Threads for the following OpenMP regions (n <= 0: every processor).
   Timing only; no result depends on it. */
void oqo_set_threads(int n) { omp_set_num_threads(n > 0 ? n : omp_get_num_procs()); }
