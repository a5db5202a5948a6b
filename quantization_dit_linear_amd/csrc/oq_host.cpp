// oq_host.cpp -- host side of liborbitquant: the C ABI declared in
// include/orbitquant.h, argument validation, the Lloyd-Max codebook solver,
// the rotation-plan builder and the per-device plan cache.
//
// The codebook is found with Max's method (J. Max, "Quantizing for minimum
// distortion", 1960; cited by the pith.science page): shoot from the
// zero threshold upwards, alternately solving the centroid condition for
// the next threshold and the midpoint condition for the next level, and
// bisect on the first positive level until the top cell's centroid
// condition holds.  The plan uses SplitMix64 (Vigna's published generator)
// driving a Durstenfeld shuffle, then one Rademacher sign per coordinate
// from the same stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <limits>
#include <mutex>
#include <tuple>
#include <vector>

#include "../../include/orbitquant.h"
#include "oq_internal.h"

namespace {

// ------------------------------------------------------------- codebook --

double npdf(double t) { return std::isinf(t) ? 0.0 : std::exp(-0.5 * t * t) * 0.3989422804014327; }

// P(a <= X < b), X ~ N(0,1), for 0 <= a < b <= inf (upper half only).
double upper_mass(double a, double b) {
  return 0.5 * std::erfc(a * M_SQRT1_2) - (std::isinf(b) ? 0.0 : 0.5 * std::erfc(b * M_SQRT1_2));
}

double cell_mean(double a, double b) { return (npdf(a) - npdf(b)) / upper_mass(a, b); }

// Given the lower edge a >= 0 of a cell and its level c (a < c < mean(a,inf)),
// the upper edge b with mean(a, b) = c.  mean(a, b) rises from a to
// mean(a, inf) as b grows, so bisection on b is safe.
double edge_for_mean(double a, double c) {
  double lo = a, hi = a + 1.0;
  while (cell_mean(a, hi) <= c) {
    lo = hi;
    hi = a + 2.0 * (hi - a);
    if (hi > 40.0) return INFINITY;
  }
  for (int i = 0; i < 200 && hi - lo > 1e-17 * hi; i++) {
    double mid = 0.5 * (lo + hi);
    if (cell_mean(a, mid) < c) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Shoot the positive half (P = L/2 levels) from the first positive level c0.
// Returns > 0 if the shot overshoots (the top cell cannot have c0's
// successor as its mean), < 0 if it undershoots.
double shoot(double c0, int P, double *pos_levels, double *pos_edges) {
  double a = 0.0, c = c0;
  for (int k = 0; k < P - 1; k++) {
    pos_levels[k] = c;
    if (c >= cell_mean(a, INFINITY)) return 1.0;
    double b = edge_for_mean(a, c);
    if (std::isinf(b)) return 1.0;
    pos_edges[k] = b;
    c = 2.0 * b - c;  // the next level: b is the midpoint of c and c'
    a = b;
  }
  pos_levels[P - 1] = c;
  return c - cell_mean(a, INFINITY);
}

// Unit-variance Lloyd-Max codebook: L = 2^bits ascending levels, L-1
// thresholds, bits 1..8.  Cached: the result depends on bits only.  At 8
// bits the shot carries the first level's rounding through 127 cells; the
// levels still come out within about 1e-9 of the fixed point, far below the
// fp32 precision the kernels use them in.
void unit_codebook(int bits, double *levels, double *thresholds) {
  static std::mutex mu;
  static bool done[9] = {};
  static double lv[9][256], th[9][255];
  std::lock_guard<std::mutex> g(mu);
  const int L = 1 << bits, P = L / 2;
  if (!done[bits]) {
    double pl[128], pe[128];
    if (P == 1) {
      pl[0] = cell_mean(0.0, INFINITY);
    } else {
      double lo = 0.0, hi = cell_mean(0.0, INFINITY);
      for (int i = 0; i < 400; i++) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (shoot(mid, P, pl, pe) > 0) hi = mid; else lo = mid;
      }
      shoot(0.5 * (lo + hi), P, pl, pe);
    }
    for (int k = 0; k < P; k++) {
      lv[bits][P + k] = pl[k];
      lv[bits][P - 1 - k] = -pl[k];
    }
    for (int k = 0; k < L - 1; k++) th[bits][k] = 0.5 * (lv[bits][k] + lv[bits][k + 1]);
    th[bits][P - 1] = 0.0;
    done[bits] = true;
  }
  std::memcpy(levels, lv[bits], sizeof(double) * L);
  std::memcpy(thresholds, th[bits], sizeof(double) * (L - 1));
}

// ---- exact sphere marginal.  One coordinate of a uniform point on
// S^{d-1} has density c_d (1 - t^2)^((d-3)/2); in unit-variance units
// u = sqrt(d) t the upper-half masses come from Gauss-Legendre quadrature
// and the first moments from the closed form
//   int u g(u) du = -sqrt(d) c_d (1 - u^2/d)^((d-1)/2) / (d - 1).

struct GaussLegendre {
  static constexpr int n = 32;
  double x[n], w[n];
  GaussLegendre() {  // nodes on [-1, 1] by Newton's method on P_n
    for (int i = 0; i < n; i++) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5)), pp = 1.0;
      for (int it = 0; it < 100; it++) {
        double p1 = 1.0, p2 = 0.0;
        for (int j = 1; j <= n; j++) {
          const double p3 = p2;
          p2 = p1;
          p1 = ((2.0 * j - 1.0) * z * p2 - (j - 1.0) * p3) / j;
        }
        pp = n * (z * p1 - p2) / (z * z - 1.0);
        const double dz = p1 / pp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * pp * pp);
    }
  }
};

struct SphereDist {
  int d;
  double lc;  // log c_d
  explicit SphereDist(int d_) : d(d_) {
    lc = std::lgamma(0.5 * d) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (d - 1));
  }
  double top() const { return std::sqrt((double)d); }
  double g(double u) const {  // density of u
    const double r = 1.0 - u * u / d;
    return r <= 0.0 ? 0.0 : std::exp(lc + 0.5 * (d - 3) * std::log(r)) / std::sqrt((double)d);
  }
  double mass(double a, double b) const {  // 0 <= a < b
    static const GaussLegendre gl;
    b = std::min(b, std::min(top(), a + 48.0));  // beyond: below 1e-300
    double s = 0.0;
    for (double lo = a; lo < b; lo += 0.25) {
      const double hi = std::min(lo + 0.25, b), h = 0.5 * (hi - lo), m = 0.5 * (hi + lo);
      for (int i = 0; i < GaussLegendre::n; i++) s += gl.w[i] * g(m + h * gl.x[i]) * h;
    }
    return s;
  }
  double moment(double a, double b) const {
    auto pw = [&](double u) {
      const double r = 1.0 - u * u / d;
      return r <= 0.0 ? 0.0 : std::exp(0.5 * (d - 1) * std::log(r));
    };
    return std::sqrt((double)d) * std::exp(lc) * (pw(a) - pw(b)) / (d - 1);
  }
  double mean(double a, double b) const { return moment(a, b) / mass(a, b); }
};

// Max's shooting method on the upper half of a symmetric density: the first
// positive level c0 is bisected until the last cell's mean matches.
template <class Mean>
void shoot_codebook(int bits, double top, const Mean &mean, double *lv, double *th) {
  const int L = 1 << bits, P = L / 2;
  double pl[128], pe[128];
  auto edge_for = [&](double a, double c) {  // b with mean(a, b) = c
    double lo = a, hi = std::min(a + 1.0, top);
    while (mean(a, hi) <= c) {
      if (hi >= top) return top;
      lo = hi;
      hi = std::min(a + 2.0 * (hi - a), top);
    }
    for (int i = 0; i < 200 && hi - lo > 1e-17 * hi; i++) {
      const double mid = 0.5 * (lo + hi);
      if (mean(a, mid) < c) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
  };
  auto shot = [&](double c0) {
    double a = 0.0, c = c0;
    for (int k = 0; k < P - 1; k++) {
      pl[k] = c;
      if (c >= mean(a, top)) return 1.0;
      const double b = edge_for(a, c);
      if (b >= top) return 1.0;
      pe[k] = b;
      c = 2.0 * b - c;
      a = b;
    }
    pl[P - 1] = c;
    return c - mean(a, top);
  };
  if (P == 1) {
    pl[0] = mean(0.0, top);
  } else {
    double lo = 0.0, hi = mean(0.0, top);
    for (int i = 0; i < 400; i++) {
      const double mid = 0.5 * (lo + hi);
      if (mid <= lo || mid >= hi) break;
      if (shot(mid) > 0) hi = mid; else lo = mid;
    }
    shot(0.5 * (lo + hi));
  }
  for (int k = 0; k < P; k++) {
    lv[P + k] = pl[k];
    lv[P - 1 - k] = -pl[k];
  }
  for (int k = 0; k < L - 1; k++) th[k] = 0.5 * (lv[k] + lv[k + 1]);
  th[P - 1] = 0.0;
}

// Newton's method on the Lloyd-Max conditions of a symmetric density over
// the upper half-line: unknowns the P positive levels c_0 < ... < c_{P-1}
// (lv on entry: a start close to the solution), cells [e_k, e_{k+1}) with
// e_0 = 0, e_k = (c_{k-1} + c_k) / 2, e_P = top; conditions
// F_k = c_k - mean(e_k, e_{k+1}) = 0.  With m the cell mass and g the
// density, d mean / d e_k = g(e_k)(mean - e_k)/m and
// d mean / d e_{k+1} = g(e_{k+1})(e_{k+1} - mean)/m, so the Jacobian is
// tridiagonal (each inner edge moves with both neighbouring levels by 1/2).
// Used where shooting loses accuracy (8 bits: its forward sweep magnifies
// the first level's rounding across 128 cells).  Stops after a step below
// 1e-14 or once steps stop shrinking.
template <class Dist>
void newton_upper_half(int P, const Dist &dist, double *c) {
  std::vector<double> e(P + 1), lo(P), di(P), up(P), rhs(P);
  double prev = INFINITY;
  for (int it = 0; it < 60; it++) {
    e[0] = 0.0;
    e[P] = dist.top();
    for (int k = 1; k < P; k++) e[k] = 0.5 * (c[k - 1] + c[k]);
    for (int k = 0; k < P; k++) {
      const double a = e[k], b = e[k + 1], m = dist.mass(a, b);
      const double mu = dist.moment(a, b) / m;
      const double da = (k == 0) ? 0.0 : dist.g(a) * (mu - a) / m;
      const double db = (k == P - 1) ? 0.0 : dist.g(b) * (b - mu) / m;
      lo[k] = -0.5 * da;
      up[k] = -0.5 * db;
      di[k] = 1.0 - 0.5 * da - 0.5 * db;
      rhs[k] = mu - c[k];
    }
    for (int k = 1; k < P; k++) {  // Thomas algorithm
      const double f = lo[k] / di[k - 1];
      di[k] -= f * up[k - 1];
      rhs[k] -= f * rhs[k - 1];
    }
    rhs[P - 1] /= di[P - 1];
    for (int k = P - 2; k >= 0; k--) rhs[k] = (rhs[k] - up[k] * rhs[k + 1]) / di[k];
    double move = 0.0;
    for (int k = 0; k < P; k++) {
      c[k] += rhs[k];
      move = std::max(move, std::fabs(rhs[k]));
    }
    if (move < 1e-14 || (it >= 2 && move > 0.5 * prev)) break;
    prev = move;
  }
}

// Unit-variance codebook of a family: Gaussian (d-independent) or the exact
// sphere marginal of dimension d (cached per (d, bits)).
void family_codebook(int d, int bits, bool sphere, double *levels, double *thresholds) {
  if (!sphere) {
    unit_codebook(bits, levels, thresholds);
    return;
  }
  static std::mutex mu;
  static std::map<std::pair<int, int>, std::vector<double>> cache;
  const int L = 1 << bits;
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find({d, bits});
  if (it == cache.end()) {
    SphereDist dist(d);
    std::vector<double> v(2 * L);
    if (bits <= 4) {
      shoot_codebook(bits, dist.top(), [&](double a, double b) { return dist.mean(a, b); },
                     v.data(), v.data() + L);
    } else {
      // from the Gaussian codebook (the d -> infinity limit, within a few
      // percent at d = 128), Newton on the sphere conditions
      const int P = L / 2;
      double gl[256], gt[255];
      unit_codebook(bits, gl, gt);
      std::vector<double> c(gl + P, gl + L);
      newton_upper_half(P, dist, c.data());
      for (int k = 0; k < P; k++) {
        v[P + k] = c[k];
        v[P - 1 - k] = -c[k];
      }
      for (int k = 0; k < L - 1; k++) v[L + k] = 0.5 * (v[k] + v[k + 1]);
      v[L + P - 1] = 0.0;
    }
    it = cache.emplace(std::make_pair(d, bits), v).first;
  }
  std::memcpy(levels, it->second.data(), sizeof(double) * L);
  std::memcpy(thresholds, it->second.data() + L, sizeof(double) * (L - 1));
}

uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  uint16_t u;
  std::memcpy(&u, &h, 2);
  return u;
}

// ----------------------------------------------------------------- plan --

struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ULL;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
  }
};

// perm[i] = pi(i) (the gather y_i = x_{pi(i)}), neg[i] = D_i < 0.
void build_plan(int d, uint64_t seed, std::vector<int32_t> &perm, std::vector<uint8_t> &neg) {
  SplitMix64 g{seed};
  perm.resize(d);
  neg.resize(d);
  for (int i = 0; i < d; i++) perm[i] = i;
  for (int i = d - 1; i >= 1; i--) {
    unsigned __int128 p = (unsigned __int128)g.next() * (unsigned __int128)(uint64_t)(i + 1);
    int j = (int)(uint64_t)(p >> 64);
    std::swap(perm[i], perm[j]);
  }
  for (int i = 0; i < d; i++) neg[i] = (uint8_t)(g.next() >> 63);
}

struct PlanKey {
  int dev, d;
  uint64_t seed;
  bool operator<(const PlanKey &o) const {
    return std::tie(dev, d, seed) < std::tie(o.dev, o.d, o.seed);
  }
};

std::mutex g_plan_mu;
std::map<PlanKey, oq::DevicePlan> g_plans;

void free_plan_tables(const oq::DevicePlan &p) {
  for (void *ptr : {(void *)p.scatter, (void *)p.scatter_nosign, (void *)p.fast_scatter,
                    (void *)p.fast_signs, (void *)p.fast_nosigns, (void *)p.scatter_id,
                    (void *)p.fast_signs_id, (void *)p.perm_inv})
    if (ptr) (void)hipFree(ptr);
}

// Returns a copy of the cached entry, taken under the lock: another thread's
// oq_plan_destroy or oq_release_plans may erase the entry right after.
int get_plan(int d, uint64_t seed, hipStream_t stream, oq::DevicePlan *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return OQ_EDEVICE;
  std::lock_guard<std::mutex> g(g_plan_mu);
  PlanKey key{dev, d, seed};
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    *out = it->second;
    return OQ_OK;
  }
  std::vector<int32_t> perm;
  std::vector<uint8_t> neg;
  build_plan(d, seed, perm, neg);
  std::vector<int32_t> sc(d), sc0(d), sid(d);
  std::vector<uint32_t> fsc(d), fsg(d / 2), fz(d / 2, 0u), fsid(d / 2);
  // fast path: slots of min(h, 1024) coordinates, each followed by 8
  // elements of padding in the kernel's LDS copy of a token
  const int slot = oq::fast_slot(d);
  for (int i = 0; i < d; i++) {
    sc[perm[i]] = i | (neg[i] ? (int32_t)0x80000000 : 0);
    sc0[perm[i]] = i;
    // source j = pi(i) goes to element i of the padded copy
    fsc[perm[i]] = 2u * (uint32_t)(i + 8 * (i / slot));
    sid[i] = i | (neg[i] ? (int32_t)0x80000000 : 0);
  }
  for (int j = 0; j < d; j += 2) {
    const int i0 = sc0[j], i1 = sc0[j + 1];
    fsg[j / 2] = (neg[i0] ? 0x8000u : 0u) | (neg[i1] ? 0x80000000u : 0u);
    fsid[j / 2] = (neg[j] ? 0x8000u : 0u) | (neg[j + 1] ? 0x80000000u : 0u);
  }
  oq::DevicePlan p;
  p.d = d;
  p.h = d & -d;
  struct Up {
    void **dst;
    const void *src;
    size_t bytes;
  } ups[] = {{(void **)&p.scatter, sc.data(), sizeof(int32_t) * d},
             {(void **)&p.scatter_nosign, sc0.data(), sizeof(int32_t) * d},
             {(void **)&p.fast_scatter, fsc.data(), sizeof(uint32_t) * d},
             {(void **)&p.fast_signs, fsg.data(), sizeof(uint32_t) * (d / 2)},
             {(void **)&p.fast_nosigns, fz.data(), sizeof(uint32_t) * (d / 2)},
             {(void **)&p.scatter_id, sid.data(), sizeof(int32_t) * d},
             {(void **)&p.fast_signs_id, fsid.data(), sizeof(uint32_t) * (d / 2)},
             {(void **)&p.perm_inv, sc0.data(), sizeof(int32_t) * d}};
  int rc = OQ_OK;
  for (auto &u : ups) {
    if (hipMalloc(u.dst, u.bytes) != hipSuccess) {
      rc = OQ_ENOMEM;
      break;
    }
    // synchronous upload: the host vectors go out of scope afterwards
    if (hipMemcpy(*u.dst, u.src, u.bytes, hipMemcpyHostToDevice) != hipSuccess) {
      rc = OQ_EDEVICE;
      break;
    }
  }
  if (rc != OQ_OK) {
    for (auto &u : ups)
      if (*u.dst) (void)hipFree(*u.dst);
    return rc;
  }
  (void)stream;
  g_plans.emplace(key, p);
  *out = p;
  return OQ_OK;
}

// Device codebook table (layout in oq_internal.h).  Cell grid of the bf16
// fast path: the kernel maps a unit-space value u (= sqrt(d) z), clamped to
// the grid's range, to cell c = floor(u / delta + C/2 + 1/16) (C cells of
// width delta; the first and last cells also take every value beyond, where
// no threshold lies).  Entry c = {tau, base}: base = number of thresholds at
// or below the cell, tau = the only threshold that can fall inside it (or
// +inf), so the code is base + (u >= tau) with the unclamped u.  The cell's
// extent allows for the kernel's rounding (1/16 cell each side, plus 2%); a
// cell holding two thresholds would need a finer grid: rejected (never the
// case for the 2-4 bit grid of 1/8 or the 8-bit grid of 1/128, whose
// closest Gaussian thresholds are 0.0169 apart).
int build_cells(int d, int bits, bool sphere, std::vector<uint32_t> &out) {
  double lv[256], th[255];
  family_codebook(d, bits, sphere, lv, th);
  const int T = (1 << bits) - 1, C = oq::cells_for_bits(bits);
  const double delta = bits == 8 ? 1.0 / 128.0 : 0.125, eps = 0.02 * delta;
  out.assign(oq::table_thresholds_word(bits) + T, 0);
  for (int c = 0; c < C; c++) {
    const double inf = std::numeric_limits<double>::infinity();
    const double lo = c == 0 ? -inf : delta * (c - 0.5 * C - 0.0625) - eps;
    const double hi = c == C - 1 ? inf : delta * (c - 0.5 * C + 0.9375) + eps;
    int base = 0, inside = 0;
    for (int k = 0; k < T; k++) {
      if ((double)(float)th[k] <= lo) base++;
      else if ((double)(float)th[k] <= hi) inside++;
    }
    if (inside > 1) return OQ_EUNSUPPORTED;
    const float tau = base < T ? (float)th[base] : std::numeric_limits<float>::infinity();
    uint32_t tb;
    std::memcpy(&tb, &tau, 4);
    out[2 * c] = tb;
    out[2 * c + 1] = (uint32_t)base;
  }
  for (int k = 0; k <= T; k++) {
    const float f = (float)lv[k];
    std::memcpy(&out[oq::table_levels_word(bits) + k], &f, 4);
  }
  for (int k = 0; k < T; k++) {
    const float f = (float)th[k];
    std::memcpy(&out[oq::table_thresholds_word(bits) + k], &f, 4);
  }
  return OQ_OK;
}

std::mutex g_cell_mu;
// (device, bits, d for the sphere family or 0) -> device codebook table
std::map<std::tuple<int, int, int>, uint32_t *> g_cells;

int get_cells(int d, int bits, bool sphere, const uint32_t **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return OQ_EDEVICE;
  std::lock_guard<std::mutex> g(g_cell_mu);
  const auto key = std::make_tuple(dev, bits, sphere ? d : 0);
  auto it = g_cells.find(key);
  if (it != g_cells.end()) {
    *out = it->second;
    return OQ_OK;
  }
  std::vector<uint32_t> tab;
  int rc = build_cells(d, bits, sphere, tab);
  if (rc != OQ_OK) return rc;
  uint32_t *dptr = nullptr;
  if (hipMalloc(&dptr, tab.size() * 4) != hipSuccess) return OQ_ENOMEM;
  if (hipMemcpy(dptr, tab.data(), tab.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dptr);
    return OQ_EDEVICE;
  }
  g_cells[key] = dptr;
  *out = dptr;
  return OQ_OK;
}

// ----------------------------------------------------------- validation --

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Byte ranges [p, p + pb) and [q, q + qb) share at least one byte.
bool overlaps(const void *p, int64_t pb, const void *q, int64_t qb) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qb && b < a + (uintptr_t)pb;
}

// Largest row count of either linear operand (tile indices stay in int).
constexpr int64_t kMaxRows = (int64_t)1 << 30;

int check_d_bits(int d, int bits) {
  if (d <= 0) return OQ_EINVAL;
  if ((bits < 2 || bits > 4) && bits != 8) return OQ_EUNSUPPORTED;
  if (d % oq::kDimStep != 0 || d > oq::kMaxD) return OQ_EUNSUPPORTED;
  return OQ_OK;
}

int rotate_common(const void *x, int dtype, int64_t n_tok, int d, uint64_t seed, uint32_t flags,
                  int bits, void *out, float *norms, void *stream, bool allow_rotated) {
  if (n_tok < 0) return OQ_EINVAL;
  if (dtype != OQ_F32 && dtype != OQ_BF16) return OQ_EINVAL;
  const uint32_t outs = OQ_OUT_F32_ROTATED | OQ_OUT_BF16_DEQUANT;
  if (flags & ~(OQ_ROT_NO_SIGNS | OQ_ROT_INPUT_PERMUTED | OQ_CODEBOOK_SPHERE | outs))
    return OQ_EINVAL;
  const bool sphere = (flags & OQ_CODEBOOK_SPHERE) != 0;
  if ((flags & outs) && !allow_rotated) return OQ_EINVAL;
  if ((flags & outs) == outs) return OQ_EINVAL;
  int rc = check_d_bits(d, bits);
  if (rc != OQ_OK) return rc;
  if (n_tok == 0) return OQ_OK;  // empty input: nothing to do, pointers may be null
  if (!x || !out || !norms) return OQ_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(norms, 4)) return OQ_EINVAL;
  oq::DevicePlan plan;
  rc = get_plan(d, seed, (hipStream_t)stream, &plan);
  if (rc != OQ_OK) return rc;
  double lv[256], th[255];
  family_codebook(d, bits, sphere, lv, th);
  oq::Thresholds t{};
  t.count = (1 << bits) - 1;
  for (int k = 0; k < t.count && k < 15; k++) t.t[k] = (float)th[k];
  oq::RotateArgs a{};
  a.x = x;
  a.dtype = dtype;
  a.n_tok = n_tok;
  a.d = d;
  a.h = d & -d;
  a.bits = bits;
  a.signs = !(flags & OQ_ROT_NO_SIGNS);
  a.rotated_out = (flags & OQ_OUT_F32_ROTATED) != 0;
  a.dequant_out = (flags & OQ_OUT_BF16_DEQUANT) != 0;
  a.input_permuted = (flags & OQ_ROT_INPUT_PERMUTED) != 0;
  for (int k = 0; k < (1 << bits) && k < 16; k++) a.levels.v[k] = (float)lv[k];
  a.out = out;
  a.norms = norms;
  a.stream = (hipStream_t)stream;
  const uint32_t *table = nullptr;
  rc = get_cells(d, bits, sphere, &table);
  if (rc != OQ_OK) return rc;
  if (a.dtype == OQ_BF16) {
    bool handled = false;
    const uint32_t *smask = a.input_permuted ? (a.signs ? plan.fast_signs_id : plan.fast_nosigns)
                                             : (a.signs ? plan.fast_signs : plan.fast_nosigns);
    hipError_t e = oq::launch_rotate_quantize_fast(a, plan.fast_scatter, smask, table, &handled);
    if (handled) return e == hipSuccess ? OQ_OK : OQ_EDEVICE;
  }
  hipError_t e = oq::launch_rotate_quantize_generic(a, plan, t, table);
  return e == hipSuccess ? OQ_OK : OQ_EDEVICE;
}

}  // namespace

// ------------------------------------------------------------------ ABI --

extern "C" {

const char *oq_strerror(int status) {
  switch (status) {
    case OQ_OK: return "success";
    case OQ_EINVAL: return "invalid argument (null or misaligned pointer, bad size, dtype or flag)";
    case OQ_EUNSUPPORTED: return "unsupported configuration (d must be a multiple of 32 in [32, 16384], and the linear's K a multiple of 64; bits in {2,3,4,8}; 8 bits on both sides of a linear; the sphere codebook at 1-4 and 8 bits)";
    case OQ_ENOMEM: return "out of device memory for the rotation plan";
    case OQ_EDEVICE: return "HIP runtime or kernel launch failure";
    default: return "unknown status";
  }
}

int oq_version(void) { return 100; }

int oq_codebook_ex(int d, int bits, uint32_t flags, float *levels, float *thresholds) {
  if (!levels || !thresholds || d < 1) return OQ_EINVAL;
  if (flags & ~OQ_CODEBOOK_SPHERE) return OQ_EINVAL;
  if (bits < 1 || bits > 8) return OQ_EUNSUPPORTED;
  const bool sphere = (flags & OQ_CODEBOOK_SPHERE) != 0;
  if (sphere && (d % oq::kDimStep != 0 || d > oq::kMaxD || (bits > 4 && bits != 8)))
    return OQ_EUNSUPPORTED;
  double lv[256], th[255];
  family_codebook(d, bits, sphere, lv, th);
  const double sigma = 1.0 / std::sqrt((double)d);
  const int L = 1 << bits;
  for (int k = 0; k < L; k++) levels[k] = (float)(lv[k] * sigma);
  for (int k = 0; k < L - 1; k++) thresholds[k] = (float)(th[k] * sigma);
  return OQ_OK;
}

int oq_codebook(int d, int bits, float *levels, float *thresholds) {
  return oq_codebook_ex(d, bits, 0, levels, thresholds);
}

int64_t oq_codes_bytes(int64_t rows, int d, int bits) {
  if (rows < 0 || d < 0 || bits < 1 || bits > 8) return -1;
  return rows * (int64_t)d * bits / 8;
}

int oq_rotate_quantize(const void *x, int dtype, int64_t n_tok, int d, uint64_t seed,
                       uint32_t flags, int bits, void *out, float *norms, void *stream) {
  return rotate_common(x, dtype, n_tok, d, seed, flags, bits, out, norms, stream, true);
}

int oq_prepare_weights(const void *W, int dtype, int64_t n_out, int d_in, uint64_t seed,
                       uint32_t flags, int bits, uint8_t *w_codes, float *row_norms,
                       void *stream) {
  return rotate_common(W, dtype, n_out, d_in, seed, flags, bits, w_codes, row_norms, stream,
                       false);
}

int oq_linear_ex(const uint8_t *a_codes, const float *a_norms, int a_bits, const uint8_t *w_codes,
                 const float *w_norms, int w_bits, int64_t M, int64_t N, int K, uint32_t flags,
                 uint16_t *y, void *stream) {
  if (M < 0 || N < 0) return OQ_EINVAL;
  if (flags & ~OQ_CODEBOOK_SPHERE) return OQ_EINVAL;
  const bool sphere = (flags & OQ_CODEBOOK_SPHERE) != 0;
  int rc = check_d_bits(K, a_bits);
  if (rc != OQ_OK) return rc;
  rc = check_d_bits(K, w_bits);
  if (rc != OQ_OK) return rc;
  if (K % oq::kLinearKStep != 0) return OQ_EUNSUPPORTED;  // whole 64-slot K steps
  if ((a_bits == 8) != (w_bits == 8)) return OQ_EUNSUPPORTED;  // W8A8 only, no mixed pair
  if (M > kMaxRows || N > kMaxRows) return OQ_EUNSUPPORTED;
  if (M == 0 || N == 0) return OQ_OK;  // empty output: pointers may be null
  if (!a_codes || !a_norms || !w_codes || !w_norms || !y) return OQ_EINVAL;
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_norms, 4) ||
      !aligned(w_norms, 4) || !aligned(y, 2))
    return OQ_EINVAL;
  // y must not share a byte with any input: a sparse last round of tiles
  // parks fp32 partial sums in y's first rows before the other tiles have
  // read their codes, so an overlap would corrupt the call's own inputs
  const int64_t y_bytes = M * N * 2;
  if (overlaps(y, y_bytes, a_codes, M * (int64_t)K * a_bits / 8) ||
      overlaps(y, y_bytes, a_norms, M * 4) ||
      overlaps(y, y_bytes, w_codes, N * (int64_t)K * w_bits / 8) ||
      overlaps(y, y_bytes, w_norms, N * 4))
    return OQ_EINVAL;
  oq::LevelsF16 la{}, lw{};
  const uint32_t *ta = nullptr, *tw = nullptr;
  if (a_bits == 8) {  // 256 levels: the kernel reads them from the device tables
    rc = get_cells(K, a_bits, sphere, &ta);
    if (rc != OQ_OK) return rc;
    rc = get_cells(K, w_bits, sphere, &tw);
    if (rc != OQ_OK) return rc;
  } else {
    double lv[16], th[15];
    family_codebook(K, a_bits, sphere, lv, th);
    for (int k = 0; k < (1 << a_bits); k++) la.v[k] = f32_to_f16_bits((float)lv[k]);
    family_codebook(K, w_bits, sphere, lv, th);
    for (int k = 0; k < (1 << w_bits); k++) lw.v[k] = f32_to_f16_bits((float)lv[k]);
  }
  oq::LinearArgs a{a_codes, a_norms, a_bits, w_codes, w_norms, w_bits, M, N, K, y,
                   (hipStream_t)stream};
  hipError_t e = oq::launch_linear(a, la, lw, ta, tw);
  return e == hipSuccess ? OQ_OK : OQ_EDEVICE;
}

int oq_linear(const uint8_t *a_codes, const float *a_norms, int a_bits, const uint8_t *w_codes,
              const float *w_norms, int w_bits, int64_t M, int64_t N, int K, uint16_t *y,
              void *stream) {
  return oq_linear_ex(a_codes, a_norms, a_bits, w_codes, w_norms, w_bits, M, N, K, 0, y, stream);
}

int oq_rtn4_prepare_weights(const void *W, int dtype, int64_t n_out, int d_in, uint8_t *q4,
                            float *scales, void *stream) {
  if (n_out < 0 || d_in <= 0) return OQ_EINVAL;
  if (dtype != OQ_F32 && dtype != OQ_BF16) return OQ_EINVAL;
  if (d_in % 32 != 0 || d_in > 16384) return OQ_EUNSUPPORTED;
  if (n_out == 0) return OQ_OK;
  if (!W || !q4 || !scales) return OQ_EINVAL;
  if (!aligned(W, 4) || !aligned(q4, 16) || !aligned(scales, 4)) return OQ_EINVAL;
  hipError_t e = oq::launch_rtn4_prepare(W, dtype, n_out, d_in, q4, scales, (hipStream_t)stream);
  return e == hipSuccess ? OQ_OK : OQ_EDEVICE;
}

int oq_rtn4_linear(const void *x, int dtype, int64_t M, const uint8_t *q4, const float *scales,
                   int64_t N, int K, uint16_t *y, void *stream) {
  if (M < 0 || N < 0 || K <= 0) return OQ_EINVAL;
  if (dtype != OQ_F32 && dtype != OQ_BF16) return OQ_EINVAL;
  if (K % 32 != 0 || K > 16384) return OQ_EUNSUPPORTED;
  if (M == 0 || N == 0) return OQ_OK;
  if (N > ((int64_t)1 << 34) / 16) return OQ_EUNSUPPORTED;
  if (!x || !q4 || !scales || !y) return OQ_EINVAL;
  if (!aligned(x, 16) || !aligned(q4, 16) || !aligned(scales, 4) || !aligned(y, 2))
    return OQ_EINVAL;
  hipError_t e =
      oq::launch_rtn4_linear(x, dtype, M, q4, scales, N, K, y, (hipStream_t)stream);
  return e == hipSuccess ? OQ_OK : OQ_EDEVICE;
}

int oq_permute_rows(const void *src, void *dst, int64_t rows, int64_t row_bytes, uint64_t seed,
                    void *stream) {
  if (!src || !dst || src == dst || row_bytes < 1 || rows <= 0) return OQ_EINVAL;
  if (rows % oq::kDimStep != 0 || rows > oq::kMaxD) return OQ_EUNSUPPORTED;
  oq::DevicePlan plan;
  int rc = get_plan((int)rows, seed, (hipStream_t)stream, &plan);
  if (rc != OQ_OK) return rc;
  hipError_t e =
      oq::launch_permute_rows(src, dst, rows, row_bytes, plan.perm_inv, (hipStream_t)stream);
  return e == hipSuccess ? OQ_OK : OQ_EDEVICE;
}

// Explicit plan handles: a handle names a cache entry and pins it; the
// entry's tables are freed when its last handle is destroyed (entries made
// implicitly by the compute calls stay until oq_release_plans).
struct PlanHandle {
  uint32_t magic;
  int dev, d;
  uint64_t seed;
};
constexpr uint32_t kPlanMagic = 0x4f51504cu;  // "OQPL"

int oq_plan_create(int d, uint64_t seed, uint32_t flags, void **plan) {
  if (!plan) return OQ_EINVAL;
  *plan = nullptr;
  if (flags & ~OQ_ROT_NO_SIGNS) return OQ_EINVAL;
  if (d <= 0) return OQ_EINVAL;
  if (d % oq::kDimStep != 0 || d > oq::kMaxD) return OQ_EUNSUPPORTED;
  oq::DevicePlan p;
  int rc = get_plan(d, seed, nullptr, &p);
  if (rc != OQ_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return OQ_EDEVICE;
  {
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_plans.find(PlanKey{dev, d, seed});
    if (it == g_plans.end()) return OQ_EDEVICE;  // released concurrently
    it->second.pins++;
  }
  *plan = new PlanHandle{kPlanMagic, dev, d, seed};
  return OQ_OK;
}

int oq_plan_destroy(void *plan) {
  if (!plan) return OQ_EINVAL;
  PlanHandle *h = (PlanHandle *)plan;
  if (h->magic != kPlanMagic) return OQ_EINVAL;
  int rc = OQ_OK;
  {
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_plans.find(PlanKey{h->dev, h->d, h->seed});
    if (it != g_plans.end() && --it->second.pins <= 0) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      if (hipSetDevice(h->dev) != hipSuccess) rc = OQ_EDEVICE;
      free_plan_tables(it->second);
      (void)hipSetDevice(cur);
      g_plans.erase(it);
    }
  }
  h->magic = 0;
  delete h;
  return rc;
}

int oq_release_plans(void) {
  std::lock_guard<std::mutex> g(g_plan_mu);
  int rc = OQ_OK;
  for (auto &kv : g_plans) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    if (hipSetDevice(kv.first.dev) != hipSuccess) rc = OQ_EDEVICE;
    free_plan_tables(kv.second);
    (void)hipSetDevice(cur);
  }
  g_plans.clear();
  std::lock_guard<std::mutex> gc(g_cell_mu);
  for (auto &kv : g_cells) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    if (hipSetDevice(std::get<0>(kv.first)) != hipSuccess) rc = OQ_EDEVICE;
    (void)hipFree(kv.second);
    (void)hipSetDevice(cur);
  }
  g_cells.clear();
  return rc;
}

}  // extern "C"
