// Host-side codebook construction (runs once per codebook, float64).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "第一阶段" items 1-2 and
// "如何实现 TurboQuant" item 1: a random orthogonal rotation from the QR of a
// Gaussian matrix, and a Lloyd-Max codebook precomputed per (head dim, bits)
// for the Beta((d-1)/2,(d-1)/2) law of a rotated coordinate on [-1, 1].
//
// Methods chosen here:
//  * Gaussian entries: splitmix64 stream from the seed, uniforms
//    (x >> 11) * 2^-53, Box-Muller cosine branch, row-major fill.
//  * QR: Householder reflections; the sign of each column of Q is fixed so
//    that diag(R) > 0, which makes Q unique for a given G.
//  * Coordinate CDF: regularized incomplete beta I_x(a, a) by its continued
//    fraction (Abramowitz & Stegun 26.5.8) evaluated with the modified Lentz
//    method; cell first moments from the antiderivative -(1-y^2)^a/(2aB).
//  * Lloyd-Max: symmetric half problem (cells in [-1, 0], middle boundary 0),
//    Lloyd iterations to a 1e-7 step, then Newton steps on the midpoint
//    residual with a tridiagonal (Thomas) solve.
#include <cmath>
#include <cstdint>
#include <string>
#include <vector>

#include "tq_internal.hpp"

namespace tq {
namespace {

// Iteration limits of the Lloyd-Max solve (per thread; tests shrink them to
// reach the non-convergence error path).
constexpr int kLloydDefault = 400000, kNewtonDefault = 80;
thread_local int g_lloyd_iters = kLloydDefault;
thread_local int g_newton_iters = kNewtonDefault;

// ---------------------------------------------------------------- Gaussian

struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return (double)(next() >> 11) * 0x1.0p-53; }
};

void gaussian_fill(uint64_t seed, std::vector<double>& out) {
  SplitMix64 g{seed};
  const double two_pi = 6.283185307179586476925286766559;
  for (double& v : out) {
    double u1 = g.uniform();
    double u2 = g.uniform();
    v = std::sqrt(-2.0 * std::log1p(-u1)) * std::cos(two_pi * u2);
  }
}

// ---------------------------------------------------------------- QR

// Q (row-major n x n) of the Householder QR of G (row-major), with the sign
// of column j flipped when R_jj < 0.
void householder_q(int n, const std::vector<double>& G, std::vector<double>& Q) {
  std::vector<double> A(G);               // overwritten by R
  std::vector<double> V((size_t)n * n, 0.0);  // reflector j in column j
  std::vector<double> beta(n, 0.0);
  for (int j = 0; j < n; ++j) {
    double norm2 = 0.0;
    for (int i = j; i < n; ++i) norm2 += A[(size_t)i * n + j] * A[(size_t)i * n + j];
    double alpha = std::sqrt(norm2);
    double x0 = A[(size_t)j * n + j];
    if (alpha == 0.0) { beta[j] = 0.0; continue; }
    // v = x + sign(x0) |x| e1 (avoids cancellation); H = I - beta v v^T
    double s = (x0 >= 0.0) ? 1.0 : -1.0;
    for (int i = j; i < n; ++i) V[(size_t)i * n + j] = A[(size_t)i * n + j];
    V[(size_t)j * n + j] += s * alpha;
    double vnorm2 = 0.0;
    for (int i = j; i < n; ++i) vnorm2 += V[(size_t)i * n + j] * V[(size_t)i * n + j];
    beta[j] = 2.0 / vnorm2;
    for (int c = j; c < n; ++c) {
      double dot = 0.0;
      for (int i = j; i < n; ++i) dot += V[(size_t)i * n + j] * A[(size_t)i * n + c];
      dot *= beta[j];
      for (int i = j; i < n; ++i) A[(size_t)i * n + c] -= dot * V[(size_t)i * n + j];
    }
  }
  // Q = H_0 H_1 ... H_{n-1} applied to the identity (right to left)
  Q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  for (int j = n - 1; j >= 0; --j) {
    if (beta[j] == 0.0) continue;
    for (int c = 0; c < n; ++c) {
      double dot = 0.0;
      for (int i = j; i < n; ++i) dot += V[(size_t)i * n + j] * Q[(size_t)i * n + c];
      dot *= beta[j];
      for (int i = j; i < n; ++i) Q[(size_t)i * n + c] -= dot * V[(size_t)i * n + j];
    }
  }
  // sign fix: make diag(R) positive
  for (int j = 0; j < n; ++j) {
    if (A[(size_t)j * n + j] < 0.0)
      for (int i = 0; i < n; ++i) Q[(size_t)i * n + j] = -Q[(size_t)i * n + j];
  }
}

// ---------------------------------------------------------------- law

struct BetaLaw {
  double a;        // (d-1)/2
  double logB;     // log B(1/2, a)
  double logBaa;   // log B(a, a)
  explicit BetaLaw(int d) : a(0.5 * (d - 1)) {
    logB = std::lgamma(0.5) + std::lgamma(a) - std::lgamma(a + 0.5);
    logBaa = 2.0 * std::lgamma(a) - std::lgamma(2.0 * a);
  }
  // continued fraction of I_x(a, a) / (x^a (1-x)^a / (a B(a,a)))
  double cf(double x) const {
    const double tiny = 1e-300;
    const double b = a;
    double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
    if (std::fabs(dd) < tiny) dd = tiny;
    dd = 1.0 / dd;
    double h = dd;
    for (int m = 1; m <= 20000; ++m) {
      double m2 = 2.0 * m;
      double num = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
      dd = 1.0 + num * dd; if (std::fabs(dd) < tiny) dd = tiny;
      c = 1.0 + num / c;   if (std::fabs(c) < tiny) c = tiny;
      dd = 1.0 / dd; h *= dd * c;
      num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
      dd = 1.0 + num * dd; if (std::fabs(dd) < tiny) dd = tiny;
      c = 1.0 + num / c;   if (std::fabs(c) < tiny) c = tiny;
      dd = 1.0 / dd;
      double del = dd * c;
      h *= del;
      if (std::fabs(del - 1.0) < 1e-16) break;
    }
    return h;
  }
  // P(Y <= y) for y in [-1, 0]: x = (1+y)/2 in [0, 1/2], where the
  // continued fraction converges directly.
  double cdf_lower(double y) const {
    if (y <= -1.0) return 0.0;
    double x = 0.5 * (1.0 + y);
    double lx = std::log(x), l1x = std::log1p(-x);
    double pre = std::exp(a * lx + a * l1x - logBaa) / a;
    return pre * cf(x);
  }
  double density(double y) const {
    if (std::fabs(y) >= 1.0) return (a == 1.0) ? std::exp(-logB) : 0.0;
    return std::exp((a - 1.0) * std::log1p(-y * y) - logB);
  }
  // int_u^v y f(y) dy for -1 <= u < v <= 0
  double moment(double u, double v) const {
    double au = (u <= -1.0) ? -INFINITY : a * std::log1p(-u * u);
    double av = a * std::log1p(-v * v);
    return std::exp(av) * std::expm1(au - av) / (2.0 * a * std::exp(logB));
  }
};

// centroids of the lower-half cells [t[k], t[k+1]], t[0] = -1, t[h] = 0
void half_centroids(const BetaLaw& law, const std::vector<double>& t, std::vector<double>& c,
                    std::vector<double>& mass) {
  const int h = (int)t.size() - 1;
  std::vector<double> F(h + 1);
  for (int k = 0; k <= h; ++k) F[k] = law.cdf_lower(t[k]);
  for (int k = 0; k < h; ++k) {
    mass[k] = F[k + 1] - F[k];
    c[k] = law.moment(t[k], t[k + 1]) / mass[k];
  }
}

// ---------------------------------------------------------------- polar angles

// Gauss-Legendre nodes and weights on [-1, 1]: roots of P_n by Newton's
// method from the Chebyshev-like start cos(pi (i + 3/4) / (n + 1/2)),
// P_n and P_n' by the three-term recurrence; w = 2 / ((1 - x^2) P_n'(x)^2).
void gauss_legendre(int n, std::vector<double>& x, std::vector<double>& w) {
  x.assign(n, 0.0);
  w.assign(n, 0.0);
  const double pi = std::acos(-1.0);
  for (int i = 0; i < (n + 1) / 2; ++i) {
    double z = std::cos(pi * (i + 0.75) / (n + 0.5)), dp = 0.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    x[i] = -z;
    x[n - 1 - i] = z;
    w[i] = w[n - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

// Law of a level-l angle psi in [0, pi/2] (k = 2^(l-1) pooled coordinates):
// sin^2(psi) ~ Beta(k/2, k/2), density 2 sin^(k-1) cos^(k-1) / B(k/2, k/2).
// Cell masses on the lower half [0, pi/4] come from the incomplete beta of
// sin^2 (the coordinate law's continued fraction with a = k/2, i.e. its
// "d" = k + 1, at y = -cos 2 psi); first moments by composite Gauss-Legendre
// (panels of at most 0.02 rad, 24 nodes each).
struct AngleLaw {
  int k;
  BetaLaw beta;
  double logB;
  std::vector<double> gx, gw;
  explicit AngleLaw(int kk) : k(kk), beta(kk + 1) {
    logB = 2.0 * std::lgamma(0.5 * k) - std::lgamma((double)k);
    gauss_legendre(24, gx, gw);
  }
  double density(double p) const {
    const double s = std::sin(p), c = std::cos(p);
    if (s <= 0.0 || c <= 0.0) return (k == 1) ? std::exp(std::log(2.0) - logB) : 0.0;
    return std::exp(std::log(2.0) + (k - 1) * (std::log(s) + std::log(c)) - logB);
  }
  double cdf_lower(double p) const {           // p in [0, pi/4]
    if (p <= 0.0) return 0.0;
    return beta.cdf_lower(-std::cos(2.0 * p));
  }
  double moment(double u, double v) const {
    const int panels = std::max(1, (int)std::ceil((v - u) / 0.02));
    const double hw = 0.5 * (v - u) / panels;
    double acc = 0.0;
    for (int q = 0; q < panels; ++q) {
      const double mid = u + (2 * q + 1) * hw;
      for (size_t i = 0; i < gx.size(); ++i) {
        const double p = mid + hw * gx[i];
        acc += gw[i] * p * density(p);
      }
    }
    return acc * hw;
  }
};

// Lloyd-Max for one higher-level angle law with L = 2^bits levels:
// symmetric about pi/4, solved on [0, pi/4] by Lloyd steps from the
// quantile start, then Newton on the midpoint residual (as the coordinate
// codebook).
bool angle_lloyd_max(int k, int bits, std::vector<double>& cent, std::vector<double>& bnd, std::string& err) {
  const int L = 1 << bits, h = L / 2;
  const double mid = std::acos(-1.0) / 4.0;
  AngleLaw law(k);
  std::vector<double> t(h + 1), c(h), mass(h);
  t[0] = 0.0;
  t[h] = mid;
  auto centroids = [&](const std::vector<double>& tt, std::vector<double>& cc) {
    std::vector<double> F(h + 1);
    for (int j = 0; j <= h; ++j) F[j] = law.cdf_lower(tt[j]);
    for (int j = 0; j < h; ++j) {
      mass[j] = F[j + 1] - F[j];
      cc[j] = law.moment(tt[j], tt[j + 1]) / mass[j];
    }
  };
  for (int j = 0; j < h; ++j) {
    const double target = (j + 0.5) / L;
    double lo = 0.0, hi = mid;
    for (int it = 0; it < 200 && hi - lo > 1e-15; ++it) {
      const double m = 0.5 * (lo + hi);
      if (law.cdf_lower(m) < target) lo = m; else hi = m;
    }
    c[j] = 0.5 * (lo + hi);
  }
  for (int it = 0; it < g_lloyd_iters; ++it) {
    for (int j = 1; j < h; ++j) t[j] = 0.5 * (c[j - 1] + c[j]);
    std::vector<double> cn(h);
    centroids(t, cn);
    double step = 0.0;
    for (int j = 0; j < h; ++j) step = std::fmax(step, std::fabs(cn[j] - c[j]));
    c.swap(cn);
    if (step <= 1e-7) break;
  }
  if (h > 1) {
    const int n = h - 1;
    for (int j = 1; j < h; ++j) t[j] = 0.5 * (c[j - 1] + c[j]);
    double best = INFINITY;
    std::vector<double> best_t(t);
    for (int it = 0; it < g_newton_iters; ++it) {
      centroids(t, c);
      std::vector<double> R(n);
      double rmax = 0.0;
      for (int j = 1; j < h; ++j) {
        R[j - 1] = t[j] - 0.5 * (c[j - 1] + c[j]);
        rmax = std::fmax(rmax, std::fabs(R[j - 1]));
      }
      if (rmax < best) { best = rmax; best_t = t; } else { break; }
      if (rmax == 0.0) break;
      std::vector<double> dl(h), dr(h);
      for (int j = 0; j < h; ++j) {
        dl[j] = law.density(t[j]) * (c[j] - t[j]) / mass[j];
        dr[j] = law.density(t[j + 1]) * (t[j + 1] - c[j]) / mass[j];
      }
      std::vector<double> sub(n), dia(n), sup(n), rhs(R);
      for (int i = 0; i < n; ++i) {
        const int j = i + 1;
        dia[i] = 1.0 - 0.5 * (dr[j - 1] + dl[j]);
        sub[i] = (i > 0) ? -0.5 * dl[j - 1] : 0.0;
        sup[i] = (i < n - 1) ? -0.5 * dr[j] : 0.0;
      }
      for (int i = 1; i < n; ++i) {
        const double wv = sub[i] / dia[i - 1];
        dia[i] -= wv * sup[i - 1];
        rhs[i] -= wv * rhs[i - 1];
      }
      std::vector<double> dt(n);
      dt[n - 1] = rhs[n - 1] / dia[n - 1];
      for (int i = n - 2; i >= 0; --i) dt[i] = (rhs[i] - sup[i] * dt[i + 1]) / dia[i];
      for (int i = 0; i < n; ++i) t[i + 1] -= dt[i];
    }
    t = best_t;
    centroids(t, c);
    if (!(best < 1e-12)) {
      err = "angle Lloyd-Max did not converge (midpoint residual " + std::to_string(best) + ")";
      return false;
    }
  } else {
    centroids(t, c);
  }
  cent.assign(L, 0.0);
  bnd.assign(L - 1, 0.0);
  for (int j = 0; j < h; ++j) {
    cent[j] = c[j];
    cent[L - 1 - j] = 2.0 * mid - c[j];
  }
  for (int j = 0; j < L - 1; ++j) bnd[j] = 0.5 * (cent[j] + cent[j + 1]);
  bnd[h - 1] = mid;
  return true;
}

}  // namespace

void set_solver_limits(int lloyd_iters, int newton_iters) {
  g_lloyd_iters = lloyd_iters > 0 ? lloyd_iters : kLloydDefault;
  g_newton_iters = newton_iters > 0 ? newton_iters : kNewtonDefault;
}

bool build_codebook_host(const tq_params& p, HostCodebook& out, std::string& err) {
  const int d = p.d, bits = p.bits, m = p.qjl_m;
  const int L = 1 << bits, h = L / 2;
  BetaLaw law(d);

  // ---- Lloyd-Max on the lower half
  std::vector<double> t(h + 1), c(h), mass(h);
  t[0] = -1.0; t[h] = 0.0;
  // start: centroids at the quantiles (k + 1/2)/L of the law (bisection)
  for (int k = 0; k < h; ++k) {
    double target = (k + 0.5) / L, lo = -1.0, hi = 0.0;
    for (int it = 0; it < 200 && hi - lo > 1e-15; ++it) {
      double mid = 0.5 * (lo + hi);
      if (law.cdf_lower(mid) < target) lo = mid; else hi = mid;
    }
    c[k] = 0.5 * (lo + hi);
  }
  for (int it = 0; it < g_lloyd_iters; ++it) {
    for (int k = 1; k < h; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    std::vector<double> cn(h);
    half_centroids(law, t, cn, mass);
    double step = 0.0;
    for (int k = 0; k < h; ++k) step = std::fmax(step, std::fabs(cn[k] - c[k]));
    c.swap(cn);
    if (step <= 1e-7) break;
  }
  if (h > 1) {
    // Newton on R_k = t_k - (c_{k-1}(t) + c_k(t))/2, k = 1..h-1
    const int n = h - 1;
    for (int k = 1; k < h; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double best = INFINITY;
    std::vector<double> best_t(t);
    for (int it = 0; it < g_newton_iters; ++it) {
      half_centroids(law, t, c, mass);
      std::vector<double> R(n);
      double rmax = 0.0;
      for (int k = 1; k < h; ++k) {
        R[k - 1] = t[k] - 0.5 * (c[k - 1] + c[k]);
        rmax = std::fmax(rmax, std::fabs(R[k - 1]));
      }
      if (rmax < best) { best = rmax; best_t = t; } else { break; }
      if (rmax == 0.0) break;
      // derivatives of the cell centroids w.r.t. their edges
      std::vector<double> dl(h), dr(h);
      for (int k = 0; k < h; ++k) {
        dl[k] = law.density(t[k]) * (c[k] - t[k]) / mass[k];
        dr[k] = law.density(t[k + 1]) * (t[k + 1] - c[k]) / mass[k];
      }
      // tridiagonal system J dt = R
      std::vector<double> sub(n), dia(n), sup(n), rhs(R);
      for (int i = 0; i < n; ++i) {
        const int k = i + 1;
        dia[i] = 1.0 - 0.5 * (dr[k - 1] + dl[k]);
        sub[i] = (i > 0) ? -0.5 * dl[k - 1] : 0.0;
        sup[i] = (i < n - 1) ? -0.5 * dr[k] : 0.0;
      }
      for (int i = 1; i < n; ++i) {
        double w = sub[i] / dia[i - 1];
        dia[i] -= w * sup[i - 1];
        rhs[i] -= w * rhs[i - 1];
      }
      std::vector<double> dt(n);
      dt[n - 1] = rhs[n - 1] / dia[n - 1];
      for (int i = n - 2; i >= 0; --i) dt[i] = (rhs[i] - sup[i] * dt[i + 1]) / dia[i];
      for (int i = 0; i < n; ++i) t[i + 1] -= dt[i];
    }
    t = best_t;
    half_centroids(law, t, c, mass);
    if (!(best < 1e-12)) {
      err = "Lloyd-Max did not converge (midpoint residual " + std::to_string(best) + ")";
      return false;
    }
  } else {
    half_centroids(law, t, c, mass);
  }
  out.centroids.assign(L, 0.0);
  out.boundaries.assign(L - 1, 0.0);
  for (int k = 0; k < h; ++k) {
    out.centroids[k] = c[k];
    out.centroids[L - 1 - k] = -c[k];
  }
  for (int k = 0; k < L - 1; ++k) out.boundaries[k] = 0.5 * (out.centroids[k] + out.centroids[k + 1]);
  out.boundaries[h - 1] = 0.0;
  for (int k = 0; k < L; ++k) {
    if (!std::isfinite(out.centroids[k])) { err = "non-finite centroid"; return false; }
  }

  // ---- rotation and sketch
  std::vector<double> G((size_t)d * d);
  gaussian_fill(p.rot_seed, G);
  householder_q(d, G, out.rot);
  out.qjl.clear();
  if (m > 0) {
    out.qjl.resize((size_t)m * d);
    gaussian_fill(p.qjl_seed, out.qjl);
  }
  return true;
}

bool build_polar_codebook_host(const tq_polar_params& p, HostCodebook& out, std::vector<int>& cent_off,
                               std::vector<int>& bnd_off, std::string& err) {
  const int d = p.d, m = p.qjl_m;
  int levels = 0;
  while ((2 << levels) <= d) ++levels;
  const double pi = std::acos(-1.0);
  out.centroids.clear();
  out.boundaries.clear();
  cent_off.assign(levels + 2, 0);
  bnd_off.assign(levels + 2, 0);
  for (int lv = 1; lv <= levels; ++lv) {
    const int bits = lv == 1 ? p.bits_first : p.bits_rest;
    const int L = 1 << bits;
    cent_off[lv] = (int)out.centroids.size();
    bnd_off[lv] = (int)out.boundaries.size();
    std::vector<double> c, t;
    if (lv == 1) {
      // uniform law on [-pi, pi]: equal cells, centroids at their centres
      const double w = 2.0 * pi / L;
      for (int j = 0; j < L; ++j) c.push_back(-pi + w * (j + 0.5));
      for (int j = 1; j < L; ++j) t.push_back(j == L / 2 ? 0.0 : -pi + w * j);
    } else if (!angle_lloyd_max(1 << (lv - 1), bits, c, t, err)) {
      return false;
    }
    out.centroids.insert(out.centroids.end(), c.begin(), c.end());
    out.boundaries.insert(out.boundaries.end(), t.begin(), t.end());
  }
  cent_off[levels + 1] = (int)out.centroids.size();
  bnd_off[levels + 1] = (int)out.boundaries.size();
  std::vector<double> G((size_t)d * d);
  gaussian_fill(p.rot_seed, G);
  householder_q(d, G, out.rot);
  out.qjl.clear();
  if (m > 0) {
    out.qjl.resize((size_t)m * d);
    gaussian_fill(p.qjl_seed, out.qjl);
  }
  return true;
}

}  // namespace tq
