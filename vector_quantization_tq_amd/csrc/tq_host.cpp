// Host-side precompute for libtq: random streams, the rotation, the QJL
// matrix and the Lloyd-Max codebooks.  Pure C++ (libm only); no GPU calls.
//
// Method references (page site, title, section):
//   rotation by QR of a Gaussian matrix: a2a-mcp.org "什麼是TurboQuant？",
//     stage 1 (random orthogonal rotation);
//   rotated-coordinate law and Lloyd-Max codebooks: same section, and
//     blog.hotdry.top "TurboQuant vector-search compression", section on
//     random rotation + scalar quantisation;
//   Gaussian QJL matrix: blog.hotdry.top, QJL residual correction section.
#include "tq_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

namespace tq {

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood 2014): output k of a stream started at
// state s is mix(s + (k+1) * gamma).  Uniforms from the top 53 bits plus half
// a unit; normals by Box-Muller on consecutive pairs.
// ---------------------------------------------------------------------------
static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void normals(uint64_t seed, int tag, int64_t n, double* out) {
  const uint64_t gamma = 0x9E3779B97F4A7C15ull;
  const uint64_t state = seed ^ (static_cast<uint64_t>(tag) << 56);
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t p = 0; 2 * p < n; ++p) {
    uint64_t z1 = mix64(state + static_cast<uint64_t>(2 * p + 1) * gamma);
    uint64_t z2 = mix64(state + static_cast<uint64_t>(2 * p + 2) * gamma);
    double u1 = (static_cast<double>(z1 >> 11) + 0.5) * 0x1.0p-53;
    double u2 = (static_cast<double>(z2 >> 11) + 0.5) * 0x1.0p-53;
    double r = std::sqrt(-2.0 * std::log(u1));
    out[2 * p] = r * std::cos(two_pi * u2);
    if (2 * p + 1 < n) out[2 * p + 1] = r * std::sin(two_pi * u2);
  }
}

// d random signs: output i of stream (seed, 3) gives -1 when its top bit is
// set, +1 otherwise.
void signs(uint64_t seed, int d, double* out) {
  const uint64_t gamma = 0x9E3779B97F4A7C15ull;
  const uint64_t state = seed ^ (static_cast<uint64_t>(3) << 56);
  for (int i = 0; i < d; ++i) out[i] = (mix64(state + static_cast<uint64_t>(i + 1) * gamma) >> 63) ? -1.0 : 1.0;
}

// Structured rotation Pi = H D / sqrt(d) (ai-coding.wiselychen.com, "Google
// TurboQuant：KV Cache 壓縮 6x…", community implementation section: a
// Walsh-Hadamard rotation): H the Sylvester-Hadamard matrix,
// H[i][j] = (-1)^popcount(i & j), D = diag(signs).  d a power of two.
void rotation_hadamard(int d, uint64_t seed, double* pi) {
  std::vector<double> sg(d);
  signs(seed, d, sg.data());
  const double inv = 1.0 / std::sqrt(static_cast<double>(d));
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      pi[static_cast<size_t>(i) * d + j] = ((__builtin_popcount(static_cast<unsigned>(i & j)) & 1) ? -sg[j] : sg[j]) * inv;
}

// ---------------------------------------------------------------------------
// Householder QR of G (d x d, row major).  Returns Q with the column signs
// chosen so that R has a positive diagonal (the unique such factor).
// ---------------------------------------------------------------------------
void rotation(int d, uint64_t seed, double* pi) {
  std::vector<double> a(static_cast<size_t>(d) * d);
  normals(seed, 1, static_cast<int64_t>(d) * d, a.data());
  std::vector<double> vs(static_cast<size_t>(d) * d, 0.0);  // Householder vectors, column k in row k of vs
  std::vector<double> rdiag(d);
  auto A = [&](int i, int j) -> double& { return a[static_cast<size_t>(i) * d + j]; };
  for (int k = 0; k < d; ++k) {
    double norm = 0;
    for (int i = k; i < d; ++i) norm += A(i, k) * A(i, k);
    norm = std::sqrt(norm);
    double alpha = A(k, k) > 0 ? -norm : norm;   // reflect onto -sign(x0) ||x|| e1
    double* v = &vs[static_cast<size_t>(k) * d];
    for (int i = k; i < d; ++i) v[i] = A(i, k);
    v[k] -= alpha;
    double vn = 0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    vn = std::sqrt(vn);
    if (vn > 0)
      for (int i = k; i < d; ++i) v[i] /= vn;
    for (int j = k; j < d; ++j) {
      double s = 0;
      for (int i = k; i < d; ++i) s += v[i] * A(i, j);
      for (int i = k; i < d; ++i) A(i, j) -= 2.0 * v[i] * s;
    }
    rdiag[k] = A(k, k);
  }
  // Q = H_0 H_1 ... H_{d-1} applied to the identity, right to left.
  std::vector<double> q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[static_cast<size_t>(i) * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &vs[static_cast<size_t>(k) * d];
    for (int j = 0; j < d; ++j) {
      double s = 0;
      for (int i = k; i < d; ++i) s += v[i] * q[static_cast<size_t>(i) * d + j];
      for (int i = k; i < d; ++i) q[static_cast<size_t>(i) * d + j] -= 2.0 * v[i] * s;
    }
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) pi[static_cast<size_t>(i) * d + j] = q[static_cast<size_t>(i) * d + j] * (rdiag[j] < 0 ? -1.0 : 1.0);
}

void qjl_matrix(int m, int d, uint64_t seed, double* s) { normals(seed, 2, static_cast<int64_t>(m) * d, s); }

// ---------------------------------------------------------------------------
// Lloyd-Max for the density w(x) = (1-x^2)^((d-3)/2) on [-1, 1] (unnormalised;
// only ratios enter).  Cell masses and first moments by composite
// Gauss-Legendre quadrature; the fixed point c = E[X | cell(c)] is solved by
// Newton's method on the centroid conditions (the Jacobian is tridiagonal),
// started from a few plain Lloyd iterations.
// ---------------------------------------------------------------------------
namespace {

struct GaussLegendre {
  static constexpr int N = 24;
  double x[N], w[N];
  GaussLegendre() {
    for (int i = 0; i < N; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (N + 0.5));
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= N; ++k) {
          double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        double dp = N * (z * p1 - p0) / (z * z - 1.0);
        double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= N; ++k) {
        double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      double dp = N * (z * p1 - p0) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre& gl() {
  static GaussLegendre g;
  return g;
}

struct Law {
  int d;
  double e;  // exponent (d-3)/2
  double panel;
  explicit Law(int d_) : d(d_), e((d_ - 3) / 2.0) { panel = std::min(0.125, 0.25 / std::sqrt(e + 1.0)); }
  double w(double x) const {
    double t = 1.0 - x * x;
    return t <= 0 ? 0.0 : (e == 0 ? 1.0 : std::pow(t, e));
  }
  // mass and first moment over [a, b], with x = sin(phi): w dx = cos^(d-2) phi dphi,
  // an analytic integrand for every d, so Gauss-Legendre converges fast.
  void integrate(double a, double b, double& m0, double& m1) const {
    m0 = m1 = 0;
    if (b <= a) return;
    double pa = std::asin(std::max(-1.0, std::min(1.0, a)));
    double pb = std::asin(std::max(-1.0, std::min(1.0, b)));
    int np = std::max(1, static_cast<int>(std::ceil((pb - pa) / panel)));
    double h = (pb - pa) / np;
    const GaussLegendre& g = gl();
    for (int p = 0; p < np; ++p) {
      double mid = pa + (p + 0.5) * h;
      for (int i = 0; i < GaussLegendre::N; ++i) {
        double phi = mid + 0.5 * h * g.x[i];
        double cs = std::cos(phi);
        double f = g.w[i] * 0.5 * h * (d == 2 ? 1.0 : std::pow(cs, d - 2));
        m0 += f;
        m1 += f * std::sin(phi);
      }
    }
  }
};

void cell_means(const Law& law, const std::vector<double>& c, std::vector<double>& mean, std::vector<double>& mass) {
  int K = static_cast<int>(c.size());
  for (int k = 0; k < K; ++k) {
    double a = k == 0 ? -1.0 : 0.5 * (c[k - 1] + c[k]);
    double b = k == K - 1 ? 1.0 : 0.5 * (c[k] + c[k + 1]);
    double m0, m1;
    law.integrate(a, b, m0, m1);
    mass[k] = m0;
    mean[k] = m1 / m0;
  }
}

}  // namespace

int codebook(int d, int K, double* centroids, double* thresholds) {
  if (d < 3 || K < 2 || K > 256) return -1;
  Law law(d);
  // start: equal-mass cells of the Gaussian approximation N(0, 1/d), clipped
  std::vector<double> c(K), mean(K), mass(K);
  double sd = 1.0 / std::sqrt(static_cast<double>(d));
  for (int k = 0; k < K; ++k) {
    double p = (k + 0.5) / K;
    // inverse normal CDF by bisection on erfc
    double lo = -10, hi = 10;
    for (int it = 0; it < 200; ++it) {
      double mid = 0.5 * (lo + hi);
      if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
    }
    c[k] = std::max(-0.999, std::min(0.999, 0.5 * (lo + hi) * sd));
  }
  for (int it = 0; it < 20; ++it) {
    cell_means(law, c, mean, mass);
    c = mean;
  }
  // Newton on F(c) = c - g(c), g = cell means; dg_k/dt = w(t)(t - g_k)/mass_k
  for (int it = 0; it < 60; ++it) {
    cell_means(law, c, mean, mass);
    std::vector<double> F(K), lo(K, 0.0), di(K, 1.0), up(K, 0.0);
    double fmax = 0;
    for (int k = 0; k < K; ++k) {
      F[k] = c[k] - mean[k];
      fmax = std::max(fmax, std::fabs(F[k]));
    }
    for (int k = 0; k < K; ++k) {
      if (k + 1 < K) {   // threshold t_k between c_k and c_{k+1} (upper edge of cell k)
        double t = 0.5 * (c[k] + c[k + 1]);
        double dg = law.w(t) * (t - mean[k]) / mass[k];       // d g_k / d t
        di[k] -= 0.5 * dg;
        up[k] -= 0.5 * dg;
      }
      if (k > 0) {       // lower edge of cell k
        double t = 0.5 * (c[k - 1] + c[k]);
        double dg = -law.w(t) * (t - mean[k]) / mass[k];
        di[k] -= 0.5 * dg;
        lo[k] -= 0.5 * dg;
      }
    }
    // Thomas algorithm for the tridiagonal system J dx = F
    std::vector<double> cp(K), dp(K);
    cp[0] = up[0] / di[0];
    dp[0] = F[0] / di[0];
    for (int k = 1; k < K; ++k) {
      double den = di[k] - lo[k] * cp[k - 1];
      cp[k] = up[k] / den;
      dp[k] = (F[k] - lo[k] * dp[k - 1]) / den;
    }
    std::vector<double> dx(K);
    dx[K - 1] = dp[K - 1];
    for (int k = K - 2; k >= 0; --k) dx[k] = dp[k] - cp[k] * dx[k + 1];
    double step = 0;
    for (int k = 0; k < K; ++k) {
      c[k] -= dx[k];
      step = std::max(step, std::fabs(dx[k]));
    }
    if (step <= 1e-16 * sd && it >= 2) break;
  }
  // symmetrise: the law is symmetric and the fixed point unique
  for (int k = 0; k < K; ++k) centroids[k] = 0.5 * (c[k] - c[K - 1 - k]);
  for (int k = 0; k + 1 < K; ++k) thresholds[k] = 0.5 * (centroids[k] + centroids[k + 1]);
  if (K % 2 == 0) thresholds[K / 2 - 1] = 0.0;
  return 0;
}

}  // namespace tq
