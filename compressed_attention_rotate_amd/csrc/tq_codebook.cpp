// Host-side Lloyd-Max codebook builder.
//
// After the random rotation, each coordinate of a unit vector in R^d follows one fixed
// law (the marginal of a uniformly random point on the sphere), so a single scalar
// codebook per width is computed once and stored (163.com explainer,
// m.163.com/dy/article/KOV7P8JI0556C3J2, section "第一步：PolarQuant").  The density is
// f(t) = (1 - t^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1].
//
// Lloyd's conditions are iterated on the upper half of the (symmetric) codebook: each
// centroid is the conditional mean of its cell, each boundary the midpoint of adjacent
// centroids.  Cell masses come from composite Gauss-Legendre quadrature of f; first
// moments from the closed-form primitive of t f(t), -(1-t^2)^((d-1)/2) / ((d-1) B).
#include <cmath>
#include <cstdint>
#include <vector>

#include "tq.h"

namespace {

struct GaussLegendre {
  static constexpr int N = 24;
  double x[N], w[N];
  GaussLegendre() {
    // nodes by Newton iteration on P_N, starting from the Chebyshev-like guesses
    for (int i = 0; i < N; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (N + 0.5));
      double dp = 1.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = 0.0;
        for (int k = 1; k <= N; ++k) {
          double p2 = p1;
          p1 = p0;
          p0 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p2) / k;
        }
        dp = N * (z * p0 - p1) / (z * z - 1.0);
        double dz = p0 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-15) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

struct Marginal {
  int d;
  double a;       // (d - 1) / 2
  double log_b;   // log B(1/2, (d-1)/2)
  double panel;   // quadrature panel width
  const GaussLegendre* gl;

  Marginal(int d_, const GaussLegendre* g) : d(d_), gl(g) {
    a = (d - 1) / 2.0;
    log_b = std::lgamma(0.5) + std::lgamma(a) - std::lgamma(a + 0.5);
    panel = std::fmin(1.0 / 32.0, 0.25 / std::sqrt((double)d));
  }
  double pdf(double t) const {
    return std::exp((a - 1.0) * std::log1p(-t * t) - log_b);
  }
  double mass(double lo, double hi) const {  // integral of pdf over [lo, hi]
    int np = (int)std::ceil((hi - lo) / panel);
    if (np < 1) np = 1;
    double h = (hi - lo) / np, s = 0.0;
    for (int p = 0; p < np; ++p) {
      double mid = lo + (p + 0.5) * h, part = 0.0;
      for (int i = 0; i < GaussLegendre::N; ++i) part += gl->w[i] * pdf(mid + 0.5 * h * gl->x[i]);
      s += 0.5 * h * part;
    }
    return s;
  }
  double prim_t(double t) const {  // primitive of t * pdf(t)
    if (std::fabs(t) >= 1.0) return 0.0;
    return -std::exp(a * std::log1p(-t * t) - log_b) / (d - 1);
  }
  double moment1(double lo, double hi) const { return prim_t(hi) - prim_t(lo); }
};

}  // namespace

extern "C" int tq_build_codebook(int32_t d, int32_t bits, float* centroids, float* bounds,
                                 double* mse) {
  if (!centroids || !bounds) return TQ_ERR_ARG;
  if (d < 8 || d > 4096 || (d & (d - 1)) || bits < 1 || bits > 4) return TQ_ERR_SHAPE;
  static const GaussLegendre gl;
  Marginal f(d, &gl);
  const int L = 1 << bits, H = L / 2;
  std::vector<double> c(H), nc(H), e(H + 1);
  const double sc = 1.0 / std::sqrt((double)d);
  for (int m = 0; m < H; ++m) c[m] = (m + 0.5) * 3.0 * sc / H;  // ordered start
  bool converged = false;
  for (int it = 0; it < 500000 && !converged; ++it) {
    e[0] = 0.0;
    e[H] = 1.0;
    for (int m = 1; m < H; ++m) e[m] = 0.5 * (c[m - 1] + c[m]);
    double delta = 0.0;
    for (int m = 0; m < H; ++m) {
      nc[m] = f.moment1(e[m], e[m + 1]) / f.mass(e[m], e[m + 1]);
      delta = std::fmax(delta, std::fabs(nc[m] - c[m]));
    }
    c.swap(nc);
    converged = delta < 1e-13;
  }
  if (!converged) return TQ_ERR_NOCONV;
  std::vector<double> full(L);
  for (int m = 0; m < H; ++m) {
    full[H + m] = c[m];
    full[H - 1 - m] = -c[m];
  }
  for (int m = 0; m < L; ++m) centroids[m] = (float)full[m];
  for (int m = 0; m + 1 < L; ++m) bounds[m] = (float)(0.5 * (full[m] + full[m + 1]));
  if (mse) {
    double s = 0.0, lo = -1.0;
    for (int m = 0; m < L; ++m) {
      double hi = (m + 1 < L) ? 0.5 * (full[m] + full[m + 1]) : 1.0;
      s += full[m] * full[m] * f.mass(lo, hi);
      lo = hi;
    }
    *mse = 1.0 / d - s;
  }
  return TQ_OK;
}
