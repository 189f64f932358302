// Lloyd-Max codebook for one coordinate of a uniform random unit vector in
// R^d (host, fp64).
//
// After the random rotation of stage 1 ("TurboQuantとは？仕組み・実測精度・
// 2026年7月時点の実装状況", 第1段: randomized Hadamard rotation, then
// per-coordinate Lloyd-Max) each coordinate of a unit vector has density
// f_d(x) proportional to (1 - x^2)^((d-3)/2) on [-1, 1], whatever the data;
// the codebook therefore depends on (d, bits) alone (same page,
// キャリブレーション不要が効く場面).
//
// Solver: Lloyd's two conditions (thresholds at midpoints, centroids at
// conditional means) iterated to their fixed point, on the positive half of
// the symmetric codebook. Cell integrals use the substitution x = sin(theta),
// which turns (1 - x^2)^((d-3)/2) dx into cos(theta)^(d-2) dtheta, a smooth
// integrand, and composite Gauss-Legendre quadrature. The normalising
// constant cancels in every conditional mean.
#include <algorithm>
#include <cmath>
#include <vector>

namespace tq {

namespace {

struct GaussLegendre {
  static constexpr int N = 20;
  double x[N], w[N];
  GaussLegendre() {
    // nodes = roots of P_N by Newton from the Chebyshev-like initial guess
    for (int i = 0; i < N; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (N + 0.5));
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= N; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        const double dp = N * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-17) break;
      }
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= N; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      const double dp = N * (z * p1 - p0) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre &gl() {
  static const GaussLegendre g;
  return g;
}

// Integrals over theta in [a, b] of cos^m and sin * cos^m: Gauss-Legendre
// panels at the resolution of 24 panels over [0, pi/2] (at least one).
void cell_integrals(double a, double b, int m, double &mass, double &moment) {
  const GaussLegendre &g = gl();
  const int panels = std::max(1, static_cast<int>(std::ceil(24.0 * (b - a) / (0.5 * M_PI) - 1e-9)));
  mass = 0.0;
  moment = 0.0;
  const double h = (b - a) / panels;
  for (int pi = 0; pi < panels; ++pi) {
    const double lo = a + pi * h;
    const double mid = lo + 0.5 * h;
    for (int k = 0; k < GaussLegendre::N; ++k) {
      const double th = mid + 0.5 * h * g.x[k];
      const double c = std::cos(th);
      const double f = (m == 0) ? 1.0 : std::pow(c > 0.0 ? c : 0.0, m);
      mass += 0.5 * h * g.w[k] * f;
      moment += 0.5 * h * g.w[k] * f * std::sin(th);
    }
  }
}

}  // namespace

// Fills the fp64 positive-half fixed point; returns false if the iteration
// fails to settle.
bool lloyd_max_positive_half(int d, int bits, std::vector<double> &c) {
  const int L = 1 << bits;
  const int H = L / 2;
  const int m = d - 2;
  c.assign(H, 0.0);
  // start: the positive half's quantiles of f_d itself, P(0 < X < c_k) =
  // (k + 1/2) / H of P(X > 0), by bisection on the cell mass: strictly
  // increasing and inside (0, 1) for every d and width
  double half_mass, unused;
  cell_integrals(0.0, 0.5 * M_PI, m, half_mass, unused);
  for (int k = 0; k < H; ++k) {
    const double target = (k + 0.5) / H * half_mass;
    double lo = 0.0, hi = 1.0;
    for (int it = 0; it < 64; ++it) {
      const double mid = 0.5 * (lo + hi);
      double mass;
      cell_integrals(0.0, std::asin(mid), m, mass, unused);
      if (mass < target) lo = mid; else hi = mid;
    }
    c[k] = 0.5 * (lo + hi);
  }
  std::vector<double> nc(H);
  double prev = 1.0;
  for (int it = 0; it < 400000; ++it) {
    double delta = 0.0;
    for (int k = 0; k < H; ++k) {
      const double x0 = (k == 0) ? 0.0 : 0.5 * (c[k - 1] + c[k]);
      const double x1 = (k == H - 1) ? 1.0 : 0.5 * (c[k] + c[k + 1]);
      double mass, moment;
      cell_integrals(std::asin(x0), std::asin(x1), m, mass, moment);
      nc[k] = (mass > 0.0) ? moment / mass : c[k];      // (an empty cell keeps its centroid)
      delta = std::fmax(delta, std::fabs(nc[k] - c[k]));
    }
    c.swap(nc);
    if (delta < 5e-16 || (delta < 1e-14 && delta >= prev)) return true;
    prev = delta;
  }
  return false;
}

}  // namespace tq
