// Host-side fp64 Lloyd-Max fitter for the marginal of a rotated coordinate.
//
// OrbitQuant page, Method: the rotated coordinates of a unit vector follow a
// fixed marginal f_d; Lloyd-Max is run on it offline to give one codebook per
// dimension.  Tables are in N(0,1) units (u = sqrt(d) x); the kernels apply
// the sqrt(d) scale.  Two marginals:
//   * N(0,1), the large-d limit (orbit_fit_codebook);
//   * the exact marginal of one coordinate T of a uniform direction on
//     S^{d-1}: f_d(t) = C_d (1 - t^2)^((d-3)/2), C_d = Gamma(d/2) /
//     (sqrt(pi) Gamma((d-1)/2)), so U = sqrt(d) T lives on [-sqrt d, sqrt d]
//     (orbit_fit_codebook_sphere).
// For u >= 0 the fitter needs the density g(u), the upper tail P(U > u) and
// the first-moment tail E[U; U > u]:
//   N(0,1):  phi(u), erfc(u / sqrt 2) / 2, phi(u);
//   sphere:  C_d / sqrt(d) (1 - t^2)^((d-3)/2),
//            (1 - I_{t^2}(1/2, (d-1)/2)) / 2   (T^2 ~ Beta(1/2, (d-1)/2)),
//            sqrt(d) C_d (1 - t^2)^((d-1)/2) / (d - 1),      t = u / sqrt(d).
// I_x(a, b) is the regularized incomplete beta function, evaluated with its
// continued fraction (DLMF 8.17.22) by the modified Lentz method, and through
// I_x(a, b) = 1 - I_{1-x}(b, a) past x = (a + 1) / (a + b + 2) (DLMF 8.17.4).
//
// Method: a few plain Lloyd alternations, then Newton's method on the
// interior thresholds.  With h = levels/2 positive cells
// 0 = tau_0 < tau_1 < ... < tau_{h-1} < tau_h = top and centroids
//   c_j = (M(tau_j) - M(tau_{j+1})) / (Q(tau_j) - Q(tau_{j+1}))
// (M the first-moment tail, Q the upper tail), the conditions
// G_j = tau_j - (c_{j-1} + c_j)/2 = 0 (j = 1..h-1) have a tridiagonal
// Jacobian from
//   dc_j/dtau_j = g(tau_j) (c_j - tau_j) / D_j,
//   dc_j/dtau_{j+1} = g(tau_{j+1}) (tau_{j+1} - c_j) / D_j,
// solved with the Thomas algorithm.  The negative half mirrors the positive
// one, so the table is exactly symmetric with a zero middle threshold.
#include <cmath>
#include <vector>

#include "orbit_internal.h"

namespace {

const double kInvSqrt2Pi = 0.3989422804014326779399460599343819;
const double kInvSqrt2 = 0.7071067811865475244008443621048490;

// 1 / (1 + d_1 / (1 + d_2 / (1 + ...))) for the incomplete beta fraction
// (DLMF 8.17.22): d_{2m} = m (b - m) x / ((a + 2m - 1)(a + 2m)),
// d_{2m+1} = -(a + m)(a + b + m) x / ((a + 2m)(a + 2m + 1)).  The fraction
// F = 1 + d_1 / (1 + d_2 / ...) is evaluated front to back by the modified
// Lentz method (Lentz 1976; Thompson and Barnett 1986): F_n = F_{n-1} C_n D_n
// with C_n = 1 + d_n / C_{n-1}, D_n = 1 / (1 + d_n D_{n-1}), zero
// denominators replaced by a tiny number, until C_n D_n is 1 to rounding.
// The fraction needs up to a few thousand terms near the switch point for
// large d; it runs in long double (64-bit significand on x86-64) so that the
// rounding its products accumulate stays below double precision.
long double beta_fraction(long double a, long double b, long double x) {
  const long double tiny = 1e-300L;
  long double F = 1.0L, C = 1.0L, D = 0.0L;
  for (int n = 1; n < 1000000; ++n) {
    const int m = n / 2;
    const long double dn = (n & 1) ? -(a + m) * (a + b + m) * x / ((a + 2.0L * m) * (a + 2.0L * m + 1.0L))
                                   : m * (b - m) * x / ((a + 2.0L * m - 1.0L) * (a + 2.0L * m));
    D = 1.0L + dn * D;
    if (fabsl(D) < tiny) D = tiny;
    C = 1.0L + dn / C;
    if (fabsl(C) < tiny) C = tiny;
    D = 1.0L / D;
    const long double delta = C * D;
    F *= delta;
    if (fabsl(delta - 1.0L) < 1e-19L) break;
  }
  return 1.0L / F;
}

struct Marginal {
  int d = 0;  // 0: N(0,1); >= 3: the sphere marginal of dimension d
  double top = INFINITY;
  long double log_c = 0;     // log C_d
  long double log_beta = 0;  // log B(1/2, (d-1)/2)

  static Marginal gaussian() { return Marginal(); }
  static Marginal sphere(int d) {
    Marginal m;
    m.d = d;
    m.top = std::sqrt((double)d);
    const long double half = 0.5L, b = 0.5L * (d - 1);
    m.log_c = lgammal(0.5L * d) - lgammal(b) - 0.5L * logl(3.141592653589793238462643383279502884L);
    m.log_beta = lgammal(half) + lgammal(b) - lgammal(half + b);
    return m;
  }

  double pdf(double u) const {
    if (d == 0) return std::isinf(u) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * u * u);
    if (u >= top) return 0.0;
    const long double t2 = (long double)u * u / d;
    return (double)(expl(log_c + 0.5L * (d - 3) * log1pl(-t2)) / top);
  }
  double tail(double u) const {  // P(U > u), u >= 0
    if (d == 0) return std::isinf(u) ? 0.0 : 0.5 * std::erfc(u * kInvSqrt2);
    if (u >= top) return 0.0;
    if (u <= 0.0) return 0.5;
    const long double x = (long double)u * u / d, a = 0.5L, b = 0.5L * (d - 1);
    // x^a (1-x)^b / B(a, b), formed in logs from x (never from 1 - x)
    const long double log_front = a * logl(x) + b * log1pl(-x) - log_beta;
    if (x < (a + 1.0L) / (a + b + 2.0L)) {
      const long double I = expl(log_front) / a * beta_fraction(a, b, x);
      return (double)(0.5L * (1.0L - I));
    }
    const long double J = expl(log_front) / b * beta_fraction(b, a, 1.0L - x);  // 1 - I_x(a, b)
    return (double)(0.5L * J);
  }
  double moment(double u) const {  // E[U; U > u], u >= 0
    if (d == 0) return pdf(u);
    if (u >= top) return 0.0;
    const long double t2 = (long double)u * u / d;
    return (double)(top * expl(log_c + 0.5L * (d - 1) * log1pl(-t2)) / (d - 1));
  }
};

// centroids of the positive cells for the given edges (tau has h+1 entries)
void centroids_of(const Marginal& f, const std::vector<double>& tau, std::vector<double>& c) {
  const size_t h = tau.size() - 1;
  for (size_t j = 0; j < h; ++j) {
    const double mass = f.tail(tau[j]) - f.tail(tau[j + 1]);
    c[j] = (f.moment(tau[j]) - f.moment(tau[j + 1])) / mass;
  }
}

orbit_status fit(const Marginal& f, int32_t d, int32_t bits, int32_t max_iter, double tol,
                 orbit_codebook* out, double* centroids_f64, double* thresholds_f64,
                 double* mse_f64) {
  if (max_iter <= 0) max_iter = 100;
  if (!(tol > 0)) tol = 1e-15;
  const int levels = 1 << bits;
  const int h = levels / 2;

  std::vector<double> tau(h + 1), c(h);
  // start: equally spaced thresholds on [0, span], inside the support
  tau[0] = 0.0;
  tau[h] = f.top;
  const double span = std::fmin(3.0 + 0.25 * bits, 0.9 * f.top);
  for (int j = 1; j < h; ++j) tau[j] = span * j / h;
  centroids_of(f, tau, c);
  // Lloyd alternations bring the start inside Newton's basin
  for (int it = 0; it < 200; ++it) {
    for (int j = 1; j < h; ++j) tau[j] = 0.5 * (c[j - 1] + c[j]);
    centroids_of(f, tau, c);
  }
  // Newton on G_j = tau_j - (c_{j-1} + c_j)/2
  std::vector<double> a(h), b(h), cc(h), rhs(h), dlo(h), dhi(h);
  for (int it = 0; it < max_iter && h > 1; ++it) {
    centroids_of(f, tau, c);
    for (int j = 0; j < h; ++j) {
      const double mass = f.tail(tau[j]) - f.tail(tau[j + 1]);
      dlo[j] = f.pdf(tau[j]) * (c[j] - tau[j]) / mass;  // dc_j/dtau_j
      // dc_j/dtau_{j+1}; the top edge is fixed, so j = h-1 never enters
      dhi[j] = j + 1 < h ? f.pdf(tau[j + 1]) * (tau[j + 1] - c[j]) / mass : 0.0;
    }
    // rows j = 1..h-1 of the tridiagonal system, stored at index j-1
    const int n = h - 1;
    for (int j = 1; j < h; ++j) {
      int r = j - 1;
      a[r] = (j > 1) ? -0.5 * dlo[j - 1] : 0.0;      // d/dtau_{j-1}
      b[r] = 1.0 - 0.5 * (dhi[j - 1] + dlo[j]);      // d/dtau_j
      cc[r] = (j < h - 1) ? -0.5 * dhi[j] : 0.0;     // d/dtau_{j+1}
      rhs[r] = -(tau[j] - 0.5 * (c[j - 1] + c[j]));
    }
    for (int r = 1; r < n; ++r) {  // Thomas forward sweep
      double m = a[r] / b[r - 1];
      b[r] -= m * cc[r - 1];
      rhs[r] -= m * rhs[r - 1];
    }
    rhs[n - 1] /= b[n - 1];
    for (int r = n - 2; r >= 0; --r) rhs[r] = (rhs[r] - cc[r] * rhs[r + 1]) / b[r];
    double step = 0.0;
    for (int j = 1; j < h; ++j) {
      tau[j] += rhs[j - 1];
      step = std::fmax(step, std::fabs(rhs[j - 1]));
    }
    if (step < tol) break;
  }
  centroids_of(f, tau, c);
  for (int j = 0; j < h; ++j)
    if (!std::isfinite(c[j]) || (j > 0 && !(c[j] > c[j - 1]))) return ORBIT_E_UNSUPPORTED;

  // E[U^2] = 1 for both marginals; at the centroid fixed point
  // D = 1 - sum_j p_j c_j^2
  double mse = 1.0;
  for (int j = 0; j < h; ++j) {
    double p = f.tail(tau[j]) - f.tail(tau[j + 1]);
    mse -= 2.0 * p * c[j] * c[j];
  }
  out->bits = bits;
  out->d = d;
  for (int i = 0; i < ORBIT_MAX_LEVELS; ++i) out->centroids[i] = 0.0f;
  for (int i = 0; i < ORBIT_MAX_LEVELS - 1; ++i) out->thresholds[i] = 0.0f;
  for (int j = 0; j < h; ++j) {
    out->centroids[h + j] = (float)c[j];
    out->centroids[h - 1 - j] = -(float)c[j];
    if (centroids_f64) {
      centroids_f64[h + j] = c[j];
      centroids_f64[h - 1 - j] = -c[j];
    }
  }
  out->thresholds[h - 1] = 0.0f;
  if (thresholds_f64) thresholds_f64[h - 1] = 0.0;
  for (int j = 1; j < h; ++j) {
    out->thresholds[h - 1 + j] = (float)tau[j];
    out->thresholds[h - 1 - j] = -(float)tau[j];
    if (thresholds_f64) {
      thresholds_f64[h - 1 + j] = tau[j];
      thresholds_f64[h - 1 - j] = -tau[j];
    }
  }
  if (mse_f64) *mse_f64 = mse;
  return ORBIT_OK;
}

bool valid_bits(int32_t bits) {
  return bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 6 || bits == 8;
}

}  // namespace

extern "C" orbit_status orbit_fit_codebook(int32_t d, int32_t bits, int32_t max_iter, double tol,
                                           orbit_codebook* out, double* centroids_f64,
                                           double* thresholds_f64, double* mse_f64) {
  if (!out || d < 1 || !valid_bits(bits)) return ORBIT_E_ARG;
  return fit(Marginal::gaussian(), d, bits, max_iter, tol, out, centroids_f64, thresholds_f64,
             mse_f64);
}

extern "C" orbit_status orbit_fit_codebook_sphere(int32_t d, int32_t bits, int32_t max_iter,
                                                  double tol, orbit_codebook* out,
                                                  double* centroids_f64, double* thresholds_f64,
                                                  double* mse_f64) {
  if (!out || d < 3 || !valid_bits(bits)) return ORBIT_E_ARG;
  return fit(Marginal::sphere(d), d, bits, max_iter, tol, out, centroids_f64, thresholds_f64,
             mse_f64);
}
