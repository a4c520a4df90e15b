// Host-side fp64 Lloyd-Max fitter for the N(0,1) marginal.
//
// OrbitQuant page, Method: the rotated coordinates of a unit vector follow a
// fixed marginal f_d ~ N(0, 1/d); Lloyd-Max is run on it offline to give one
// codebook per dimension.  The quantizer is scale-equivariant, so the table
// is fitted for N(0,1) and the kernels apply the sqrt(d) scale.
//
// Method used here: a few plain Lloyd alternations, then Newton's method on
// the interior thresholds.  With h = levels/2 positive cells
// 0 = tau_0 < tau_1 < ... < tau_{h-1} < tau_h = inf and centroids
//   c_j = (phi(tau_j) - phi(tau_{j+1})) / (Q(tau_j) - Q(tau_{j+1})),
// the conditions G_j = tau_j - (c_{j-1} + c_j)/2 = 0 (j = 1..h-1) have a
// tridiagonal Jacobian from
//   dc_j/dtau_j = phi(tau_j) (c_j - tau_j) / D_j,
//   dc_j/dtau_{j+1} = phi(tau_{j+1}) (tau_{j+1} - c_j) / D_j,
// solved with the Thomas algorithm.  The negative half mirrors the positive
// one, so the table is exactly symmetric with a zero middle threshold.
#include <cmath>
#include <vector>

#include "orbit_internal.h"

namespace {

const double kInvSqrt2Pi = 0.3989422804014326779399460599343819;
const double kInvSqrt2 = 0.7071067811865475244008443621048490;

double pdf(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }
double upper_tail(double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x * kInvSqrt2); }

// centroids of the positive cells for the given edges (tau has h+1 entries)
void centroids_of(const std::vector<double>& tau, std::vector<double>& c) {
  const size_t h = tau.size() - 1;
  for (size_t j = 0; j < h; ++j) {
    double mass = upper_tail(tau[j]) - upper_tail(tau[j + 1]);
    c[j] = (pdf(tau[j]) - pdf(tau[j + 1])) / mass;
  }
}

}  // namespace

extern "C" orbit_status orbit_fit_codebook(int32_t d, int32_t bits, int32_t max_iter, double tol,
                                           orbit_codebook* out, double* centroids_f64,
                                           double* thresholds_f64, double* mse_f64) {
  if (!out || d < 1) return ORBIT_E_ARG;
  if (!(bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 6 || bits == 8))
    return ORBIT_E_ARG;
  if (max_iter <= 0) max_iter = 100;
  if (!(tol > 0)) tol = 1e-15;
  const int levels = 1 << bits;
  const int h = levels / 2;

  std::vector<double> tau(h + 1), c(h);
  // start: equally spaced thresholds on [0, 3.5 + bits/4]
  tau[0] = 0.0;
  tau[h] = INFINITY;
  const double span = 3.0 + 0.25 * bits;
  for (int j = 1; j < h; ++j) tau[j] = span * j / h;
  centroids_of(tau, c);
  // Lloyd alternations bring the start inside Newton's basin
  for (int it = 0; it < 200; ++it) {
    for (int j = 1; j < h; ++j) tau[j] = 0.5 * (c[j - 1] + c[j]);
    centroids_of(tau, c);
  }
  // Newton on G_j = tau_j - (c_{j-1} + c_j)/2
  std::vector<double> a(h), b(h), cc(h), rhs(h), dlo(h), dhi(h);
  for (int it = 0; it < max_iter && h > 1; ++it) {
    centroids_of(tau, c);
    for (int j = 0; j < h; ++j) {
      double mass = upper_tail(tau[j]) - upper_tail(tau[j + 1]);
      dlo[j] = pdf(tau[j]) * (c[j] - tau[j]) / mass;                              // dc_j/dtau_j
      dhi[j] = std::isinf(tau[j + 1]) ? 0.0 : pdf(tau[j + 1]) * (tau[j + 1] - c[j]) / mass;  // dc_j/dtau_{j+1}
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
  centroids_of(tau, c);

  double mse = 1.0;
  for (int j = 0; j < h; ++j) {
    double p = upper_tail(tau[j]) - upper_tail(tau[j + 1]);
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
