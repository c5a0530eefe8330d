// Per-iteration quintic schedules (host code).
//
// [GNS §3.2] runs Gram Newton-Schulz with the Polar Express quintics, one odd
// polynomial p_t(x) = a_t x + b_t x^3 + c_t x^5 per iteration; its printed
// table is garbled (p_1(1) > 2), so the schedule is derived here from the
// method's defining idea: each p_t is the odd quintic closest to 1 in the
// maximum norm on the interval [l_t, u_t] that holds the singular values at
// that iteration, and the next interval is the image of the current one.
// [GNS §3.3] adds a safety factor f: each polynomial is applied as p_t(x / f),
// so singular values up to f u_t still map into the design range.
//
// The minimax polynomial is found by the Remez exchange: the error 1 - p
// equioscillates at four points, l_t, two interior extrema and u_t (the
// alternation theorem for the Chebyshev system x, x^3, x^5 on 0 < l < u).
#include <cmath>
#include <utility>

#include "../../include/muon.h"

namespace {

// Relative width (u - l) / u below which the limit polynomial is used.
constexpr double kNarrow = 1e-2;

// Solve the 4 x 4 system A y = r by Gaussian elimination with partial
// pivoting.  Returns false if it is singular to working precision.
bool solve4(double A[4][4], double r[4], double y[4]) {
  for (int c = 0; c < 4; ++c) {
    int p = c;
    for (int i = c + 1; i < 4; ++i)
      if (std::fabs(A[i][c]) > std::fabs(A[p][c])) p = i;
    if (!(std::fabs(A[p][c]) > 0.0)) return false;
    if (p != c) {
      for (int j = 0; j < 4; ++j) std::swap(A[p][j], A[c][j]);
      std::swap(r[p], r[c]);
    }
    for (int i = c + 1; i < 4; ++i) {
      const double f = A[i][c] / A[c][c];
      for (int j = c; j < 4; ++j) A[i][j] -= f * A[c][j];
      r[i] -= f * r[c];
    }
  }
  for (int i = 3; i >= 0; --i) {
    double s = r[i];
    for (int j = i + 1; j < 4; ++j) s -= A[i][j] * y[j];
    y[i] = s / A[i][i];
  }
  return std::isfinite(y[0]) && std::isfinite(y[1]) && std::isfinite(y[2]) && std::isfinite(y[3]);
}

// Positive roots x of p'(x) = a + 3 b x^2 + 5 c x^4 (a quadratic in x^2),
// ascending; returns how many.
int critical_points(double a, double b, double c, double x[2]) {
  double y[2];
  int n = 0;
  if (c == 0.0) {
    if (b != 0.0) y[n++] = -a / (3.0 * b);
  } else {
    const double disc = 9.0 * b * b - 20.0 * a * c;
    if (disc < 0.0) return 0;
    const double q = -0.5 * (3.0 * b + std::copysign(std::sqrt(disc), b));
    if (q != 0.0) {
      y[n++] = q / (5.0 * c);
      y[n++] = a / q;
    }
  }
  int m = 0;
  for (int i = 0; i < n; ++i)
    if (y[i] > 0.0 && std::isfinite(y[i])) x[m++] = std::sqrt(y[i]);
  if (m == 2 && x[0] > x[1]) std::swap(x[0], x[1]);
  return m;
}

double poly(double a, double b, double c, double x) {
  const double x2 = x * x;
  return x * (a + x2 * (b + x2 * c));
}

// Minimax odd quintic for the constant 1 on [l, u], 0 < l < u.  Works on
// [l / u, 1] for conditioning and scales back.  Returns false if the exchange
// does not settle.
bool minimax_quintic(double l, double u, double* a, double* b, double* c, double* err) {
  const double s = l / u;
  double z[4];
  for (int i = 0; i < 4; ++i) z[i] = s + (1.0 - s) * 0.5 * (1.0 - std::cos(M_PI * i / 3.0));
  double y[4] = {0, 0, 0, 0};
  bool settled = false;
  for (int it = 0; it < 200 && !settled; ++it) {
    double A[4][4], r[4];
    for (int i = 0; i < 4; ++i) {
      const double x = z[i], x2 = x * x;
      A[i][0] = x;
      A[i][1] = x * x2;
      A[i][2] = x * x2 * x2;
      A[i][3] = (i % 2 == 0) ? 1.0 : -1.0;  // 1 - p(z_i) = +E, -E, +E, -E
      r[i] = 1.0;
    }
    if (!solve4(A, r, y)) return false;
    double x[2];
    if (critical_points(y[0], y[1], y[2], x) != 2 || !(x[0] > s) || !(x[1] < 1.0)) return false;
    // settled once the error at the new interior extrema has the level E of
    // the alternation points (relative 1e-9, or the rounding of 1 - p): then
    // the maximum error on the interval is E and the polynomial is minimax
    const double e = std::fabs(y[3]), tol = 1e-9 * e + 1e-14;
    const double d1 = std::fabs(std::fabs(1.0 - poly(y[0], y[1], y[2], x[0])) - e);
    const double d2 = std::fabs(std::fabs(1.0 - poly(y[0], y[1], y[2], x[1])) - e);
    settled = d1 <= tol && d2 <= tol;
    z[1] = x[0];
    z[2] = x[1];
  }
  if (!settled || !(y[3] > 0.0)) return false;
  *a = y[0] / u;
  *b = y[1] / (u * u * u);
  *c = y[2] / (u * u * u * u * u);
  *err = y[3];
  return true;
}

}  // namespace

extern "C" muon_status muon_quintic_schedule(int T, double ell, double safety, float* coeffs, double* bounds) {
  if (T < 1 || T > MUON_MAX_T || coeffs == nullptr) return MUON_ERR_INVALID_ARG;
  if (!(ell > 0.0) || !(ell < 1.0) || !(safety >= 1.0) || !(safety <= 2.0)) return MUON_ERR_INVALID_ARG;
  double l = ell, u = 1.0;
  if (bounds != nullptr) {
    bounds[0] = l;
    bounds[1] = u;
  }
  for (int t = 0; t < T; ++t) {
    double a, b, c, e;
    // Once the interval is this narrow the minimax polynomials are close to
    // their limit, the one with p(1) = 1, p'(1) = p''(1) = 0, i.e. (15/8,
    // -10/8, 3/8), whose error there (below 3e-6) is under 16-bit rounding.
    if (!(u - l > kNarrow * u)) {
      a = 15.0 / 8.0;
      b = -10.0 / 8.0;
      c = 3.0 / 8.0;
    } else if (!minimax_quintic(l, u, &a, &b, &c, &e)) {
      return MUON_ERR_UNSUPPORTED;  // the exchange did not settle (not seen for 1e-7 <= ell < 1)
    }
    // applied as p(x / f), with the coefficients rounded to the fp32 the
    // iteration uses
    const double f = safety;
    a = static_cast<float>(a / f);
    b = static_cast<float>(b / (f * f * f));
    c = static_cast<float>(c / (f * f * f * f * f));
    // image of [l, u] under the applied polynomial: its extremes are at the
    // ends or at interior critical points
    double lo = poly(a, b, c, l), hi = lo;
    const double pu = poly(a, b, c, u);
    lo = pu < lo ? pu : lo;
    hi = pu > hi ? pu : hi;
    double x[2];
    const int n = critical_points(a, b, c, x);
    for (int i = 0; i < n; ++i)
      if (x[i] > l && x[i] < u) {
        const double v = poly(a, b, c, x[i]);
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
      }
    coeffs[3 * t + 0] = static_cast<float>(a);  // exact: a, b, c are fp32 values
    coeffs[3 * t + 1] = static_cast<float>(b);
    coeffs[3 * t + 2] = static_cast<float>(c);
    l = lo;
    u = hi;
    if (bounds != nullptr) {
      bounds[2 * t + 2] = l;
      bounds[2 * t + 3] = u;
    }
  }
  return MUON_OK;
}
