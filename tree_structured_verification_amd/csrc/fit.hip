// tsv_fit_cost: the convex, monotone verification cost C_v(n; l) fitted to
// measured latencies (host code only).
//
// [caddtree] Methodology, item 5: C_v is estimated once, offline, by convex
// regression on latencies measured over context lengths and node counts, so
// that it stays convex and monotone and the throughput objective (item 3)
// stays unimodal.  Model: C_v(n; l) = a + b*n + c*n^2 + e*l*n + f*l with
// a, b, c, e, f >= 0, fitted by non-negative least squares; the f*l term is
// the part of a request's verification that does not grow with its tree
// (reading its prefix once), which dominates a memory-bound attention.
//
// With five unknowns the non-negative least-squares problem is solved
// exactly by trying every support: for each non-empty subset S of the
// columns, the unconstrained least-squares solution on S (QR of the
// column-scaled design); the best residual among those whose
// coefficients are all >= 0 is the optimum (the zero vector is the empty
// support).  Columns are scaled to unit norm first, which leaves the
// non-negative solution unchanged and keeps QR well conditioned when n*l
// reaches millions.

#include <math.h>
#include <string.h>

#include "tsv_internal.hpp"

namespace {

constexpr int kCols = 5;

double column(int j, double n, double l) {
  switch (j) {
    case 0: return 1.0;
    case 1: return n;
    case 2: return n * n;
    case 3: return l * n;
    default: return l;
  }
}

// Least squares min ||A_S x - t|| over the columns in `cols` (k of them) of
// the scaled design; false if A_S is rank deficient.  The measurements are
// folded into an upper-triangular [R | z] one row at a time by Givens
// rotations (a streaming QR), so no storage grows with m; then R x = z.
bool subset_lsq(const double* n, const double* l, const double* t, const double* scale, int m,
                const int* cols, int k, double* x) {
  double R[kCols][kCols + 1];
  for (int r = 0; r < k; ++r)
    for (int c = 0; c <= k; ++c) R[r][c] = 0.0;
  for (int i = 0; i < m; ++i) {
    double v[kCols + 1];
    for (int c = 0; c < k; ++c) v[c] = column(cols[c], n[i], l[i]) / scale[cols[c]];
    v[k] = t[i];
    for (int c = 0; c < k; ++c) {
      if (v[c] == 0.0) continue;
      const double h = hypot(R[c][c], v[c]);
      const double cs = R[c][c] / h, sn = v[c] / h;
      for (int c2 = c; c2 <= k; ++c2) {
        const double r = R[c][c2];
        R[c][c2] = cs * r + sn * v[c2];
        v[c2] = -sn * r + cs * v[c2];
      }
    }
  }
  for (int c = 0; c < k; ++c)
    if (!(fabs(R[c][c]) > 1e-12)) return false;
  for (int c = k - 1; c >= 0; --c) {
    double s = R[c][k];
    for (int c2 = c + 1; c2 < k; ++c2) s -= R[c][c2] * x[c2];
    x[c] = s / R[c][c];
  }
  return true;
}

}  // namespace

extern "C" int tsv_fit_cost(const double* n, const double* l, const double* t, int m, double c_d,
                            tsv_cost_fitted* out) {
  if (!n || !l || !t || !out || m < kCols || m > (1 << 24)) return TSV_EINVAL;
  if (!isfinite(c_d)) return TSV_EINVAL;
  for (int i = 0; i < m; ++i)
    if (!isfinite(n[i]) || !isfinite(l[i]) || !isfinite(t[i]) || n[i] < 0 || l[i] < 0 ||
        t[i] < 0)
      return TSV_EINVAL;
  double scale[kCols];
  for (int j = 0; j < kCols; ++j) {
    double s = 0.0;
    for (int i = 0; i < m; ++i) {
      const double v = column(j, n[i], l[i]);
      s += v * v;
    }
    scale[j] = s > 0.0 ? sqrt(s) : 1.0;
  }
  double best_res = 0.0, best[kCols] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (int i = 0; i < m; ++i) best_res += t[i] * t[i];  // the empty support
  for (int mask = 1; mask < (1 << kCols); ++mask) {
    int cols[kCols], k = 0;
    for (int j = 0; j < kCols; ++j)
      if (mask >> j & 1) cols[k++] = j;
    double xs[kCols];
    if (!subset_lsq(n, l, t, scale, m, cols, k, xs)) continue;
    bool feasible = true;
    for (int c = 0; c < k; ++c) feasible &= xs[c] >= 0.0;
    if (!feasible) continue;
    double coef[kCols] = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int c = 0; c < k; ++c) coef[cols[c]] = xs[c] / scale[cols[c]];
    double res = 0.0;
    for (int i = 0; i < m; ++i) {
      double p = 0.0;
      for (int j = 0; j < kCols; ++j) p += coef[j] * column(j, n[i], l[i]);
      res += (p - t[i]) * (p - t[i]);
    }
    // a later support must be better beyond rounding: when the design is
    // rank deficient (one context length makes n and l*n collinear) equal
    // optima keep the first support in this order (a, b, c, e, f bits)
    if (res < best_res * (1.0 - 1e-12)) {
      best_res = res;
      memcpy(best, coef, sizeof(best));
    }
  }
  out->a = best[0];
  out->b = best[1];
  out->c = best[2];
  out->e = best[3];
  out->f = best[4];
  out->c_d = c_d;
  return TSV_OK;
}
