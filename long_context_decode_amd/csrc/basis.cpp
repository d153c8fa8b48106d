// jssa_basis (host): M* = TopEig_r(G~_Qbar + G~_K)^T per KV head — paper
// summary page, Theoretical Foundation Eq. 5; README page §2 Calibration
// ("one eigendecomposition per (layer, KV head)").
//
// Symmetric eigensolver in double precision: Householder reduction to
// tridiagonal form with the reflections accumulated into Z, then the implicit
// QL algorithm on the tridiagonal matrix, rotating the columns of Z along.
// The QL step follows the published method of Bowdler, Martin, Reinsch and
// Wilkinson ("The QR and QL algorithms for symmetric matrices", Numerische
// Mathematik 11, 1968; the EISPACK routine tql2): a Wilkinson shift from the
// leading 2 x 2 block, then a chase of plane rotations up the matrix.
// O(n^3) once per head (n <= 512).
#include <algorithm>
#include <cmath>
#include <limits>
#include <numeric>
#include <vector>

#include "jssa.h"

namespace jssa {

// Reduce symmetric a (n x n, row-major, overwritten) to tridiagonal form
// T = Z^T a Z.  Returns diag in d[0..n), sub-diagonal in e[0..n-1) (e[n-1] = 0).
static void tridiagonalise(std::vector<double>& a, int n, std::vector<double>& z, std::vector<double>& d,
                           std::vector<double>& e) {
  z.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) z[(size_t)i * n + i] = 1.0;
  std::vector<double> v(n), p(n), w(n);
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;  // length of the column below the diagonal
    double norm = 0.0;
    for (int i = 0; i < m; ++i) norm += a[(size_t)(k + 1 + i) * n + k] * a[(size_t)(k + 1 + i) * n + k];
    norm = std::sqrt(norm);
    if (norm == 0.0) continue;
    const double x0 = a[(size_t)(k + 1) * n + k];
    const double alpha = x0 > 0 ? -norm : norm;
    for (int i = 0; i < m; ++i) v[i] = a[(size_t)(k + 1 + i) * n + k];
    v[0] -= alpha;
    double vn = 0.0;
    for (int i = 0; i < m; ++i) vn += v[i] * v[i];
    vn = std::sqrt(vn);
    if (vn == 0.0) continue;
    for (int i = 0; i < m; ++i) v[i] /= vn;
    // p = A_sub v, kappa = v^T p, w = p - kappa v;  A_sub -= 2 v w^T + 2 w v^T
    double kappa = 0.0;
    for (int i = 0; i < m; ++i) {
      double s = 0.0;
      const double* row = &a[(size_t)(k + 1 + i) * n + k + 1];
      for (int j = 0; j < m; ++j) s += row[j] * v[j];
      p[i] = s;
      kappa += v[i] * s;
    }
    for (int i = 0; i < m; ++i) w[i] = p[i] - kappa * v[i];
    for (int i = 0; i < m; ++i) {
      double* row = &a[(size_t)(k + 1 + i) * n + k + 1];
      for (int j = 0; j < m; ++j) row[j] -= 2.0 * (v[i] * w[j] + w[i] * v[j]);
    }
    // column/row k become (alpha, 0, ..., 0)
    a[(size_t)(k + 1) * n + k] = alpha;
    a[(size_t)k * n + k + 1] = alpha;
    for (int i = 1; i < m; ++i) {
      a[(size_t)(k + 1 + i) * n + k] = 0.0;
      a[(size_t)k * n + k + 1 + i] = 0.0;
    }
    // Z <- Z H on columns k+1..n-1
    for (int r = 0; r < n; ++r) {
      double* zr = &z[(size_t)r * n + k + 1];
      double s = 0.0;
      for (int j = 0; j < m; ++j) s += zr[j] * v[j];
      for (int j = 0; j < m; ++j) zr[j] -= 2.0 * s * v[j];
    }
  }
  d.resize(n);
  e.assign(n, 0.0);
  for (int i = 0; i < n; ++i) d[i] = a[(size_t)i * n + i];
  for (int i = 0; i + 1 < n; ++i) e[i] = a[(size_t)(i + 1) * n + i];
}

// QL iteration with implicit shifts on (d, e); rotates the columns of z.
static bool tridiagonal_ql(std::vector<double>& d, std::vector<double>& e, std::vector<double>& z, int n) {
  const double eps = std::numeric_limits<double>::epsilon();
  for (int l = 0; l < n; ++l) {
    int iter = 0;
    int m;
    do {
      for (m = l; m + 1 < n; ++m) {
        const double dd = std::fabs(d[m]) + std::fabs(d[m + 1]);
        if (std::fabs(e[m]) <= eps * dd) break;
      }
      if (m != l) {
        if (++iter > 100) return false;
        double g = (d[l + 1] - d[l]) / (2.0 * e[l]);
        double r = std::hypot(g, 1.0);
        g = d[m] - d[l] + e[l] / (g + (g >= 0 ? r : -r));
        double s = 1.0, c = 1.0, p = 0.0;
        int i;
        bool underflow = false;
        for (i = m - 1; i >= l; --i) {
          const double f = s * e[i];
          const double b = c * e[i];
          r = std::hypot(f, g);
          e[i + 1] = r;
          if (r == 0.0) {
            d[i + 1] -= p;
            e[m] = 0.0;
            underflow = true;
            break;
          }
          s = f / r;
          c = g / r;
          g = d[i + 1] - p;
          r = (d[i] - g) * s + 2.0 * c * b;
          p = s * r;
          d[i + 1] = g + p;
          g = c * r - b;
          for (int k = 0; k < n; ++k) {
            const double zf = z[(size_t)k * n + i + 1];
            const double zi = z[(size_t)k * n + i];
            z[(size_t)k * n + i + 1] = s * zi + c * zf;
            z[(size_t)k * n + i] = c * zi - s * zf;
          }
        }
        if (underflow) continue;
        d[l] -= p;
        e[l] = g;
        e[m] = 0.0;
      }
    } while (m != l);
  }
  return true;
}

static int32_t basis_one(const float* gq, const float* gk, int n, int r, float* m_out) {
  double tq = 0.0, tk = 0.0;
  for (int i = 0; i < n; ++i) {
    tq += gq[(size_t)i * n + i];
    tk += gk[(size_t)i * n + i];
  }
  if (!(tq > 0.0) || !(tk > 0.0)) return JSSA_ERR_SHAPE;
  std::vector<double> a((size_t)n * n);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      // symmetrise: the accumulated sums are symmetric up to rounding
      const double q = 0.5 * ((double)gq[(size_t)i * n + j] + (double)gq[(size_t)j * n + i]);
      const double k = 0.5 * ((double)gk[(size_t)i * n + j] + (double)gk[(size_t)j * n + i]);
      a[(size_t)i * n + j] = q / tq + k / tk;
    }
  std::vector<double> z, d, e;
  tridiagonalise(a, n, z, d, e);
  if (!tridiagonal_ql(d, e, z, n)) return JSSA_ERR_UNSUPPORTED;
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return d[x] > d[y]; });
  for (int row = 0; row < r; ++row) {
    const int col = order[row];
    int arg = 0;
    double best = -1.0;
    for (int i = 0; i < n; ++i) {
      const double v = std::fabs(z[(size_t)i * n + col]);
      if (v > best) {
        best = v;
        arg = i;
      }
    }
    const double sgn = z[(size_t)arg * n + col] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i) m_out[(size_t)row * n + i] = (float)(sgn * z[(size_t)i * n + col]);
  }
  return JSSA_OK;
}

int32_t basis_impl(int hkv, int n, int r, const float* gq, const float* gk, float* m_out) {
  for (int h = 0; h < hkv; ++h) {
    const int32_t st = basis_one(gq + (size_t)h * n * n, gk + (size_t)h * n * n, n, r, m_out + (size_t)h * r * n);
    if (st != JSSA_OK) return st;
  }
  return JSSA_OK;
}

}  // namespace jssa
