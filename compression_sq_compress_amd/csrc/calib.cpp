// Host-side, one-time SpectralQuant calibration of one attention head.
//
// Follows the SpectralQuant README "Repository Structure" (calibration.py: PCA,
// d_eff, kappa; nonuniform_quantization.py: Lloyd-Max with per-regime
// codebooks; selective_qjl.py: QJL on the signal dims) and the repository's
// tests/conftest.py fixture pre_computed_calibration (uncentered second moment,
// eigenvalues in descending order, d_eff = int(round(participation ratio)),
// spectral gap).  The bit allocation is the integer form of the reverse
// water-filling named by the ossradar.top summary's core-capability list.
//
// Everything here runs in double precision on the host.  The eigensolver is
// the cyclic Jacobi method (Golub & Van Loan, "Matrix Computations", sec. 8.5),
// chosen for its accuracy on the small (d <= 256) symmetric matrices involved.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <string>
#include <vector>

#include "internal.h"

namespace sq {
namespace {

// Cyclic Jacobi eigendecomposition of the symmetric d x d matrix `a`
// (row-major, destroyed).  On return diag(a) holds the eigenvalues and the
// columns of `v` the matching orthonormal eigenvectors.
void jacobi_eigen(std::vector<double> &a, std::vector<double> &v, int d) {
  v.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) v[(size_t)i * d + i] = 1.0;
  auto A = [&](int r, int c) -> double & { return a[(size_t)r * d + c]; };
  auto V = [&](int r, int c) -> double & { return v[(size_t)r * d + c]; };
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) off += A(p, q) * A(p, q);
    if (off == 0.0) break;
    for (int p = 0; p < d - 1; ++p) {
      for (int q = p + 1; q < d; ++q) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double app = A(p, p), aqq = A(q, q);
        // an off-diagonal entry far below both diagonal entries is treated as zero
        if (sweep >= 4 && std::fabs(app) + 1e2 * std::fabs(apq) == std::fabs(app) &&
            std::fabs(aqq) + 1e2 * std::fabs(apq) == std::fabs(aqq)) {
          A(p, q) = A(q, p) = 0.0;
          continue;
        }
        // symmetric 2x2 Schur decomposition: choose t = tan(theta) of the
        // smaller rotation that annihilates a_pq
        const double tau = (aqq - app) / (2.0 * apq);
        const double t = (tau >= 0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < d; ++k) {  // A <- A J  (columns p, q)
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {  // A <- J^T A  (rows p, q)
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        A(p, q) = A(q, p) = 0.0;
        for (int k = 0; k < d; ++k) {  // V <- V J
          const double vkp = V(k, p), vkq = V(k, q);
          V(k, p) = c * vkp - s * vkq;
          V(k, q) = s * vkp + c * vkq;
        }
      }
    }
  }
}

// Greedy integer reverse water-filling: each bit of the budget goes to the
// coordinate with the largest l_i * 4^-b_i (ties to the lower index).
std::vector<int32_t> water_fill(const std::vector<double> &lam, long total, int max_bits) {
  const int d = (int)lam.size();
  std::vector<int32_t> b(d, 0);
  for (long step = 0; step < total; ++step) {
    int best = -1;
    double bv = -1.0;
    for (int i = 0; i < d; ++i) {
      if (b[i] >= max_bits) continue;
      const double v = std::ldexp(lam[i], -2 * b[i]);
      if (v > bv) { bv = v; best = i; }
    }
    if (best < 0) break;
    b[best] += 1;
  }
  return b;
}

// Lloyd-Max on sorted samples u: start at the (j + 1/2)/L sample quantiles,
// alternate midpoint thresholds and cell means until the partition repeats or
// max_iter updates; empty cells keep their level.  Returns converged flag.
bool lloyd_max(const std::vector<double> &u, int L, int max_iter, std::vector<double> &c) {
  const int64_t n = (int64_t)u.size();
  c.assign(L, 0.0);
  if (n == 0) return true;
  for (int j = 0; j < L; ++j) c[j] = u[(size_t)(((int64_t)(2 * j + 1) * n) / (2 * (int64_t)L))];
  std::vector<double> prefix(n + 1, 0.0);
  for (int64_t k = 0; k < n; ++k) prefix[k + 1] = prefix[k] + u[k];
  std::vector<int64_t> cut(L - 1), prev;
  int updates = 0;
  for (;;) {
    for (int j = 0; j + 1 < L; ++j) {
      const double t = (c[j] + c[j + 1]) / 2;
      cut[j] = std::upper_bound(u.begin(), u.end(), t) - u.begin();  // #{u <= t}
    }
    if (!prev.empty() && cut == prev) return true;
    if (updates == max_iter) return false;
    for (int j = 0; j < L; ++j) {
      const int64_t lo = j == 0 ? 0 : cut[j - 1];
      const int64_t hi = j == L - 1 ? n : cut[j];
      if (hi > lo) c[j] = (prefix[hi] - prefix[lo]) / (double)(hi - lo);
    }
    prev = cut;
    ++updates;
  }
}

}  // namespace

void finish_layout(HeadCal &h) {
  const int d = h.d;
  h.bit_off.assign(d, 0);
  h.thr_base.assign(d, 0);
  h.cent_base.assign(d, 0);
  int bits = 0, nt = 0, nc = 0;
  for (int i = 0; i < d; ++i) {
    h.bit_off[i] = bits;
    h.thr_base[i] = nt;
    h.cent_base[i] = nc;
    bits += h.widths[i];
    if (h.widths[i] > 0) {
      nt += (1 << h.widths[i]) - 1;
      nc += 1 << h.widths[i];
    }
  }
  h.code_bits = bits;
  h.n_thr = nt;
  h.n_cent = nc;
  const int total = bits + h.m + (h.m > 0 ? 16 : 0) + (h.normalized ? 16 : 0);
  h.W = std::max(1, (total + 31) / 32);
}

sq_status calibrate_head(const float *x, int64_t n, int d, const sq_calib_opts &o,
                         const float *gauss, HeadCal &h, std::string &err) {
  h = HeadCal();
  h.d = d;
  h.normalized = o.normalize != 0;
  // normalised variant: every sample divided by its norm (a zero sample stays zero)
  std::vector<double> unit;
  if (h.normalized) {
    unit.assign((size_t)n * d, 0.0);
    for (int64_t t = 0; t < n; ++t) {
      const float *xr = x + (size_t)t * d;
      double s = 0.0;
      for (int i = 0; i < d; ++i) s += (double)xr[i] * (double)xr[i];
      const double nrm = std::sqrt(s);
      for (int i = 0; i < d; ++i) unit[(size_t)t * d + i] = nrm > 0 ? (double)xr[i] / nrm : 0.0;
    }
  }
  auto sample = [&](int64_t t, int i) -> double {
    return h.normalized ? unit[(size_t)t * d + i] : (double)x[(size_t)t * d + i];
  };
  // 1. second moment C = X^T X / n (uncentered), double
  std::vector<double> C((size_t)d * d, 0.0);
  std::vector<double> row(d);
  for (int64_t t = 0; t < n; ++t) {
    const float *xr = x + (size_t)t * d;
    for (int i = 0; i < d; ++i) {
      if (!std::isfinite(xr[i])) {
        err = "non-finite calibration sample";
        return SQ_ERR_NUMERIC;
      }
      row[i] = sample(t, i);
    }
    for (int i = 0; i < d; ++i) {
      const double ri = row[i];
      double *ci = &C[(size_t)i * d];
      for (int j = i; j < d; ++j) ci[j] += ri * row[j];
    }
  }
  for (int i = 0; i < d; ++i)
    for (int j = i; j < d; ++j) {
      C[(size_t)i * d + j] /= (double)n;
      C[(size_t)j * d + i] = C[(size_t)i * d + j];
    }
  // 2. eigendecomposition, descending, clamped, sign rule
  std::vector<double> V;
  jacobi_eigen(C, V, d);
  std::vector<double> lam, R;
  order_eigenpairs(C, V, d, lam, R);
  // rotated samples y_t = R x_t (x_t divided by its norm in the normalised variant)
  std::vector<double> Y((size_t)n * d);
  for (int64_t t = 0; t < n; ++t)
    for (int i = 0; i < d; ++i) {
      const double *Ri = &R[(size_t)i * d];
      double y = 0.0;
      for (int j = 0; j < d; ++j) y += Ri[j] * sample(t, j);
      Y[(size_t)t * d + i] = y;
    }
  return finish_head_from_eigen(lam, R, Y.data(), n, d, o, gauss, h, err);
}

void order_eigenpairs(const std::vector<double> &a, const std::vector<double> &V, int d, std::vector<double> &lam,
                      std::vector<double> &R) {
  std::vector<int> order(d);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return a[(size_t)x * d + x] > a[(size_t)y * d + y];
  });
  lam.resize(d);
  R.assign((size_t)d * d, 0.0);
  for (int k = 0; k < d; ++k) {
    const int src = order[k];
    lam[k] = std::max(0.0, a[(size_t)src * d + src]);
    int jmax = 0;
    double vmax = -1.0;
    for (int j = 0; j < d; ++j) {
      const double v = std::fabs(V[(size_t)j * d + src]);
      if (v > vmax) { vmax = v; jmax = j; }
    }
    const double sgn = V[(size_t)jmax * d + src] < 0 ? -1.0 : 1.0;
    for (int j = 0; j < d; ++j) R[(size_t)k * d + j] = sgn * V[(size_t)j * d + src];
  }
}

int deff_from_spectrum(const std::vector<double> &lam, double cumvar) {
  const int d = (int)lam.size();
  double s1 = 0.0, s2 = 0.0;
  for (double l : lam) { s1 += l; s2 += l * l; }
  if (cumvar > 0) {
    // smallest k whose leading k eigenvalues hold at least the fraction cumvar of the total
    double acc = 0.0;
    for (int k = 1; k <= d; ++k) {
      acc += lam[k - 1];
      if (acc >= cumvar * s1) return k;
    }
    return d;
  }
  const double pr = s2 > 0 ? s1 * s1 / s2 : 0.0;
  const long r = (long)std::nearbyint(pr);  // default rounding mode: half to even
  return (int)std::min<long>(std::max<long>(r, 1), d);
}

sq_status finish_head_from_eigen(const std::vector<double> &lam, const std::vector<double> &R, const double *Y,
                                 int64_t n, int d, const sq_calib_opts &o, const float *gauss, HeadCal &h,
                                 std::string &err) {
  h = HeadCal();
  h.d = d;
  h.normalized = o.normalize != 0;
  h.lam = lam;
  h.R = R;
  // 3. participation ratio, d_eff (rounded PR, or the cumulative-variance rule), kappa
  double s1 = 0.0, s2 = 0.0;
  for (double l : h.lam) { s1 += l; s2 += l * l; }
  h.pr = s2 > 0 ? s1 * s1 / s2 : 0.0;
  h.d_eff = deff_from_spectrum(h.lam, o.deff_cumvar);
  h.kappa = (h.d_eff >= d || h.lam[h.d_eff] <= 0) ? std::numeric_limits<double>::infinity()
                                                  : h.lam[h.d_eff - 1] / h.lam[h.d_eff];
  // 4. widths
  const long budget = (long)std::nearbyint(o.avg_bits * d);
  h.widths = water_fill(h.lam, budget, o.max_bits);
  h.m = o.qjl_bits_per_signal_dim > 0 ? o.qjl_bits_per_signal_dim * h.d_eff : 0;
  finish_layout(h);
  // 5. per-region Lloyd-Max on pooled standardised rotated samples
  std::vector<double> sigma(d);
  for (int i = 0; i < d; ++i) sigma[i] = std::sqrt(h.lam[i]);
  h.thr.assign(h.n_thr, 0.0f);
  h.cent.assign(h.n_cent, 0.0f);
  for (int regime = 0; regime < 2; ++regime) {
    for (int b = 1; b <= o.max_bits; ++b) {
      std::vector<int> coords;
      for (int i = 0; i < d; ++i)
        if (h.widths[i] == b && ((i < h.d_eff) == (regime == 0))) coords.push_back(i);
      if (coords.empty()) continue;
      h.n_regions += 1;
      std::vector<double> u;
      u.reserve((size_t)n * coords.size());
      for (int i : coords) {
        if (!(sigma[i] > 0)) continue;
        for (int64_t t = 0; t < n; ++t) u.push_back(Y[(size_t)t * d + i] / sigma[i]);
      }
      std::sort(u.begin(), u.end());
      const int L = 1 << b;
      std::vector<double> c;
      if (!lloyd_max(u, L, o.lloyd_max_iters, c)) h.unconverged += 1;
      for (int i : coords) {
        for (int j = 0; j < L; ++j) h.cent[h.cent_base[i] + j] = (float)(sigma[i] * c[j]);
        for (int j = 0; j + 1 < L; ++j)
          h.thr[h.thr_base[i] + j] = (float)(sigma[i] * ((c[j] + c[j + 1]) / 2));
      }
    }
  }
  // 6. QJL sketch S = G[0:m, 0:d_eff]
  h.S.assign((size_t)h.m * h.d_eff, 0.0f);
  if (h.m > 0) {
    if (!gauss) {
      err = "qjl_gauss is NULL but qjl_bits_per_signal_dim > 0";
      return SQ_ERR_ARG;
    }
    for (int j = 0; j < h.m; ++j)
      for (int i = 0; i < h.d_eff; ++i) h.S[(size_t)j * h.d_eff + i] = gauss[(size_t)j * d + i];
  }
  return SQ_OK;
}

// Lloyd-Max quantiser of the standard normal density with L levels (Max,
// 1960): iterate the centroid condition c_j = (phi(a) - phi(b)) / (Phi(b) -
// Phi(a)) over the cells (a, b] between midpoints from uniformly spread
// levels until the levels stop moving; returns the levels, ascending.
static std::vector<double> gaussian_lloyd_max(int L) {
  std::vector<double> c(L, 0.0);
  if (L == 1) return c;
  for (int j = 0; j < L; ++j) c[j] = -2.0 + 4.0 * j / (L - 1);
  auto phi = [](double t) { return std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI); };
  auto Phi = [](double t) { return 0.5 * std::erfc(-t / std::sqrt(2.0)); };
  for (int it = 0; it < 200000; ++it) {
    double delta = 0.0;
    std::vector<double> nc(L);
    for (int j = 0; j < L; ++j) {
      const double a = j == 0 ? -INFINITY : 0.5 * (c[j - 1] + c[j]);
      const double b = j == L - 1 ? INFINITY : 0.5 * (c[j] + c[j + 1]);
      const double pa = std::isinf(a) ? 0.0 : phi(a), pb = std::isinf(b) ? 0.0 : phi(b);
      const double mass = (std::isinf(b) ? 1.0 : Phi(b)) - (std::isinf(a) ? 0.0 : Phi(a));
      nc[j] = (pa - pb) / mass;
      delta = std::max(delta, std::fabs(nc[j] - c[j]));
    }
    c = nc;
    if (delta < 1e-15) break;
  }
  return c;
}

sq_status calibrate_head_tq(const float *rotation, int d, const sq_calib_opts &o, const float *gauss,
                            HeadCal &h, std::string &err) {
  h = HeadCal();
  h.d = d;
  h.normalized = true;
  const bool keys = o.qjl_bits_per_signal_dim > 0;
  const int bits = (int)std::lround(o.avg_bits);
  const int b = keys ? bits - 1 : bits;
  h.R.assign((size_t)d * d, 0.0);
  for (size_t k = 0; k < (size_t)d * d; ++k) {
    if (!std::isfinite(rotation[k])) {
      err = "non-finite rotation entry";
      return SQ_ERR_NUMERIC;
    }
    h.R[k] = (double)rotation[k];
  }
  h.lam.assign(d, 1.0 / d);  // a rotated unit vector's coordinate variance
  h.pr = (double)d;
  h.d_eff = d;                // the QJL sketch covers every coordinate
  h.kappa = std::numeric_limits<double>::infinity();
  h.widths.assign(d, b);
  h.m = keys ? d : 0;
  finish_layout(h);
  h.thr.assign(h.n_thr, 0.0f);
  h.cent.assign(h.n_cent, 0.0f);
  if (b > 0) {
    const int L = 1 << b;
    const std::vector<double> c = gaussian_lloyd_max(L);
    const double s = 1.0 / std::sqrt((double)d);
    for (int i = 0; i < d; ++i) {
      for (int j = 0; j < L; ++j) h.cent[h.cent_base[i] + j] = (float)(s * c[j]);
      for (int j = 0; j + 1 < L; ++j) h.thr[h.thr_base[i] + j] = (float)(s * 0.5 * (c[j] + c[j + 1]));
    }
    h.n_regions = 1;
  }
  h.S.assign((size_t)h.m * h.d_eff, 0.0f);
  if (h.m > 0) {
    if (!gauss) {
      err = "qjl_gauss is NULL but the keys' QJL sketch was requested";
      return SQ_ERR_ARG;
    }
    for (size_t k = 0; k < (size_t)d * d; ++k) h.S[k] = gauss[k];
  }
  return SQ_OK;
}

}  // namespace sq
