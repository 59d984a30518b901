// Calibration on the device: the second-moment matrix, its eigendecomposition
// and the rotated calibration samples of every head run in fp64 on the GPU;
// the host finishes each head (eigen-order and sign rule, d_eff, widths, the
// per-region Lloyd-Max codebooks) with the same code as the host calibration.
//
// SpectralQuant README "Overview" (a one-time calibration) and "Repository
// Structure" (calibration: PCA, d_eff, kappa); the repository's
// tests/conftest.py fixture pre_computed_calibration (uncentered X^T X / n,
// eigh).  The eigensolver is the parallel cyclic Jacobi method (Brent & Luk,
// SIAM J. Sci. Stat. Comput. 6 (1985)): each step applies d/2 rotations on
// the disjoint index pairs of a round-robin tournament, d - 1 steps a sweep,
// so all pairs of a step update disjoint rows and columns at once.
#include <algorithm>
#include <atomic>
#include <memory>
#include <cmath>
#include <thread>
#include <vector>

#include "devcommon.h"
#include "internal.h"

namespace sq {

constexpr int JACOBI_MAX_SWEEPS = 100;

// inv_norm[h][t] = 1 / |x_t| (0 for a zero sample), fp64.
__global__ __launch_bounds__(256) void inv_norm_kernel(const float *x, int64_t n, int d, double *inv_norm) {
  const int h = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const float *r = x + ((size_t)h * n + t) * d;
  double s = 0.0;
  for (int i = 0; i < d; ++i) s = fma((double)r[i], (double)r[i], s);
  inv_norm[(size_t)h * n + t] = s > 0 ? 1.0 / sqrt(s) : 0.0;
}

// C[h] = X_h^T X_h / n, fp64 (rows scaled by inv_norm when normalising).
// Workgroup = (16 x 16 output tile, head); thread = one output entry; the
// samples stream through LDS 64 rows at a time.
__global__ __launch_bounds__(256) void covariance_kernel(const float *x, int64_t n, int d, int normalize,
                                                         const double *inv_norm, double *C) {
  const int h = blockIdx.z;
  const int li = threadIdx.x >> 4, lj = threadIdx.x & 15;
  const int ti = blockIdx.y * 16 + li, tj = blockIdx.x * 16 + lj;
  const float *xh = x + (size_t)h * n * d;
  __shared__ double a[64][17], b[64][17];
  double acc = 0.0;
  for (int64_t t0 = 0; t0 < n; t0 += 64) {
    for (int k = threadIdx.x; k < 64 * 16; k += 256) {
      const int r = k >> 4, c = k & 15;
      const int64_t t = t0 + r;
      const double s = (t < n && normalize) ? inv_norm[(size_t)h * n + t] : 1.0;
      a[r][c] = t < n ? s * (double)xh[t * d + blockIdx.y * 16 + c] : 0.0;
      b[r][c] = t < n ? s * (double)xh[t * d + blockIdx.x * 16 + c] : 0.0;
    }
    __syncthreads();
    for (int r = 0; r < 64; ++r) acc = fma(a[r][li], b[r][lj], acc);
    __syncthreads();
  }
  C[((size_t)h * d + ti) * d + tj] = acc / (double)n;
}

// Parallel cyclic Jacobi on A[h] (d x d, destroyed: its diagonal ends as the
// eigenvalues); V[h] receives the eigenvectors as columns.  One workgroup per
// head.  Each rotation is the symmetric 2 x 2 Schur decomposition of the host
// solver (the smaller angle that annihilates a_pq; from the fifth sweep an
// entry negligible next to both diagonal entries is set to zero instead).
// Stops after a sweep that starts with no off-diagonal entry left, or after
// JACOBI_MAX_SWEEPS.  status[h] = 1 when the matrix is not finite (a non-
// finite sample), else 0.
// LDSA: A is worked on in LDS (d <= 128: 128 KB of fp64) and written back at
// the end; V stays in device memory.
template <bool LDSA>
__global__ __launch_bounds__(256) void jacobi_kernel(double *A, double *V, int d, int *status) {
  extern __shared__ double a_lds[];
  const int h = blockIdx.x;
  double *a_g = A + (size_t)h * d * d;
  double *a = LDSA ? a_lds : a_g;
  double *v = V + (size_t)h * d * d;
  if constexpr (LDSA) {
    for (int k = threadIdx.x; k < d * d; k += 256) a_lds[k] = a_g[k];
    __syncthreads();
  }
  __shared__ double cs[128], sn[128];
  __shared__ int pp[128], qq[128];
  __shared__ double red[256];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int half = d / 2;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int k = tid; k < d * d; k += 256) {
    v[k] = (k / d == k % d) ? 1.0 : 0.0;
    if (!isfinite(a[k])) bad = 1;
  }
  __syncthreads();
  if (tid == 0) status[h] = bad;
  if (bad) return;
  for (int sweep = 0; sweep < JACOBI_MAX_SWEEPS; ++sweep) {
    double off = 0.0;
    for (int k = tid; k < d * d; k += 256) {
      const int r = k / d, c = k - r * d;
      if (r < c) off += a[k] * a[k];
    }
    red[tid] = off;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    const bool done = red[0] == 0.0;
    __syncthreads();
    if (done) break;
    for (int step = 0; step < d - 1; ++step) {
      // round robin: player 0 stays, players 1 .. d-1 shift by one per step;
      // slot k meets slot d-1-k
      for (int k = tid; k < half; k += 256) {
        const int sa = k, sb = d - 1 - k;
        int p = sa == 0 ? 0 : 1 + (sa - 1 + step) % (d - 1);
        int q = 1 + (sb - 1 + step) % (d - 1);
        if (p > q) { const int t = p; p = q; q = t; }
        pp[k] = p;
        qq[k] = q;
        const double apq = a[(size_t)p * d + q], app = a[(size_t)p * d + p], aqq = a[(size_t)q * d + q];
        double c = 1.0, s = 0.0;
        const bool negligible = sweep >= 4 && fabs(app) + 1e2 * fabs(apq) == fabs(app) &&
                                fabs(aqq) + 1e2 * fabs(apq) == fabs(aqq);
        if (apq != 0.0 && !negligible) {
          const double tau = (aqq - app) / (2.0 * apq);
          const double t = (tau >= 0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        cs[k] = c;
        sn[k] = s;
      }
      __syncthreads();
      // A <- A J and V <- V J (columns p, q of every pair); neighbouring
      // threads take different pairs of one row (distinct LDS banks)
      for (int k = tid; k < half * d; k += 256) {
        const int r = k / half, pr = k - r * half;
        const double s = sn[pr];
        if (s == 0.0) continue;
        const int p = pp[pr], q = qq[pr];
        const double c = cs[pr];
        const double arp = a[(size_t)r * d + p], arq = a[(size_t)r * d + q];
        a[(size_t)r * d + p] = c * arp - s * arq;
        a[(size_t)r * d + q] = s * arp + c * arq;
        const double vrp = v[(size_t)r * d + p], vrq = v[(size_t)r * d + q];
        v[(size_t)r * d + p] = c * vrp - s * vrq;
        v[(size_t)r * d + q] = s * vrp + c * vrq;
      }
      __syncthreads();
      // A <- J^T A (rows p, q of every pair)
      for (int k = tid; k < half * d; k += 256) {
        const int pr = k / d, col = k - pr * d;
        const double s = sn[pr];
        if (s == 0.0) continue;
        const int p = pp[pr], q = qq[pr];
        const double c = cs[pr];
        const double apc = a[(size_t)p * d + col], aqc = a[(size_t)q * d + col];
        a[(size_t)p * d + col] = c * apc - s * aqc;
        a[(size_t)q * d + col] = s * apc + c * aqc;
      }
      __syncthreads();
      // the annihilated (or negligible) entries are exactly zero
      for (int k = tid; k < half; k += 256) {
        a[(size_t)pp[k] * d + qq[k]] = 0.0;
        a[(size_t)qq[k] * d + pp[k]] = 0.0;
      }
      __syncthreads();
    }
  }
  if constexpr (LDSA) {
    __syncthreads();
    for (int k = threadIdx.x; k < d * d; k += 256) a_g[k] = a_lds[k];
  }
}

// Y[h][t] = R_h x_t (x_t scaled to unit norm when normalising), fp64.
// Thread = one (sample, coordinate); R_h rows are the ordered, signed
// eigenvectors.
__global__ __launch_bounds__(256) void rotate_samples_kernel(const float *x, int64_t n, int d, int normalize,
                                                             const double *inv_norm, const double *R, double *Y) {
  const int h = blockIdx.z;
  const int64_t t = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  const int i = blockIdx.x * 16 + (threadIdx.x & 15);
  if (t >= n) return;
  const float *xr = x + ((size_t)h * n + t) * d;
  const double *ri = R + ((size_t)h * d + i) * d;
  const double s = normalize ? inv_norm[(size_t)h * n + t] : 1.0;
  double acc = 0.0;
  for (int j = 0; j < d; ++j) acc = fma(ri[j], s * (double)xr[j], acc);
  Y[((size_t)h * n + t) * d + i] = acc;
}

namespace {
struct DevBuf {
  void *p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

// Host memory for the rotated samples of one chunk of heads.
constexpr size_t CHUNK_BYTES = (size_t)512 << 20;
}  // namespace

}  // namespace sq

using namespace sq;

extern "C" sq_status sq_calibrate_device(const float *samples, int n_heads, int64_t n_samples,
                                         const sq_calib_opts *opts, const float *qjl_gauss, sq_stream stream,
                                         sq_calib **out) {
  const char *fn = "sq_calibrate_device";
  if (!out) return fail(SQ_ERR_ARG, "sq_calibrate_device: out is NULL");
  *out = nullptr;
  sq_status st = check_calib_opts(opts);
  if (st != SQ_OK) return st;
  if (!samples) return fail(SQ_ERR_ARG, "sq_calibrate_device: samples is NULL");
  if (n_heads <= 0) return fail(SQ_ERR_ARG, "sq_calibrate_device: n_heads must be > 0");
  if (n_heads > 65535) return fail(SQ_ERR_UNSUPPORTED, "sq_calibrate_device: at most 65535 heads per call");
  if (n_samples < 2) return fail(SQ_ERR_NUMERIC, "sq_calibrate_device: need at least 2 samples per head");
  if (n_samples > ((int64_t)1 << 30)) return fail(SQ_ERR_UNSUPPORTED, "sq_calibrate_device: at most 2^30 samples");
  if (opts->qjl_bits_per_signal_dim > 0 && !qjl_gauss)
    return fail(SQ_ERR_ARG, "sq_calibrate_device: qjl_gauss is NULL but QJL bits were requested");
  const int d = opts->head_dim;
  const size_t dd = (size_t)d * d;
  const size_t per_head_y = (size_t)n_samples * d * sizeof(double);
  if (per_head_y > CHUNK_BYTES)
    return fail(SQ_ERR_UNSUPPORTED, "sq_calibrate_device: samples of one head exceed the 512 MiB staging limit");
  const int chunk = (int)std::max<size_t>(1, std::min<size_t>(n_heads, CHUNK_BYTES / per_head_y));
  hipStream_t s = (hipStream_t)stream;
  const int norm = opts->normalize ? 1 : 0;
  DevBuf bC, bV, bN, bR, bY, bS;
  hipError_t e;
  if ((e = hipMalloc(&bC.p, sizeof(double) * dd * n_heads)) != hipSuccess ||
      (e = hipMalloc(&bV.p, sizeof(double) * dd * n_heads)) != hipSuccess ||
      (e = hipMalloc(&bR.p, sizeof(double) * dd * n_heads)) != hipSuccess ||
      (e = hipMalloc(&bS.p, sizeof(int) * n_heads)) != hipSuccess ||
      (e = hipMalloc(&bY.p, per_head_y * chunk)) != hipSuccess ||
      (norm && (e = hipMalloc(&bN.p, sizeof(double) * (size_t)n_samples * n_heads)) != hipSuccess))
    return fail(SQ_ERR_ALLOC, std::string("sq_calibrate_device: hipMalloc: ") + hipGetErrorString(e));
  double *C = (double *)bC.p, *V = (double *)bV.p, *N = (double *)bN.p, *R = (double *)bR.p, *Y = (double *)bY.p;
  int *S = (int *)bS.p;
  if (norm)
    hipLaunchKernelGGL(inv_norm_kernel, dim3((unsigned)((n_samples + 255) / 256), n_heads), dim3(256), 0, s,
                       samples, n_samples, d, N);
  hipLaunchKernelGGL(covariance_kernel, dim3(d / 16, d / 16, n_heads), dim3(256), 0, s, samples, n_samples, d, norm,
                     (const double *)N, C);
  if (d <= 128)
    hipLaunchKernelGGL(jacobi_kernel<true>, dim3(n_heads), dim3(256), sizeof(double) * dd, s, C, V, d, S);
  else
    hipLaunchKernelGGL(jacobi_kernel<false>, dim3(n_heads), dim3(256), 0, s, C, V, d, S);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(fn, e);
  std::vector<double> hC(dd * n_heads), hV(dd * n_heads);
  std::vector<int> hS(n_heads);
  if ((e = hipMemcpyAsync(hC.data(), C, sizeof(double) * hC.size(), hipMemcpyDeviceToHost, s)) != hipSuccess ||
      (e = hipMemcpyAsync(hV.data(), V, sizeof(double) * hV.size(), hipMemcpyDeviceToHost, s)) != hipSuccess ||
      (e = hipMemcpyAsync(hS.data(), S, sizeof(int) * n_heads, hipMemcpyDeviceToHost, s)) != hipSuccess ||
      (e = hipStreamSynchronize(s)) != hipSuccess)
    return hip_fail(fn, e);
  for (int h = 0; h < n_heads; ++h)
    if (hS[h]) return fail(SQ_ERR_NUMERIC, "sq_calibrate_device: head " + std::to_string(h) + ": non-finite calibration sample");
  // eigen-order and sign rule on the host; the rotation goes back to the device
  std::vector<std::vector<double>> lam(n_heads), Rh(n_heads);
  std::vector<double> hR(dd * n_heads);
  for (int h = 0; h < n_heads; ++h) {
    std::vector<double> ah(hC.begin() + dd * h, hC.begin() + dd * (h + 1));
    std::vector<double> vh(hV.begin() + dd * h, hV.begin() + dd * (h + 1));
    order_eigenpairs(ah, vh, d, lam[h], Rh[h]);
    std::copy(Rh[h].begin(), Rh[h].end(), hR.begin() + dd * h);
  }
  if ((e = hipMemcpyAsync(R, hR.data(), sizeof(double) * hR.size(), hipMemcpyHostToDevice, s)) != hipSuccess)
    return hip_fail(fn, e);
  sq_calib *c = new (std::nothrow) sq_calib();
  if (!c) return fail(SQ_ERR_ALLOC, "sq_calibrate_device: out of host memory");
  std::unique_ptr<sq_calib> guard(c);
  c->opts = *opts;
  std::vector<double> hY;
  try {
    c->heads.resize(n_heads);
    hY.resize((size_t)n_samples * d * chunk);
  } catch (...) {
    return fail(SQ_ERR_ALLOC, "sq_calibrate_device: out of host memory");
  }
  const int64_t gstride = (int64_t)std::max(1, opts->qjl_bits_per_signal_dim) * d * d;
  int nt = opts->n_threads > 0 ? opts->n_threads : (int)std::thread::hardware_concurrency();
  nt = std::max(1, std::min(nt, chunk));
  std::vector<sq_status> sts(n_heads, SQ_OK);
  std::vector<std::string> errs(n_heads);
  for (int h0 = 0; h0 < n_heads; h0 += chunk) {
    const int nh = std::min(chunk, n_heads - h0);
    const float *xs = samples + (size_t)h0 * n_samples * d;
    hipLaunchKernelGGL(rotate_samples_kernel, dim3(d / 16, (unsigned)((n_samples + 15) / 16), nh), dim3(256), 0, s,
                       xs, n_samples, d, norm, norm ? (const double *)N + (size_t)h0 * n_samples : nullptr,
                       (const double *)R + dd * h0, Y);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(fn, e);
    if ((e = hipMemcpyAsync(hY.data(), Y, per_head_y * nh, hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
      return hip_fail(fn, e);
    std::atomic<int> next(0);
    auto work = [&]() {
      for (;;) {
        const int k = next.fetch_add(1);
        if (k >= nh) break;
        const int h = h0 + k;
        try {
          sts[h] = finish_head_from_eigen(lam[h], Rh[h], hY.data() + (size_t)n_samples * d * k, n_samples, d, *opts,
                                          qjl_gauss ? qjl_gauss + (size_t)h * gstride : nullptr, c->heads[h], errs[h]);
        } catch (...) {
          sts[h] = SQ_ERR_ALLOC;
          errs[h] = "out of host memory";
        }
      }
    };
    std::vector<std::thread> pool;
    for (int i = 1; i < std::min(nt, nh); ++i) pool.emplace_back(work);
    work();
    for (auto &t : pool) t.join();
    for (int k = 0; k < nh; ++k)
      if (sts[h0 + k] != SQ_OK)
        return fail(sts[h0 + k], "sq_calibrate_device: head " + std::to_string(h0 + k) + ": " + errs[h0 + k]);
  }
  c->W_max = 0;
  for (auto &hh : c->heads) c->W_max = std::max(c->W_max, hh.W);
  *out = guard.release();
  clear_error();
  return SQ_OK;
}
