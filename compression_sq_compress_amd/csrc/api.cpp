// C ABI of libsq: host-side entry points (calibration, handle management,
// save/load, host unpack, error reporting).  Device entry points are in
// kernels.hip.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"

namespace sq {

static thread_local std::string g_last_error;

sq_status fail(sq_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }

}  // namespace sq

using namespace sq;

extern "C" const char *sq_last_error(void) { return g_last_error.c_str(); }

#ifndef SQ_SOURCE_DIGEST
#define SQ_SOURCE_DIGEST "unknown"
#endif
extern "C" const char *sq_build_digest(void) { return SQ_SOURCE_DIGEST; }

static bool supported_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

extern "C" sq_status sq_calib_default_opts(sq_calib_opts *o, int head_dim) {
  if (!o) return fail(SQ_ERR_ARG, "sq_calib_default_opts: opts is NULL");
  o->head_dim = head_dim;
  o->avg_bits = 3.0;
  o->qjl_bits_per_signal_dim = 1;
  o->max_bits = 8;
  o->lloyd_max_iters = 200;
  o->n_threads = 0;
  o->normalize = 0;
  o->deff_cumvar = 0.0;
  clear_error();
  return SQ_OK;
}

sq_status sq::check_calib_opts(const sq_calib_opts *o) {
  if (!o) return fail(SQ_ERR_ARG, "opts is NULL");
  if (!supported_dim(o->head_dim))
    return fail(SQ_ERR_UNSUPPORTED, "head_dim must be 32, 64, 128 or 256");
  if (o->max_bits < 1 || o->max_bits > 8) return fail(SQ_ERR_ARG, "max_bits must be in [1, 8]");
  if (!(o->avg_bits > 0.0) || o->avg_bits > o->max_bits)
    return fail(SQ_ERR_ARG, "avg_bits must be in (0, max_bits]");
  if (o->qjl_bits_per_signal_dim < 0 || o->qjl_bits_per_signal_dim > 8)
    return fail(SQ_ERR_ARG, "qjl_bits_per_signal_dim must be in [0, 8]");
  if (o->lloyd_max_iters < 0) return fail(SQ_ERR_ARG, "lloyd_max_iters must be >= 0");
  if (o->normalize != 0 && o->normalize != 1) return fail(SQ_ERR_ARG, "normalize must be 0 or 1");
  if (!(o->deff_cumvar >= 0.0 && o->deff_cumvar <= 1.0))
    return fail(SQ_ERR_ARG, "deff_cumvar must be 0 (participation ratio) or in (0, 1]");
  return SQ_OK;
}

static void compute_wmax(sq_calib *c) {
  c->W_max = 0;
  for (auto &h : c->heads) c->W_max = std::max(c->W_max, h.W);
}

extern "C" sq_status sq_calibrate(const float *samples, int n_heads, int64_t n_samples,
                                  const sq_calib_opts *opts, const float *qjl_gauss,
                                  sq_calib **out) {
  if (!out) return fail(SQ_ERR_ARG, "sq_calibrate: out is NULL");
  *out = nullptr;
  sq_status st = check_calib_opts(opts);
  if (st != SQ_OK) return st;
  if (!samples) return fail(SQ_ERR_ARG, "sq_calibrate: samples is NULL");
  if (n_heads <= 0) return fail(SQ_ERR_ARG, "sq_calibrate: n_heads must be > 0");
  if (n_samples < 2) return fail(SQ_ERR_NUMERIC, "sq_calibrate: need at least 2 samples per head");
  if (opts->qjl_bits_per_signal_dim > 0 && !qjl_gauss)
    return fail(SQ_ERR_ARG, "sq_calibrate: qjl_gauss is NULL but QJL bits were requested");
  sq_calib *c = new (std::nothrow) sq_calib();
  if (!c) return fail(SQ_ERR_ALLOC, "sq_calibrate: out of host memory");
  c->opts = *opts;
  const int d = opts->head_dim;
  try {
    c->heads.resize(n_heads);
  } catch (...) {
    delete c;
    return fail(SQ_ERR_ALLOC, "sq_calibrate: out of host memory");
  }
  int nt = opts->n_threads > 0 ? opts->n_threads : (int)std::thread::hardware_concurrency();
  nt = std::max(1, std::min(nt, n_heads));
  std::vector<sq_status> sts(n_heads, SQ_OK);
  std::vector<std::string> errs(n_heads);
  std::atomic<int> next(0);
  const int64_t gstride = (int64_t)std::max(1, opts->qjl_bits_per_signal_dim) * d * d;
  auto work = [&]() {
    for (;;) {
      const int h = next.fetch_add(1);
      if (h >= n_heads) break;
      try {
        sts[h] = calibrate_head(samples + (size_t)h * n_samples * d, n_samples, d, *opts,
                                qjl_gauss ? qjl_gauss + (size_t)h * gstride : nullptr,
                                c->heads[h], errs[h]);
      } catch (...) {
        sts[h] = SQ_ERR_ALLOC;
        errs[h] = "out of host memory";
      }
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < nt; ++i) pool.emplace_back(work);
  work();
  for (auto &t : pool) t.join();
  for (int h = 0; h < n_heads; ++h)
    if (sts[h] != SQ_OK) {
      delete c;
      return fail(sts[h], "sq_calibrate: head " + std::to_string(h) + ": " + errs[h]);
    }
  compute_wmax(c);
  *out = c;
  clear_error();
  return SQ_OK;
}

extern "C" sq_status sq_calibrate_tq(const float *rotation, const float *qjl_gauss, int n_heads,
                                     const sq_calib_opts *opts, sq_calib **out) {
  if (!out) return fail(SQ_ERR_ARG, "sq_calibrate_tq: out is NULL");
  *out = nullptr;
  sq_status st = check_calib_opts(opts);
  if (st != SQ_OK) return st;
  if (!rotation) return fail(SQ_ERR_ARG, "sq_calibrate_tq: rotation is NULL");
  if (n_heads <= 0) return fail(SQ_ERR_ARG, "sq_calibrate_tq: n_heads must be > 0");
  const bool keys = opts->qjl_bits_per_signal_dim > 0;
  if (keys && opts->qjl_bits_per_signal_dim != 1)
    return fail(SQ_ERR_ARG, "sq_calibrate_tq: the keys' sketch has one bit per dim (qjl_bits_per_signal_dim 1)");
  const double b = opts->avg_bits;
  const int lo = keys ? 2 : 1, hi = keys ? 9 : 8;
  if (b != std::floor(b) || b < lo || b > hi)
    return fail(SQ_ERR_ARG, "sq_calibrate_tq: avg_bits must be an integer in [1, 8] (values) or [2, 9] (keys)");
  if (keys && !qjl_gauss) return fail(SQ_ERR_ARG, "sq_calibrate_tq: qjl_gauss is NULL for keys");
  sq_calib *c = new (std::nothrow) sq_calib();
  if (!c) return fail(SQ_ERR_ALLOC, "sq_calibrate_tq: out of host memory");
  c->opts = *opts;
  c->opts.normalize = 1;
  const int d = opts->head_dim;
  try {
    c->heads.resize(n_heads);
    for (int h = 0; h < n_heads; ++h) {
      std::string err;
      st = calibrate_head_tq(rotation + (size_t)h * d * d, d, c->opts,
                             keys ? qjl_gauss + (size_t)h * d * d : nullptr, c->heads[h], err);
      if (st != SQ_OK) {
        delete c;
        return fail(st, "sq_calibrate_tq: head " + std::to_string(h) + ": " + err);
      }
    }
  } catch (...) {
    delete c;
    return fail(SQ_ERR_ALLOC, "sq_calibrate_tq: out of host memory");
  }
  compute_wmax(c);
  *out = c;
  clear_error();
  return SQ_OK;
}

extern "C" int sq_calib_n_heads(const sq_calib *c) { return c ? (int)c->heads.size() : 0; }

extern "C" sq_status sq_calib_info(const sq_calib *c, int head, sq_head_info *info) {
  if (!c || !info) return fail(SQ_ERR_ARG, "sq_calib_info: NULL argument");
  if (head < 0 || head >= (int)c->heads.size()) return fail(SQ_ERR_ARG, "sq_calib_info: head out of range");
  const HeadCal &h = c->heads[head];
  info->head_dim = h.d;
  info->d_eff = h.d_eff;
  info->m = h.m;
  info->code_bits = h.code_bits;
  info->record_words = h.W;
  info->n_thresholds = h.n_thr;
  info->n_centroids = h.n_cent;
  info->n_regions = h.n_regions;
  info->lloyd_unconverged = h.unconverged;
  info->participation_ratio = h.pr;
  info->kappa = h.kappa;
  info->normalized = h.normalized ? 1 : 0;
  clear_error();
  return SQ_OK;
}

extern "C" sq_status sq_calib_export(const sq_calib *c, int head, double *eigenvalues,
                                     double *rotation, int32_t *widths, float *thresholds,
                                     float *centroids, float *qjl) {
  if (!c) return fail(SQ_ERR_ARG, "sq_calib_export: handle is NULL");
  if (head < 0 || head >= (int)c->heads.size()) return fail(SQ_ERR_ARG, "sq_calib_export: head out of range");
  const HeadCal &h = c->heads[head];
  if (eigenvalues) std::memcpy(eigenvalues, h.lam.data(), h.lam.size() * sizeof(double));
  if (rotation) std::memcpy(rotation, h.R.data(), h.R.size() * sizeof(double));
  if (widths) std::memcpy(widths, h.widths.data(), h.widths.size() * sizeof(int32_t));
  if (thresholds && !h.thr.empty()) std::memcpy(thresholds, h.thr.data(), h.thr.size() * sizeof(float));
  if (centroids && !h.cent.empty()) std::memcpy(centroids, h.cent.data(), h.cent.size() * sizeof(float));
  if (qjl && !h.S.empty()) std::memcpy(qjl, h.S.data(), h.S.size() * sizeof(float));
  clear_error();
  return SQ_OK;
}

// ---------------------------------------------------------------- save / load
// File: "SQCALIB1", u32 version, opts (fixed fields; version 2 adds
// normalize, version 3 the f64 deff_cumvar after avg_bits), u32 n_heads, then per head: i32 d, d_eff, m; f64 pr, kappa;
// f64 lam[d]; f64 R[d*d]; i32 widths[d]; i32 n_regions, unconverged
// (version 2: and normalized); f32 thr[n_thr]; f32 cent[n_cent];
// f32 S[m*d_eff].  Little-endian.  Version 1 files load as unnormalised.
static const char kMagic[8] = {'S', 'Q', 'C', 'A', 'L', 'I', 'B', '1'};
static const uint32_t kVersion = 3;  // 2: normalised variant flag; 3: d_eff rule in the options

namespace {
struct File {
  FILE *f = nullptr;
  bool ok = true;
  ~File() { if (f) fclose(f); }
  void w(const void *p, size_t n) { if (ok && n && fwrite(p, 1, n, f) != n) ok = false; }
  void r(void *p, size_t n) { if (ok && n && fread(p, 1, n, f) != n) ok = false; }
};
}  // namespace

extern "C" sq_status sq_calib_save(const sq_calib *c, const char *path) {
  if (!c || !path) return fail(SQ_ERR_ARG, "sq_calib_save: NULL argument");
  File F;
  F.f = fopen(path, "wb");
  if (!F.f) return fail(SQ_ERR_IO, std::string("sq_calib_save: cannot open ") + path);
  F.w(kMagic, 8);
  F.w(&kVersion, 4);
  int32_t oi[6] = {c->opts.head_dim, c->opts.qjl_bits_per_signal_dim, c->opts.max_bits,
                   c->opts.lloyd_max_iters, c->opts.n_threads, c->opts.normalize};
  F.w(oi, sizeof(oi));
  F.w(&c->opts.avg_bits, 8);
  F.w(&c->opts.deff_cumvar, 8);
  uint32_t nh = (uint32_t)c->heads.size();
  F.w(&nh, 4);
  for (const HeadCal &h : c->heads) {
    int32_t hi[3] = {h.d, h.d_eff, h.m};
    F.w(hi, sizeof(hi));
    F.w(&h.pr, 8);
    F.w(&h.kappa, 8);
    F.w(h.lam.data(), h.lam.size() * 8);
    F.w(h.R.data(), h.R.size() * 8);
    F.w(h.widths.data(), h.widths.size() * 4);
    int32_t extra[3] = {h.n_regions, h.unconverged, h.normalized ? 1 : 0};
    F.w(extra, sizeof(extra));
    F.w(h.thr.data(), h.thr.size() * 4);
    F.w(h.cent.data(), h.cent.size() * 4);
    F.w(h.S.data(), h.S.size() * 4);
  }
  if (!F.ok) return fail(SQ_ERR_IO, "sq_calib_save: write failed");
  clear_error();
  return SQ_OK;
}

extern "C" sq_status sq_calib_load(const char *path, sq_calib **out) {
  if (!path || !out) return fail(SQ_ERR_ARG, "sq_calib_load: NULL argument");
  *out = nullptr;
  File F;
  F.f = fopen(path, "rb");
  if (!F.f) return fail(SQ_ERR_IO, std::string("sq_calib_load: cannot open ") + path);
  char magic[8];
  uint32_t ver = 0;
  F.r(magic, 8);
  F.r(&ver, 4);
  if (!F.ok || std::memcmp(magic, kMagic, 8) != 0 || ver < 1 || ver > kVersion)
    return fail(SQ_ERR_IO, "sq_calib_load: not a calibration file of a known version");
  sq_calib *c = new (std::nothrow) sq_calib();
  if (!c) return fail(SQ_ERR_ALLOC, "sq_calib_load: out of host memory");
  int32_t oi[6] = {0, 0, 0, 0, 0, 0};
  F.r(oi, ver >= 2 ? sizeof(oi) : 5 * sizeof(int32_t));
  c->opts.head_dim = oi[0];
  c->opts.qjl_bits_per_signal_dim = oi[1];
  c->opts.max_bits = oi[2];
  c->opts.lloyd_max_iters = oi[3];
  c->opts.n_threads = oi[4];
  c->opts.normalize = oi[5];
  F.r(&c->opts.avg_bits, 8);
  c->opts.deff_cumvar = 0.0;
  if (ver >= 3) F.r(&c->opts.deff_cumvar, 8);
  uint32_t nh = 0;
  F.r(&nh, 4);
  if (!F.ok || check_calib_opts(&c->opts) != SQ_OK || nh == 0 || nh > (1u << 24)) {
    delete c;
    return fail(SQ_ERR_IO, "sq_calib_load: malformed header");
  }
  c->heads.resize(nh);
  for (HeadCal &h : c->heads) {
    int32_t hi[3];
    F.r(hi, sizeof(hi));
    if (!F.ok || hi[0] != c->opts.head_dim || hi[1] < 1 || hi[1] > hi[0] || hi[2] < 0 ||
        hi[2] > 8 * hi[0]) {
      delete c;
      return fail(SQ_ERR_IO, "sq_calib_load: malformed head record");
    }
    h.d = hi[0];
    h.d_eff = hi[1];
    h.m = hi[2];
    F.r(&h.pr, 8);
    F.r(&h.kappa, 8);
    h.lam.resize(h.d);
    h.R.resize((size_t)h.d * h.d);
    h.widths.resize(h.d);
    F.r(h.lam.data(), h.lam.size() * 8);
    F.r(h.R.data(), h.R.size() * 8);
    F.r(h.widths.data(), h.widths.size() * 4);
    int32_t extra[3] = {0, 0, 0};
    F.r(extra, ver >= 2 ? sizeof(extra) : 2 * sizeof(int32_t));
    h.n_regions = extra[0];
    h.unconverged = extra[1];
    if (extra[2] != 0 && extra[2] != 1) F.ok = false;
    h.normalized = extra[2] == 1;
    for (int32_t b : h.widths)
      if (b < 0 || b > 8) F.ok = false;
    if (!F.ok) {
      delete c;
      return fail(SQ_ERR_IO, "sq_calib_load: malformed widths");
    }
    finish_layout(h);
    h.thr.resize(h.n_thr);
    h.cent.resize(h.n_cent);
    h.S.resize((size_t)h.m * h.d_eff);
    F.r(h.thr.data(), h.thr.size() * 4);
    F.r(h.cent.data(), h.cent.size() * 4);
    F.r(h.S.data(), h.S.size() * 4);
  }
  if (!F.ok) {
    delete c;
    return fail(SQ_ERR_IO, "sq_calib_load: truncated file");
  }
  compute_wmax(c);
  *out = c;
  clear_error();
  return SQ_OK;
}

extern "C" void sq_calib_destroy(sq_calib *c) {
  if (!c) return;
  release_tables(c);
  delete c;
}

extern "C" int64_t sq_paged_block_words(const sq_calib *c, int block_tiles) {
  if (!c || block_tiles < 1) return -1;
  return (int64_t)block_tiles * 64 * c->W_max;
}

extern "C" int64_t sq_packed_head_words(const sq_calib *c, int64_t n_tokens) {
  if (!c || n_tokens < 0) return -1;
  return ((n_tokens + 63) / 64) * 64 * (int64_t)c->W_max;
}

// ---------------------------------------------------------------- host unpack
static float half_to_float(uint32_t hb) {
  const uint32_t sgn = (hb >> 15) & 1, ex = (hb >> 10) & 31, man = hb & 1023;
  float v;
  if (ex == 0) v = std::ldexp((float)man, -24);
  else if (ex == 31) v = man ? NAN : INFINITY;
  else v = std::ldexp((float)(man | 1024), (int)ex - 25);
  return sgn ? -v : v;
}

extern "C" sq_status sq_unpack(const sq_calib *c, int head, const uint32_t *packed,
                               int64_t n_tokens, uint8_t *codes, uint8_t *qjl, float *gamma,
                               float *nu) {
  if (!c || !packed || !codes) return fail(SQ_ERR_ARG, "sq_unpack: NULL argument");
  if (head < 0 || head >= (int)c->heads.size()) return fail(SQ_ERR_ARG, "sq_unpack: head out of range");
  if (n_tokens < 0) return fail(SQ_ERR_ARG, "sq_unpack: n_tokens < 0");
  const HeadCal &h = c->heads[head];
  if (h.m > 0 && !qjl) return fail(SQ_ERR_ARG, "sq_unpack: qjl is NULL but the head has QJL bits");
  const int W = h.W;
  std::vector<uint32_t> rec(W + 1);
  auto field = [&](int pos, int width) -> uint32_t {
    const int w = pos >> 5, s = pos & 31;
    const uint64_t both = (uint64_t)rec[w] | ((uint64_t)rec[w + 1] << 32);
    return (uint32_t)((both >> s) & ((1ull << width) - 1));
  };
  for (int64_t t = 0; t < n_tokens; ++t) {
    for (int w = 0; w < W; ++w) rec[w] = packed[((t / 64) * W + w) * 64 + t % 64];
    rec[W] = 0;
    for (int i = 0; i < h.d; ++i)
      codes[(size_t)t * h.d + i] = h.widths[i] ? (uint8_t)field(h.bit_off[i], h.widths[i]) : 0;
    for (int j = 0; j < h.m; ++j) qjl[(size_t)t * h.m + j] = (uint8_t)field(h.code_bits + j, 1);
    if (gamma) gamma[t] = h.m > 0 ? half_to_float(rec[W - 1] >> 16) : 0.0f;
    if (nu) nu[t] = h.normalized ? half_to_float(h.m > 0 ? rec[W - 1] & 0xFFFFu : rec[W - 1] >> 16) : 0.0f;
  }
  clear_error();
  return SQ_OK;
}
