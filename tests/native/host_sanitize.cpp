// Host-side driver for the sanitizer build of libsq's host code (calibration,
// handle management, save/load, host unpack, error paths).  Compiled with
// g++ -fsanitize=address,undefined together with csrc/calib.cpp and
// csrc/api.cpp; the two device-table entry points are stubbed here (no GPU
// code is built into this binary).  Exits 0 when every call behaved as
// documented in include/sq.h.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace sq {
sq_status upload_tables(sq_calib *, void *) { return fail(SQ_ERR_UNSUPPORTED, "no device in this build"); }
void release_tables(sq_calib *c) {
  c->dev_blob = nullptr;
  c->dev_heads = nullptr;
}
}  // namespace sq

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double uni() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return ((g_state >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static double gauss() { return std::sqrt(-2.0 * std::log(uni())) * std::cos(6.283185307179586 * uni()); }

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "CHECK failed line %d: %s (%s)\n", __LINE__, #cond, sq_last_error()); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

struct Export {
  std::vector<double> lam, R;
  std::vector<int32_t> widths;
  std::vector<float> thr, cent, S;
};

static Export export_head(const sq_calib *c, int h) {
  sq_head_info inf{};
  Export e;
  CHECK(sq_calib_info(c, h, &inf) == SQ_OK);
  const int d = inf.head_dim;
  e.lam.resize(d);
  e.R.resize((size_t)d * d);
  e.widths.resize(d);
  e.thr.resize(inf.n_thresholds);
  e.cent.resize(inf.n_centroids);
  e.S.resize((size_t)inf.m * inf.d_eff);
  CHECK(sq_calib_export(c, h, e.lam.data(), e.R.data(), e.widths.data(), e.thr.data(), e.cent.data(),
                        e.S.data()) == SQ_OK);
  int sum = 0;
  for (int b : e.widths) sum += b;
  CHECK(sum == inf.code_bits);
  CHECK(inf.d_eff >= 1 && inf.d_eff <= d);
  return e;
}

static void one_case(int d, int n_heads, int64_t n, double bits, int qjl, int max_bits, const char *tmp,
                     int normalize = 0) {
  std::vector<float> x((size_t)n_heads * n * d), g((size_t)n_heads * std::max(1, qjl) * d * d);
  for (int h = 0; h < n_heads; ++h)
    for (int64_t t = 0; t < n; ++t)
      for (int i = 0; i < d; ++i)
        x[((size_t)h * n + t) * d + i] = (float)(gauss() * (i < 4 ? 20.0 : 1.0 / (1 + i)));
  for (float &v : g) v = (float)gauss();
  sq_calib_opts o;
  CHECK(sq_calib_default_opts(&o, d) == SQ_OK);
  o.avg_bits = bits;
  o.qjl_bits_per_signal_dim = qjl;
  o.max_bits = max_bits;
  o.lloyd_max_iters = 50;
  o.n_threads = 2;
  o.normalize = normalize;
  sq_calib *c = nullptr;
  CHECK(sq_calibrate(x.data(), n_heads, n, &o, qjl ? g.data() : nullptr, &c) == SQ_OK);
  if (!c) return;
  CHECK(sq_calib_n_heads(c) == n_heads);
  CHECK(sq_calib_save(c, tmp) == SQ_OK);
  sq_calib *c2 = nullptr;
  CHECK(sq_calib_load(tmp, &c2) == SQ_OK);
  for (int h = 0; h < n_heads && c2; ++h) {
    Export a = export_head(c, h), b = export_head(c2, h);
    CHECK(a.lam == b.lam && a.R == b.R && a.widths == b.widths);
    CHECK(a.thr == b.thr && a.cent == b.cent && a.S == b.S);
  }
  CHECK(sq_packed_head_words(c, 100) == 128 * (int64_t)c->W_max);
  // host unpack of random words, every head
  const int64_t T = 70;
  std::vector<uint32_t> words((size_t)sq_packed_head_words(c, T));
  for (uint32_t &w : words) w = (uint32_t)(uni() * 4294967296.0);
  std::vector<uint8_t> codes((size_t)T * d), z((size_t)T * 8 * d + 1);
  std::vector<float> gam(T);
  for (int h = 0; h < n_heads; ++h) {
    std::vector<float> nus(T);
    CHECK(sq_unpack(c, h, words.data(), T, codes.data(), z.data(), gam.data(), nus.data()) == SQ_OK);
    sq_head_info inf{};
    sq_calib_info(c, h, &inf);
    for (int64_t t = 0; t < T; ++t)
      for (int i = 0; i < d; ++i) CHECK(codes[(size_t)t * d + i] < (1u << 8));
  }
  // truncated copies of the file are refused, never read past their end
  FILE *f = std::fopen(tmp, "rb");
  std::vector<char> bytes;
  if (f) {
    int ch;
    while ((ch = std::fgetc(f)) != EOF) bytes.push_back((char)ch);
    std::fclose(f);
  }
  const size_t cuts[] = {0, 5, 12, 40, bytes.size() / 3, bytes.size() / 2, bytes.size() - 1};
  for (size_t cut : cuts) {
    if (cut >= bytes.size()) continue;
    FILE *w = std::fopen(tmp, "wb");
    std::fwrite(bytes.data(), 1, cut, w);
    std::fclose(w);
    sq_calib *c3 = nullptr;
    CHECK(sq_calib_load(tmp, &c3) != SQ_OK && c3 == nullptr);
  }
  sq_calib_destroy(c2);
  sq_calib_destroy(c);
}

int main(int argc, char **argv) {
  const char *tmp = argc > 1 ? argv[1] : "/tmp/sq_sanitize.sqcal";
  one_case(32, 3, 256, 3.0, 1, 8, tmp);
  one_case(32, 1, 2, 3.0, 1, 8, tmp);        // fewer samples than dimensions
  one_case(64, 2, 40, 0.5, 0, 8, tmp);       // many zero-width coordinates
  one_case(64, 1, 100, 8.0, 2, 8, tmp);      // every coordinate at 8 bits, 2 QJL rows per signal dim
  one_case(128, 2, 300, 3.0, 1, 8, tmp);
  one_case(128, 1, 200, 2.0, 1, 2, tmp);     // capped widths
  one_case(256, 1, 300, 3.0, 1, 8, tmp);
  one_case(64, 2, 120, 3.0, 1, 8, tmp, 1);   // normalised variant
  // TurboQuant-style calibrations: random rotation, keys and values
  {
    const int d = 64;
    std::vector<float> rot((size_t)2 * d * d), g((size_t)2 * d * d);
    for (float &v : rot) v = (float)gauss();
    for (float &v : g) v = (float)gauss();
    sq_calib_opts o;
    sq_calib_default_opts(&o, d);
    o.avg_bits = 3.0;
    sq_calib *k = nullptr, *v = nullptr;
    CHECK(sq_calibrate_tq(rot.data(), g.data(), 2, &o, &k) == SQ_OK);
    o.qjl_bits_per_signal_dim = 0;
    CHECK(sq_calibrate_tq(rot.data(), nullptr, 2, &o, &v) == SQ_OK);
    o.avg_bits = 2.5;
    sq_calib *bad = nullptr;
    CHECK(sq_calibrate_tq(rot.data(), nullptr, 2, &o, &bad) == SQ_ERR_ARG && !bad);
    if (k && v) {
      Export ek = export_head(k, 1), ev = export_head(v, 0);
      CHECK(ek.widths[0] == 2 && ev.widths[5] == 3);
      CHECK(sq_calib_save(k, tmp) == SQ_OK);
      sq_calib *k2 = nullptr;
      CHECK(sq_calib_load(tmp, &k2) == SQ_OK);
      sq_head_info inf{};
      if (k2) CHECK(sq_calib_info(k2, 0, &inf) == SQ_OK && inf.normalized == 1 && inf.m == d);
      sq_calib_destroy(k2);
    }
    sq_calib_destroy(k);
    sq_calib_destroy(v);
  }
  // error paths
  sq_calib_opts o;
  sq_calib *c = nullptr;
  std::vector<float> x(64 * 32, 1.0f);
  CHECK(sq_calib_default_opts(nullptr, 32) == SQ_ERR_ARG);
  CHECK(sq_calib_default_opts(&o, 48) == SQ_OK);
  CHECK(sq_calibrate(x.data(), 1, 64, &o, nullptr, &c) == SQ_ERR_UNSUPPORTED && !c);
  sq_calib_default_opts(&o, 32);
  o.qjl_bits_per_signal_dim = 0;
  CHECK(sq_calibrate(x.data(), 1, 1, &o, nullptr, &c) == SQ_ERR_NUMERIC && !c);
  x[7] = NAN;
  CHECK(sq_calibrate(x.data(), 1, 64, &o, nullptr, &c) == SQ_ERR_NUMERIC && !c);
  x[7] = 1.0f;
  o.avg_bits = 9.0;
  CHECK(sq_calibrate(x.data(), 1, 64, &o, nullptr, &c) == SQ_ERR_ARG && !c);
  o.avg_bits = 3.0;
  o.qjl_bits_per_signal_dim = 1;
  CHECK(sq_calibrate(x.data(), 1, 64, &o, nullptr, &c) == SQ_ERR_ARG && !c);
  CHECK(sq_calibrate(nullptr, 1, 64, &o, nullptr, &c) == SQ_ERR_ARG);
  CHECK(sq_calib_load("/nonexistent/dir/file", &c) == SQ_ERR_IO);
  CHECK(sq_calib_info(nullptr, 0, nullptr) == SQ_ERR_ARG);
  CHECK(sq_packed_head_words(nullptr, 10) == -1);
  CHECK(sq_unpack(nullptr, 0, nullptr, 1, nullptr, nullptr, nullptr, nullptr) == SQ_ERR_ARG);
  CHECK(std::strlen(sq_build_digest()) > 0);
  sq_calib_destroy(nullptr);
  std::printf("host sanitize driver: %d failures\n", g_fail);
  return g_fail ? 1 : 0;
}
