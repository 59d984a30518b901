// SpectralQuant hot path on gfx950 (MI355X): table upload, sq_compress,
// sq_scores, sq_attend, sq_dequantize.
//
// The method (SpectralQuant README, "Overview" and "Repository Structure";
// ossradar.top summary, core capabilities): rotate each K/V vector into the
// calibrated eigenbasis, quantise every rotated coordinate with its region's
// Lloyd-Max codebook at its water-filled width, add a 1-bit QJL sketch of the
// residual on the d_eff signal coordinates of keys only, pack bit-dense; at
// decode time rotate the query once and score directly from the codes, and
// dequantise values for the softmax-weighted sum.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <limits>
#include <string>
#include <type_traits>
#include <vector>

#include "internal.h"

namespace sq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float((uint32_t)u << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs)
__host__ __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t half_bits_rne(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Uniform table reads go through the constant address space so that they
// become scalar loads: the compiler can then neither confuse them with the
// kernel's own global stores nor make them wait for those stores.
#define SQ_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const SQ_CONST T *cptr(const void *p) {
  return (const SQ_CONST T *)(uintptr_t)p;
}
__device__ __forceinline__ DevCoord load_coord(const SQ_CONST DevCoord *p) {
  DevCoord r;
  r.bit_off = p->bit_off;
  r.width = p->width;
  r.thr_base = p->thr_base;
  r.cent_base = p->cent_base;
  return r;
}

// ------------------------------------------------------------------ upload

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Score schedule of one head (layout: SCHED_WORDS).  Adjacent coordinates
// are paired greedily when their widths sum to at most 8 bits; while the
// joint tables exceed SCORE_LUT_BYTES, the pair with the largest table is
// split again.  An odd number of halves gets an empty half (table entry:
// the trailing zero entry).
constexpr int SCORE_PAIR_BITS = 8;
constexpr size_t SCORE_LUT_BYTES = 80 * 1024;

struct ScoreSched {
  std::vector<uint32_t> quads;  // [n_quads][SCHED_WORDS]
  std::vector<uint32_t> lut;    // [n_plut][2]
  int n_quads = 0, n_plut = 0;
};

static void bf16_split(float v, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16_rne(v);
  float vh;
  const uint32_t u = (uint32_t)hi << 16;
  std::memcpy(&vh, &u, 4);
  lo = f32_to_bf16_rne(v - vh);
}

static ScoreSched build_score_sched(const HeadCal &hc) {
  const int d = hc.d;
  const std::vector<int32_t> &w = hc.widths;
  std::vector<char> paired(d, 0);  // paired[i]: coordinates i and i+1 form one half
  for (int i = 0; i + 1 < d;) {
    if (w[i] + w[i + 1] <= SCORE_PAIR_BITS) {
      paired[i] = 1;
      i += 2;
    } else {
      i += 1;
    }
  }
  auto entries = [&]() {
    size_t n = 1;  // trailing zero entry
    for (int i = 0; i < d;) {
      if (paired[i]) { n += (size_t)1 << (w[i] + w[i + 1]); i += 2; }
      else { n += (size_t)1 << w[i]; i += 1; }
    }
    return n;
  };
  while (entries() * 8 > SCORE_LUT_BYTES) {
    int best = -1, bw = -1;
    for (int i = 0; i + 1 < d; ++i)
      if (paired[i] && w[i] + w[i + 1] > bw) { bw = w[i] + w[i + 1]; best = i; }
    if (best < 0) break;
    paired[best] = 0;
  }
  struct Half { int a, b, pos, width; uint32_t first; };
  std::vector<Half> halves;
  ScoreSched S;
  auto cent = [&](int i, int code) -> float {
    return w[i] > 0 ? hc.cent[hc.cent_base[i] + code] : 0.0f;
  };
  for (int i = 0; i < d;) {
    Half h;
    h.a = i;
    h.b = paired[i] ? i + 1 : -1;
    h.pos = hc.bit_off[i];
    h.width = w[i] + (h.b >= 0 ? w[h.b] : 0);
    h.first = 0;
    halves.push_back(h);
    i += paired[i] ? 2 : 1;
  }
  if (halves.size() & 1) halves.push_back(Half{-1, -1, 0, 0, 0});  // empty half: one zero entry
  // tables placed largest first, so each starts at a multiple of its own size
  // (entry address = table base | code << 3)
  std::vector<int> order(halves.size());
  for (size_t k = 0; k < order.size(); ++k) order[k] = (int)k;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return halves[x].width > halves[y].width; });
  uint32_t next = 0;
  for (int k : order) {
    halves[k].first = next;
    next += 1u << halves[k].width;
  }
  S.lut.assign((size_t)next * 2, 0u);
  for (size_t k = 0; k < halves.size(); ++k) {
    const Half &h = halves[k];
    if (h.a < 0) continue;
    const int wa = w[h.a];
    const bool first = (k & 1) == 0;  // first half of its quad: (lo, hi), second: (hi, lo)
    for (int v = 0; v < (1 << h.width); ++v) {
      uint16_t ah, al, bh = 0, bl = 0;
      bf16_split(cent(h.a, v & ((1 << wa) - 1)), ah, al);
      if (h.b >= 0) bf16_split(cent(h.b, v >> wa), bh, bl);
      const uint32_t hp = (uint32_t)ah | ((uint32_t)bh << 16), lp = (uint32_t)al | ((uint32_t)bl << 16);
      S.lut[2 * ((size_t)h.first + v)] = first ? lp : hp;
      S.lut[2 * ((size_t)h.first + v) + 1] = first ? hp : lp;
    }
  }
  S.n_quads = (int)halves.size() / 2;
  S.n_plut = (int)next;
  auto slot = [](int c) { return c < 0 ? 0xFFFFu : (uint32_t)c; };
  for (int q = 0; q < S.n_quads; ++q) {
    const Half &h0 = halves[2 * q], &h1 = halves[2 * q + 1];
    const uint32_t e[SCHED_WORDS] = {
        (uint32_t)h0.pos | ((uint32_t)h0.width << 16), (uint32_t)h1.pos | ((uint32_t)h1.width << 16),
        h0.first, h1.first, slot(h0.a) | (slot(h0.b) << 16), slot(h1.a) | (slot(h1.b) << 16), 0u, 0u};
    S.quads.insert(S.quads.end(), e, e + SCHED_WORDS);
  }
  return S;
}

static sq_status hip_fail(const char *what, hipError_t e) {
  return fail(SQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void release_tables(sq_calib *c) {
  if (c->dev_blob) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (c->device >= 0 && cur != c->device) (void)hipSetDevice(c->device);
    (void)hipFree(c->dev_blob);
    if (c->device >= 0 && cur != c->device && cur >= 0) (void)hipSetDevice(cur);
  }
  c->dev_blob = nullptr;
  c->dev_heads = nullptr;
  c->dev_bytes = 0;
  c->device = -1;
}

// Compress plan of one head (layout in devtypes.h): wave headers, chunks,
// padded threshold trees and signal centroids.
struct HostPlan {
  std::vector<uint32_t> words;
  std::vector<float> tree, csig;
  int n_chunks = 0;
};

static uint32_t f32_bits(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  return u;
}

// Does the compress kernel fold the QJL sketch into the quantiser of wave 0?
// (Small sketches: the whole signal range then lies in wave 0's coordinates.)
static bool qjl_inline(const HeadCal &hc) { return hc.m > 0 && hc.m <= 8 && hc.d_eff <= 8; }

// Estimated cycles of one chunk of n coordinates of width b: each tree level
// is one dependent LDS round trip, plus the issue of ~3b + 2 VALU per slot.
static double chunk_cost(int b, int n) { return 300.0 * (b + 1) + 8.0 * n * (3 * b + 2) + 150.0; }

// Cost of a run of n equal-width coordinates, cut into chunks of 8, 4, 2, 1.
static double run_cost(int b, int n) {
  double c = 0.0;
  while (n > 0) {
    int k = 8;
    while (k > n) k >>= 1;
    c += chunk_cost(b, k);
    n -= k;
  }
  return c;
}

static HostPlan build_plan(const HeadCal &hc) {
  const int d = hc.d, NW = d / 16;
  HostPlan P;
  // Wave ranges: contiguous, minimising the largest estimated quantiser time
  // (dynamic programme over cut points); with the QJL folded in, wave 0 must
  // hold the whole signal range.
  const bool qin = qjl_inline(hc);
  std::vector<double> rc((size_t)(d + 1) * (d + 1), 0.0);  // rc[a*(d+1)+b]: cost of [a, b)
  for (int a0 = 0; a0 < d; ++a0) {
    double done = 0.0;
    int rw = -1, rn = 0;
    for (int b1 = a0 + 1; b1 <= d; ++b1) {
      const int wd = hc.widths[b1 - 1];
      if (wd != rw) {
        if (rn && rw > 0) done += run_cost(rw, rn);
        rw = wd;
        rn = 0;
      }
      ++rn;
      rc[(size_t)a0 * (d + 1) + b1] = done + (rw > 0 ? run_cost(rw, rn) : 0.0);
    }
  }
  const double INF = 1e30;
  if (qin) {
    for (int b1 = 0; b1 < hc.d_eff; ++b1) rc[b1] = INF;   // wave 0 = [0, b1) needs b1 >= d_eff
    for (int b1 = hc.d_eff; b1 <= d; ++b1) rc[b1] += 8.0 * hc.m * hc.d_eff + 500.0;
  }
  // f[k][b]: best max cost of covering [0, b) with k waves
  std::vector<double> f((size_t)(NW + 1) * (d + 1), INF);
  std::vector<int> arg((size_t)(NW + 1) * (d + 1), 0);
  f[0] = 0.0;
  for (int k = 1; k <= NW; ++k)
    for (int b1 = 0; b1 <= d; ++b1)
      for (int a0 = 0; a0 <= b1; ++a0) {
        const double prev = f[(size_t)(k - 1) * (d + 1) + a0];
        if (prev >= INF) continue;
        const double c = std::max(prev, rc[(size_t)a0 * (d + 1) + b1]);
        if (c < f[(size_t)k * (d + 1) + b1]) {
          f[(size_t)k * (d + 1) + b1] = c;
          arg[(size_t)k * (d + 1) + b1] = a0;
        }
      }
  std::vector<int> cut(NW + 1, d);
  cut[0] = 0;
  for (int k = NW, b1 = d; k >= 1; --k) {
    cut[k] = b1;
    b1 = arg[(size_t)k * (d + 1) + b1];
  }
  std::vector<int> sbit(NW), ebit(NW);
  for (int w = 0; w < NW; ++w) {
    sbit[w] = cut[w] < d ? hc.bit_off[cut[w]] : hc.code_bits;
    ebit[w] = cut[w + 1] < d ? hc.bit_off[cut[w + 1]] : hc.code_bits;
  }
  ebit[NW - 1] = 32 * hc.W;  // the last wave also covers QJL bits and gamma
  // words a wave stores straight from its bit window: wholly inside its code
  // bits (for the last wave with QJL, below the QJL bits)
  std::vector<int> dfirst(NW), dend(NW);
  for (int w = 0; w < NW; ++w) {
    const int ecode = (w == NW - 1 && hc.m > 0) ? hc.code_bits : ebit[w];
    dfirst[w] = (sbit[w] + 31) / 32;
    dend[w] = std::max(dfirst[w], ecode / 32);
    if (w == NW - 1 && hc.m == 0) dend[w] = std::max(dfirst[w], hc.W);
  }
  // every other word is OR-assembled in LDS and stored by the highest wave
  // that touches it
  std::vector<int> owner(hc.W, -1);
  for (int k = 0; k < hc.W; ++k) {
    bool direct = false;
    for (int w = 0; w < NW; ++w)
      if (k >= dfirst[w] && k < dend[w]) direct = true;
    if (direct) continue;
    owner[k] = NW - 1;
    for (int w = 0; w < NW; ++w)
      if (sbit[w] < ebit[w] && sbit[w] < 32 * (k + 1) && ebit[w] > 32 * k) owner[k] = w;
  }
  struct Ch { int start, cnt, b; };
  std::vector<std::vector<Ch>> wch(NW);
  for (int w = 0; w < NW; ++w)
    for (int i = cut[w]; i < cut[w + 1];) {
      int j = i;
      while (j < cut[w + 1] && hc.widths[j] == hc.widths[i]) ++j;
      // a run of equal width: chunks of 8, then the binary remainder
      for (int k = i; k < j;) {
        int n = 8;
        while (n > j - k) n >>= 1;
        const bool sig = hc.m > 0 && k < hc.d_eff;
        if (hc.widths[i] > 0 || sig) wch[w].push_back({k, n, hc.widths[i]});
        k += n;
      }
      i = j;
    }
  for (int w = 0; w < NW; ++w) P.n_chunks += (int)wch[w].size();
  P.words.assign((size_t)(NW + P.n_chunks + 1) * PLAN_WORDS, 0u);
  const float inf = std::numeric_limits<float>::infinity();
  // thresholds are compared through the sign of (threshold - y): store +0, never -0
  auto canon = [](float v) { return v == 0.0f ? 0.0f : v; };
  int q = 0;
  for (int w = 0; w < NW; ++w) {
    uint32_t *H = P.words.data() + (size_t)w * PLAN_WORDS;
    H[0] = (uint32_t)wch[w].size();
    H[1] = (uint32_t)sbit[w] | ((uint32_t)ebit[w] << 16);
    int f = -1, e = -1;
    for (int k = 0; k < hc.W; ++k)
      if (owner[k] == w) {
        if (f < 0) f = k;
        e = k + 1;
      }
    if (f < 0) f = e = 0;
    H[2] = (uint32_t)f | ((uint32_t)e << 16);
    H[3] = (uint32_t)dfirst[w] | ((uint32_t)dend[w] << 16);
    H[4] = (uint32_t)q;
    if (qin && w == 0) {
      int n_sig_chunks = 0;
      for (const Ch &ch : wch[w])
        if (ch.start < hc.d_eff) ++n_sig_chunks;
      H[5] = (uint32_t)n_sig_chunks;
    }
    for (const Ch &ch : wch[w]) {
      uint32_t *C = P.words.data() + (size_t)(NW + q) * PLAN_WORDS;
      const int b = ch.b, L = 1 << b;
      const int nsig = hc.m > 0 ? std::max(0, std::min(ch.cnt, hc.d_eff - ch.start)) : 0;
      C[8] = (uint32_t)(b > 0 ? P.tree.size() : 0);
      C[9] = (uint32_t)ch.start;
      C[10] = (uint32_t)ch.cnt;
      C[11] = (uint32_t)b;
      C[12] = (uint32_t)nsig;
      C[13] = (uint32_t)(nsig > 0 && b > 0 ? P.csig.size() : 0);
      C[14] = (uint32_t)(ch.cnt == 8 ? 3 : ch.cnt == 4 ? 2 : ch.cnt == 2 ? 1 : 0);
      for (int c = 0; c < 8; ++c) C[c] = f32_bits(inf);
      if (b > 0) {
        const size_t tb = P.tree.size();
        P.tree.resize(tb + (size_t)ch.cnt * L, inf);
        for (int c = 0; c < ch.cnt; ++c) {
          const int i = ch.start + c;
          // node n (depth k, position p = n - 2^k) holds sorted threshold
          // (2p + 1) * 2^(b - 1 - k) - 1
          for (int n = 1; n < L; ++n) {
            int k = 0;
            while ((2 << k) <= n) ++k;
            const int pos = n - (1 << k);
            P.tree[tb + (size_t)c * L + n - 1] =
                canon(hc.thr[hc.thr_base[i] + (2 * pos + 1) * (1 << (b - 1 - k)) - 1]);
          }
          C[c] = f32_bits(P.tree[tb + (size_t)c * L]);
        }
        if (nsig > 0) {
          const size_t cb = P.csig.size();
          P.csig.resize(cb + (size_t)ch.cnt * L, 0.0f);
          for (int c = 0; c < nsig; ++c)
            for (int k = 0; k < L; ++k)
              P.csig[cb + (size_t)c * L + k] = hc.cent[hc.cent_base[ch.start + c] + k];
        }
      }
      ++q;
    }
  }
  return P;
}

// Register-quantising compress plan (layout: P2_WAVE).  Groups of 4
// consecutive coordinates (depth = largest width) are dealt to the waves'
// accumulator registers largest depth first, each to the least loaded wave
// with a free register.
struct HostPlan2 {
  std::vector<uint32_t> words;
  std::vector<float> tree, csig;
  std::vector<int> row_coord;  // [d]: coordinate of MFMA row (w*16 + rho)
  bool ok = false;
};

static HostPlan2 build_plan2(const HeadCal &hc) {
  HostPlan2 P;
  const int d = hc.d;
  if (d != 32 && d != 64 && d != 128) return P;
  if (hc.m > 0 && (hc.d_eff > 16 || hc.m > 32)) return P;
  const int NW = d / 16, NG = d / 4;
  // Groups of 4 coordinates of equal width where possible (depth = the
  // largest width): each width class, in coordinate order, is cut into four
  // equal runs and group t takes the t-th coordinate of each run, so the four
  // codes of a group usually sit in different record words (the lane groups
  // of a register OR them into the record tile in one instruction); the
  // remainders of the classes are grouped by decreasing width.
  std::vector<int> byw(d);
  for (int c = 0; c < d; ++c) byw[c] = c;
  std::stable_sort(byw.begin(), byw.end(), [&](int x, int y) { return hc.widths[x] > hc.widths[y]; });
  std::vector<std::array<int, 4>> grp;
  std::vector<int> rest;
  for (int i = 0; i < d;) {
    int j = i;
    while (j < d && hc.widths[byw[j]] == hc.widths[byw[i]]) ++j;
    const int q = (j - i) / 4;
    for (int t = 0; t < q; ++t) grp.push_back({byw[i + t], byw[i + q + t], byw[i + 2 * q + t], byw[i + 3 * q + t]});
    for (int k = i + 4 * q; k < j; ++k) rest.push_back(byw[k]);
    i = j;
  }
  for (size_t k = 0; k < rest.size(); k += 4) grp.push_back({rest[k], rest[k + 1], rest[k + 2], rest[k + 3]});
  std::vector<int> depth(NG, 0);
  for (int g = 0; g < NG; ++g)
    for (int s = 0; s < 4; ++s) depth[g] = std::max(depth[g], hc.widths[grp[g][s]]);
  std::vector<int> order(NG);
  for (int g = 0; g < NG; ++g) order[g] = g;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return depth[x] > depth[y]; });
  std::vector<int> load(NW, 0), nslot(NW, 0), slot_g((size_t)NW * 4, -1);
  for (int g : order) {
    int best = -1;
    for (int w = 0; w < NW; ++w)
      if (nslot[w] < 4 && (best < 0 || load[w] < load[best])) best = w;
    slot_g[(size_t)best * 4 + nslot[best]++] = g;
    load[best] += 4 * depth[g] + 3;
  }
  // the kernel's descent relies on each wave's registers by decreasing depth
  for (int w = 0; w < NW; ++w)
    std::stable_sort(slot_g.begin() + (size_t)w * 4, slot_g.begin() + (size_t)w * 4 + 4,
                     [&](int x, int y) { return depth[x] > depth[y]; });
  const float inf = std::numeric_limits<float>::infinity();
  auto canon = [](float v) { return v == 0.0f ? 0.0f : v; };
  P.row_coord.assign(d, 0);
  std::vector<uint32_t> hdr((size_t)NW * P2_WAVE, 0u);
  for (int w = 0; w < NW; ++w) {
    uint32_t *H = hdr.data() + (size_t)w * P2_WAVE;
    for (int r = 0; r < 4; ++r) {
      const int g = slot_g[(size_t)w * 4 + r], D = depth[g], L = 1 << D;
      H[r] = (uint32_t)D;
      // the register's four trees start at 16 s (mod 64) words, so that the
      // nodes of one level (up to 16 of them per tree) that the four lane
      // groups read together fall in disjoint LDS banks
      const size_t stride = L - 1 <= 16 ? 16 : 16 + 64 * (((size_t)L - 1 - 16 + 63) / 64);
      const size_t rbase = (P.tree.size() + 63) & ~(size_t)63;
      if (D > 0) P.tree.resize(rbase + 4 * stride, inf);
      for (int s = 0; s < 4; ++s) {
        const int c = grp[g][s], b = hc.widths[c];
        P.row_coord[w * 16 + 4 * s + r] = c;
        H[36 + 4 * r + s] = (uint32_t)c;
        const size_t tb = D > 0 ? rbase + s * stride : 0;
        H[4 + 4 * r + s] = (uint32_t)tb;
        if (D > 0) {
          // sorted thresholds padded with +inf to L - 1; node n (depth k,
          // position p = n - 2^k) holds padded entry (2p + 1) * 2^(D - 1 - k) - 1
          std::vector<float> padded(L - 1, inf);
          for (int k = 0; k + 1 < (1 << b); ++k) padded[k] = canon(hc.thr[hc.thr_base[c] + k]);
          for (int n = 1; n < L; ++n) {
            int k = 0;
            while ((2 << k) <= n) ++k;
            const int pos = n - (1 << k);
            P.tree[tb + n - 1] = padded[(size_t)(2 * pos + 1) * (1 << (D - 1 - k)) - 1];
          }
        }
        if (hc.m > 0 && c < hc.d_eff) {
          const size_t cb = P.csig.size();
          H[20 + 4 * r + s] = (uint32_t)cb;
          P.csig.resize(cb + L, 0.0f);
          for (int k = 0; k < (1 << b) && b > 0; ++k) P.csig[cb + k] = hc.cent[hc.cent_base[c] + k];
        } else {
          H[20 + 4 * r + s] = 0xFFFFFFFFu;
        }
      }
    }
  }
  P.words = hdr;
  P.ok = P.tree.size() < 65536 && hc.W < 256;  // 16-bit tree bases, 8-bit word indices in the kernel
  return P;
}

sq_status upload_tables(sq_calib *c, void *stream) {
  const int nh = (int)c->heads.size();
  std::vector<HostPlan> plans(nh);
  for (int h = 0; h < nh; ++h) plans[h] = build_plan(c->heads[h]);
  std::vector<ScoreSched> scheds(nh);
  for (int h = 0; h < nh; ++h) scheds[h] = build_score_sched(c->heads[h]);
  std::vector<HostPlan2> plans2(nh);
  for (int h = 0; h < nh; ++h) plans2[h] = build_plan2(c->heads[h]);
  // host image of the blob: [DevHead x nh] then per-head sections
  std::vector<DevHead> desc(nh);
  size_t off = align256(sizeof(DevHead) * nh);
  for (int h = 0; h < nh; ++h) {
    const HeadCal &hc = c->heads[h];
    const HostPlan &P = plans[h];
    const int d = hc.d;
    DevHead &D = desc[h];
    std::memset(&D, 0, sizeof(D));
    D.d = d;
    D.d_eff = hc.d_eff;
    D.m = hc.m;
    D.W = hc.W;
    D.code_bits = hc.code_bits;
    D.n_tree = (int)P.tree.size();
    D.n_cent = hc.n_cent;
    D.has_gamma = hc.m > 0;
    D.qjl_scale = hc.m > 0 ? (float)(std::sqrt(M_PI / 2.0) / hc.m) : 0.0f;
    D.n_csig = (int)P.csig.size();
    D.n_chunks = P.n_chunks;
    D.n_quads = scheds[h].n_quads;
    D.n_plut = scheds[h].n_plut;
    D.off_R = off;       off = align256(off + sizeof(float) * d * d);
    D.off_RT = off;      off = align256(off + sizeof(float) * d * d);
    D.off_Rfrag = off;   off = align256(off + sizeof(uint16_t) * 3 * d * d);
    D.off_coord = off;   off = align256(off + sizeof(DevCoord) * d);
    D.off_tree = off;    off = align256(off + sizeof(float) * std::max<size_t>(1, P.tree.size()));
    D.off_cent = off;    off = align256(off + sizeof(float) * std::max(1, hc.n_cent));
    D.off_S = off;       off = align256(off + sizeof(float) * std::max(1, hc.m * hc.d_eff));
    D.off_plan = off;    off = align256(off + sizeof(uint32_t) * P.words.size());
    D.off_sched = off;   off = align256(off + sizeof(uint32_t) * scheds[h].quads.size());
    D.off_plut = off;    // read in whole 1 KB pieces: reserve them
    off = align256(off + ((sizeof(uint32_t) * scheds[h].lut.size() + 1023) & ~(size_t)1023));
    D.off_lutp = off;    off = align256(off + sizeof(uint32_t) * std::max(1, hc.n_cent));
    D.off_csig = off;    off = align256(off + sizeof(float) * std::max<size_t>(1, P.csig.size()));
    const HostPlan2 &P2 = plans2[h];
    D.n_p2 = P2.ok ? (int)P2.words.size() : 0;
    D.n_tree2 = (int)P2.tree.size();
    D.n_csig2 = (int)P2.csig.size();
    D.off_p2 = off;      off = align256(off + sizeof(uint32_t) * std::max<size_t>(1, P2.words.size()));
    D.off_tree2 = off;   off = align256(off + sizeof(float) * std::max<size_t>(1, P2.tree.size()));
    D.off_csig2 = off;   off = align256(off + sizeof(float) * std::max<size_t>(1, P2.csig.size()));
    D.off_Rfrag2 = off;  off = align256(off + (P2.ok ? sizeof(uint16_t) * 3 * d * d : 1));
  }
  std::vector<uint8_t> img(off, 0);
  std::memcpy(img.data(), desc.data(), sizeof(DevHead) * nh);
  for (int h = 0; h < nh; ++h) {
    const HeadCal &hc = c->heads[h];
    const DevHead &D = desc[h];
    const HostPlan &P = plans[h];
    const int d = hc.d;
    float *R = (float *)(img.data() + D.off_R);
    for (int k = 0; k < d * d; ++k) R[k] = (float)hc.R[k];
    float *RT = (float *)(img.data() + D.off_RT);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) RT[(size_t)j * d + i] = (float)hc.R[(size_t)i * d + j];
    // bf16 x3 split of R (hi + mid + lo reproduces R to ~2^-24 relative), laid
    // out as MFMA 16x16x32 A operands: fragment (s, mb, kb), lane l, element e
    // holds R_s[mb*16 + l%16][kb*32 + 8*(l/16) + e].
    uint16_t *F = (uint16_t *)(img.data() + D.off_Rfrag);
    const int MB = d / 16, KB = d / 32;
    for (int mb = 0; mb < MB; ++mb)
      for (int kb = 0; kb < KB; ++kb)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            const int row = mb * 16 + (l & 15), col = kb * 32 + 8 * (l >> 4) + e;
            double v = hc.R[(size_t)row * d + col];
            uint16_t parts[3];
            for (int s = 0; s < 3; ++s) {
              parts[s] = f32_to_bf16_rne((float)v);
              float back;
              uint32_t u = (uint32_t)parts[s] << 16;
              std::memcpy(&back, &u, 4);
              v -= (double)back;
            }
            for (int s = 0; s < 3; ++s)
              F[((((size_t)s * MB + mb) * KB + kb) * 64 + l) * 8 + e] = parts[s];
          }
    {
      const HostPlan2 &P2 = plans2[h];
      if (P2.ok) {
        std::memcpy(img.data() + D.off_p2, P2.words.data(), sizeof(uint32_t) * P2.words.size());
        if (!P2.tree.empty()) std::memcpy(img.data() + D.off_tree2, P2.tree.data(), sizeof(float) * P2.tree.size());
        if (!P2.csig.empty()) std::memcpy(img.data() + D.off_csig2, P2.csig.data(), sizeof(float) * P2.csig.size());
        // the bf16 x3 split of R with rows permuted: MFMA row w*16 + rho holds coordinate row_coord[...]
        uint16_t *F2 = (uint16_t *)(img.data() + D.off_Rfrag2);
        const uint16_t *F1 = (const uint16_t *)(img.data() + D.off_Rfrag);
        const int MB2 = d / 16, KB2 = d / 32;
        for (int sp = 0; sp < 3; ++sp)
          for (int mb = 0; mb < MB2; ++mb)
            for (int kb = 0; kb < KB2; ++kb)
              for (int l = 0; l < 64; ++l) {
                const int c = P2.row_coord[mb * 16 + (l & 15)];
                const int mb1 = c / 16, l1 = (c % 16) | (l & 48);
                std::memcpy(F2 + ((((size_t)sp * MB2 + mb) * KB2 + kb) * 64 + l) * 8,
                            F1 + ((((size_t)sp * MB2 + mb1) * KB2 + kb) * 64 + l1) * 8, 16);
              }
      }
    }
    DevCoord *Cd = (DevCoord *)(img.data() + D.off_coord);
    for (int i = 0; i < d; ++i) Cd[i] = DevCoord{hc.bit_off[i], hc.widths[i], hc.thr_base[i], hc.cent_base[i]};
    std::memcpy(img.data() + D.off_sched, scheds[h].quads.data(), sizeof(uint32_t) * scheds[h].quads.size());
    std::memcpy(img.data() + D.off_plut, scheds[h].lut.data(), sizeof(uint32_t) * scheds[h].lut.size());
    if (!P.tree.empty()) std::memcpy(img.data() + D.off_tree, P.tree.data(), sizeof(float) * P.tree.size());
    if (!P.csig.empty()) std::memcpy(img.data() + D.off_csig, P.csig.data(), sizeof(float) * P.csig.size());
    std::memcpy(img.data() + D.off_plan, P.words.data(), sizeof(uint32_t) * P.words.size());
    if (hc.n_cent) std::memcpy(img.data() + D.off_cent, hc.cent.data(), sizeof(float) * hc.n_cent);
    {
      uint32_t *Pp = (uint32_t *)(img.data() + D.off_lutp);
      for (int k = 0; k < hc.n_cent; ++k) {
        uint16_t hi, lo;
        bf16_split(hc.cent[k], hi, lo);
        Pp[k] = (uint32_t)hi | ((uint32_t)lo << 16);
      }
    }
    if (hc.m) std::memcpy(img.data() + D.off_S, hc.S.data(), sizeof(float) * hc.m * hc.d_eff);
  }
  release_tables(c);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  void *p = nullptr;
  e = hipMalloc(&p, off);
  if (e != hipSuccess) return fail(SQ_ERR_ALLOC, std::string("hipMalloc tables: ") + hipGetErrorString(e));
  hipStream_t s = (hipStream_t)stream;
  e = hipMemcpyAsync(p, img.data(), off, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail("table upload", e);
  }
  c->dev_blob = p;
  c->dev_heads = (DevHead *)p;
  c->host_desc = desc;
  c->dev_bytes = off;
  c->device = dev;
  return SQ_OK;
}

// ------------------------------------------------------------------ compress
//
// A workgroup of D/16 waves serves one calibration head and walks many
// 64-token tiles.
//   rotate:   wave w computes y^T[coord][token] = R x^T for eigen-coordinates
//             [16w, 16w+16) with MFMA 16x16x32 bf16.  R is split into three
//             bf16 terms (Henry, Tang & Heinecke, ARITH 2019: bf16x3) so every
//             product is exact in the fp32 accumulator; for head_dim <= 128 the
//             wave's 16 rows of the three terms stay in registers for the
//             workgroup's whole life, for 256 they are read per tile from the
//             L2.  fp32 inputs are split into three terms as well and the six
//             leading cross products are accumulated.  The x tile (B operand)
//             is shared through LDS; the accumulators go to an LDS y tile.
//   quantise: each wave owns a contiguous coordinate range (balanced on the
//             search cost, not tied to its MFMA rows) cut into chunks of 1, 2,
//             4 or 8 equal-width coordinates; lane = token, the chunk's binary
//             searches advance in lock-step (see quant_chunk) and its codes are
//             appended to a bit window that emits the record words.
//   pack:     words wholly inside one wave's code bits are stored from its
//             window; words shared between ranges are OR-ed together in LDS
//             and, after a barrier, stored by one wave, the last one adding
//             the QJL bits z_j = [(S r)_j >= 0] and gamma = |r| as IEEE half
//             in word W-1.  Every store is one coalesced 256-byte row.

struct CompressArgs {
  const DevHead *heads;
  const uint8_t *blob;
  const void *x;
  uint32_t *packed;
  int64_t xs_b, xs_h, xs_t;
  int64_t ps_b, ps_h;
  int64_t n_tokens;
  int64_t token0;       // source token i goes to token slot token0 + i
  int first_head, cbs;
  int n_tiles;          // ceil(T / 64) per (batch, head)
  int items;            // tiles one head's workgroups share
  int lds_csig_off;     // floats: signal-centroid table (after the trees)
  int lds_plan_off;     // floats: the head's compress plan
  int lds_s_off;        // floats: QJL sketch S [m][d_eff], or -1: read from the table blob
  int lds_sp_off;       // floats: S zero-padded to [8][8] (used when m, d_eff <= 8)
  int lds_x_off;        // floats: x tile
  int lds_y_off;        // floats: y tile; residuals replace y in place
  int lds_b_off;        // floats: shared record-word buffer
  int ys;               // y tile row stride (floats, d + 3)
  int bws;              // word buffer row stride (words, odd)
};

__device__ __forceinline__ void split3(const float *v, uint4 &p0, uint4 &p1, uint4 &p2) {
  uint16_t a[8], b[8], c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = v[e];
    a[e] = f32_to_bf16_rne(x);
    x -= __uint_as_float((uint32_t)a[e] << 16);
    b[e] = f32_to_bf16_rne(x);
    x -= __uint_as_float((uint32_t)b[e] << 16);
    c[e] = f32_to_bf16_rne(x);
  }
  p0 = make_uint4(a[0] | (a[1] << 16), a[2] | (a[3] << 16), a[4] | (a[5] << 16), a[6] | (a[7] << 16));
  p1 = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
  p2 = make_uint4(c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16), c[6] | (c[7] << 16));
}

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Wait for this wave's LDS operations and keep the compiler from moving LDS
// accesses across this point (cross-lane exchange within one wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Bit window of one wave's record words while it appends code fields:
// bits [0, fill) of lo are filled; lo is word kw of the record.
struct PackWin {
  uint32_t lo;
  int fill, kw;
};

// Emit the window's full word into the LDS word buffer and move on to the
// next one.  A word wholly inside the wave's code bits is written; a word
// shared with another wave's range is OR-ed in.
__device__ __forceinline__ void win_flush(PackWin &pw, uint32_t next, uint32_t *bwrow, int dfirst,
                                          int dend) {
  if (pw.kw >= dfirst && pw.kw < dend) bwrow[pw.kw] = pw.lo;
  else atomicOr(bwrow + pw.kw, pw.lo);
  ++pw.kw;
  pw.lo = next;
  pw.fill -= 32;
}

// One chunk of NS (1, 2, 4 or 8) coordinates of equal width B (lane =
// token).  The NS searches advance together down their breadth-first trees:
// the root comes from a scalar register, each further level is one table
// read at a compile-time offset; the step is decided by the sign of
// (threshold - y), so a tie goes to the lower cell and the code is
// #{thresholds < y}.  NaN coordinates are mapped to -inf first (code 0).
// The chunk's NS * B code bits are assembled at compile-time shifts into one
// 64-bit value and appended to the window at once.  Residuals of signal
// coordinates replace y in the tile.
struct ChunkArgs {
  float root[8];  // per coordinate (wave-uniform values)
  int tbase, start, nsig, cbase;
};

// Running QJL sums of the wave that holds the signal range: the dots
// (S r)_j and |r|^2, from residuals still in registers.
struct QjlAcc {
  float dot[8];
  float g2;
};

template <int B, int NS, bool TG, bool QJ>
__device__ __forceinline__ void quant_chunk(const ChunkArgs &cd, float *yrow, const float *trees,
                                            const float *csig, PackWin &pw, uint32_t *bwrow,
                                            int dfirst, int dend, const float *sp, QjlAcc &qa) {
  constexpr int L = 1 << B;
  const int start = cd.start, nsig = cd.nsig;
  float y[NS];
  uint32_t code[NS];
  const float *ys = yrow + start;
#pragma unroll
  for (int c = 0; c < NS; ++c) y[c] = fmaxf(ys[c], -INFINITY);
  if constexpr (B > 0) {
#pragma unroll
    for (int c = 0; c < NS; ++c) code[c] = __float_as_uint(cd.root[c] - y[c]) >> 31;
    const float *tb = trees + cd.tbase;
#pragma unroll
    for (int l = 1; l < B; ++l) {
      float th[NS];
#pragma unroll
      for (int c = 0; c < NS; ++c) th[c] = tb[c * L + (1 << l) - 1 + (int)code[c]];
#pragma unroll
      for (int c = 0; c < NS; ++c)
        code[c] = __builtin_amdgcn_alignbit(code[c], __float_as_uint(th[c] - y[c]), 31);
    }
    uint32_t v0 = 0u, v1 = 0u;
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const int sh = c * B;
      if (sh < 32) {
        v0 |= code[c] << sh;
        if (sh + B > 32) v1 |= code[c] >> (32 - sh);
      } else {
        v1 |= code[c] << (sh - 32);
      }
    }
    // append the NS * B bits of (v1:v0) at bit fill of the window; the
    // double shifts keep every shift count below 32
    const int f = pw.fill;
    pw.lo |= v0 << f;
    uint32_t w1 = (v0 >> 1) >> (31 - f);
    uint32_t w2 = 0u;
    if constexpr (NS * B > 32) {
      w1 |= v1 << f;
      w2 = (v1 >> 1) >> (31 - f);
    }
    pw.fill += NS * B;
    if (pw.fill >= 32) {
      win_flush(pw, w1, bwrow, dfirst, dend);
      if constexpr (NS * B > 32) {
        if (pw.fill >= 32) win_flush(pw, w2, bwrow, dfirst, dend);
      }
    }
  }
  if (nsig > 0) {
    const float *cs = csig + cd.cbase;
#pragma unroll
    for (int c = 0; c < NS; ++c)
      if (c < nsig) {
        float r = ys[c];  // (a NaN y keeps a NaN residual: no QJL bit, NaN gamma)
        if constexpr (B > 0) r -= cs[c * L + code[c]];
        if constexpr (QJ) {  // signal coordinate start + c < 8: column of the padded sketch
          qa.g2 = fmaf(r, r, qa.g2);
#pragma unroll
          for (int j = 0; j < 8; ++j) qa.dot[j] = fmaf(sp[j * 8 + start + c], r, qa.dot[j]);
        } else {
          yrow[start + c] = r;
        }
      }
  }
}

template <int B, bool TG, bool QJ>
__device__ __forceinline__ void quant_chunk_ns(int lg, const ChunkArgs &cd, float *yrow,
                                               const float *trees, const float *csig, PackWin &pw,
                                               uint32_t *bwrow, int dfirst, int dend,
                                               const float *sp, QjlAcc &qa) {
  switch (lg) {
    case 0: quant_chunk<B, 1, TG, QJ>(cd, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 1: quant_chunk<B, 2, TG, QJ>(cd, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 2: quant_chunk<B, 4, TG, QJ>(cd, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    default: quant_chunk<B, 8, TG, QJ>(cd, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
  }
}

// Decode one chunk descriptor (four 16-byte words from the LDS plan) and run
// the chunk's quantiser for its width and size.
template <bool TG, bool QJ>
__device__ __forceinline__ void run_chunk(uint4 c0, uint4 c1, uint4 c2, uint4 c3, float *yrow,
                                          const float *trees, const float *csig, PackWin &pw,
                                          uint32_t *bwrow, int dfirst, int dend, const float *sp,
                                          QjlAcc &qa) {
  ChunkArgs ca;
  ca.root[0] = __uint_as_float(c0.x); ca.root[1] = __uint_as_float(c0.y);
  ca.root[2] = __uint_as_float(c0.z); ca.root[3] = __uint_as_float(c0.w);
  ca.root[4] = __uint_as_float(c1.x); ca.root[5] = __uint_as_float(c1.y);
  ca.root[6] = __uint_as_float(c1.z); ca.root[7] = __uint_as_float(c1.w);
  ca.tbase = __builtin_amdgcn_readfirstlane(c2.x);
  ca.start = __builtin_amdgcn_readfirstlane(c2.y);
  const int bw = __builtin_amdgcn_readfirstlane(c2.w);
  ca.nsig = __builtin_amdgcn_readfirstlane(c3.x);
  ca.cbase = __builtin_amdgcn_readfirstlane(c3.y);
  const int lg = __builtin_amdgcn_readfirstlane(c3.z);  // log2 of the coordinate count
  switch (bw) {
    case 0: quant_chunk_ns<0, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 1: quant_chunk_ns<1, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 2: quant_chunk_ns<2, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 3: quant_chunk_ns<3, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 4: quant_chunk_ns<4, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 5: quant_chunk_ns<5, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 6: quant_chunk_ns<6, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    case 7: quant_chunk_ns<7, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
    default: quant_chunk_ns<8, TG, QJ>(lg, ca, yrow, trees, csig, pw, bwrow, dfirst, dend, sp, qa); break;
  }
}

// At least 4 waves per SIMD (<= 128 VGPRs): two workgroups per CU for
// head_dim 128, and what a 16-wave workgroup needs for 256.
template <int D, bool F32, bool TG>
__global__ __launch_bounds__(D * 4, 4) void compress_kernel(CompressArgs a) {
  extern __shared__ float smem[];
  constexpr int NW = D / 16, KB = D / 32, MB = D / 16, NT = 64 * NW;
  constexpr bool RES = D <= 128;           // rotation rows resident in registers
  constexpr int XS = F32 ? D + 4 : D + 8;  // x tile row stride (elements)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int h = blockIdx.y, bz = blockIdx.z;
  const int ch = a.first_head + bz * a.cbs + h;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d_eff = hd->d_eff, m = hd->m, W = hd->W, code_bits = hd->code_bits;
  float *ytile = smem + a.lds_y_off;             // [64][ys]
  uint32_t *bwords = (uint32_t *)(smem + a.lds_b_off);  // [64][bws] shared record words
  const float *trees;
  float *s_csig = smem + a.lds_csig_off;
  {
    const int n_tree = hd->n_tree, n_csig = hd->n_csig;
    const float *g_tree = (const float *)(a.blob + hd->off_tree);
    if constexpr (TG) {
      trees = g_tree;
    } else {
      for (int k = threadIdx.x; k < n_tree; k += NT) smem[k] = g_tree[k];
      trees = smem;
    }
    const float *g_csig = (const float *)(a.blob + hd->off_csig);
    for (int k = threadIdx.x; k < n_csig; k += NT) s_csig[k] = g_csig[k];
    const uint32_t *g_plan = (const uint32_t *)(a.blob + hd->off_plan);
    uint32_t *s_plan = (uint32_t *)(smem + a.lds_plan_off);
    const int n_plan = (NW + hd->n_chunks + 1) * PLAN_WORDS;
    for (int k = threadIdx.x; k < n_plan; k += NT) s_plan[k] = g_plan[k];
    const float *g_S = (const float *)(a.blob + hd->off_S);
    if (a.lds_s_off >= 0)
      for (int k = threadIdx.x; k < hd->m * hd->d_eff; k += NT) smem[a.lds_s_off + k] = g_S[k];
    if (threadIdx.x < 64) {
      const int j = threadIdx.x >> 3, i = threadIdx.x & 7;
      smem[a.lds_sp_off + threadIdx.x] = (j < hd->m && i < hd->d_eff) ? g_S[j * hd->d_eff + i] : 0.0f;
    }
  }
  const uint4 *Rf = (const uint4 *)(a.blob + hd->off_Rfrag);
  uint4 rf[RES ? 3 : 1][RES ? KB : 1];
  if constexpr (RES) {
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) rf[sp][kb] = Rf[((sp * MB + w) * KB + kb) * 64 + lane];
  }
  const SQ_CONST uint32_t *plan = cptr<uint32_t>(a.blob + hd->off_plan);
  const float *S_lds = smem + max(0, a.lds_s_off);
  const SQ_CONST float *S_glb = cptr<float>(a.blob + hd->off_S);
  const int64_t T = a.n_tokens;
  const SQ_CONST uint32_t *hdr = plan + w * PLAN_WORDS;
  const int nch = (int)hdr[0];
  const int sbit = (int)(hdr[1] & 0xFFFF);
  const int own_f = (int)(hdr[2] & 0xFFFF), own_e = (int)(hdr[2] >> 16);
  const int dfirst = (int)(hdr[3] & 0xFFFF), dend = (int)(hdr[3] >> 16);
  const int nsc = (int)hdr[5];  // leading chunks with signal coordinates (small sketch, wave 0)
  // chunk descriptors are read from the LDS copy of the plan: in-order LDS
  // reads leave the compiler exact partial waits for the search reads
  const uint4 *chunks = (const uint4 *)(smem + a.lds_plan_off) + (NW + (int)hdr[4]) * (PLAN_WORDS / 4);

  // x tile chunks of 16 bytes: CPR per row, CH per thread; the next tile's
  // chunks are prefetched into registers while the current tile is processed
  constexpr int ESZ = F32 ? 4 : 2;
  constexpr int CPR = D * ESZ / 16;
  constexpr int CH = 64 * CPR / NT;
  uint4 xr[CH];
  auto load_x = [&](int item) {
    const int bb = a.cbs ? bz : item / a.n_tiles;
    const int tl = a.cbs ? item : item % a.n_tiles;
    const char *xp = (const char *)a.x + ((int64_t)bb * a.xs_b + (int64_t)h * a.xs_h) * ESZ;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int c = threadIdx.x + q * NT;
      const int tt = c / CPR, col = c % CPR;
      const int64_t t = (int64_t)tl * 64 + tt;
      xr[q] = t < T ? *(const uint4 *)(xp + t * a.xs_t * ESZ + col * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  if (blockIdx.x < a.items) load_x(blockIdx.x);
  // The record words of a tile are assembled in the LDS word buffer and stored
  // at the top of the next tile, before the next prefetch is issued: each
  // wait for a prefetch then covers only memory operations issued a whole
  // tile earlier.  A wave stores the words it finalises (its direct words and
  // the shared words it owns) and zeroes the shared ones for the next tile.
  for (int k = threadIdx.x; k < 64 * a.bws; k += NT) bwords[k] = 0u;
  uint32_t *const bwrow = bwords + lane * a.bws;
  uint32_t *pdst = nullptr;  // destination of the previous tile's records
  bool pvalid = false, pin = false;
  // Source token i lands in slot token token0 + i: lane l of a source tile
  // writes destination lane (token0 + l) % 64 of its tile or of the next.
  // Lanes past the last token zero their words up to the end of the last
  // destination tile and write nothing beyond it.
  const int ol = (int)(a.token0 & 63) + lane;
  const int64_t lofs = (int64_t)(ol >> 6) * W * 64 + (ol & 63);
  const int64_t send = ((a.token0 + T + 63) & ~(int64_t)63) - a.token0;
  auto store_prev = [&]() {
    for (int k = dfirst; k < dend; ++k)
      if (pin) pdst[(int64_t)k * 64] = pvalid ? bwrow[k] : 0u;
    for (int k = own_f; k < own_e; ++k) {
      if (k >= dfirst && k < dend) continue;
      if (pin) pdst[(int64_t)k * 64] = pvalid ? bwrow[k] : 0u;
      bwrow[k] = 0u;
    }
  };

  for (int item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int b = a.cbs ? bz : item / a.n_tiles;
    const int tile = a.cbs ? item : item % a.n_tiles;
    const int64_t t0 = (int64_t)tile * 64;
    // ---- prefetched x tile -> LDS, previous tile's records -> HBM, then
    // start loading the next tile
    {
      char *xt = (char *)(smem + a.lds_x_off);
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = threadIdx.x + q * NT;
        *(uint4 *)(xt + (c / CPR) * XS * ESZ + (c % CPR) * 16) = xr[q];
      }
    }
    if (pdst) store_prev();
    __syncthreads();
    if (item + (int)gridDim.x < a.items) load_x(item + gridDim.x);
    // ---- rotate this wave's 16 coordinates for the 64 tokens (4 blocks of 16)
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint4 r0, r1, r2;
      if constexpr (RES) {
        r0 = rf[0][kb]; r1 = rf[1][kb]; r2 = rf[2][kb];
      } else {
        r0 = Rf[((0 * MB + w) * KB + kb) * 64 + lane];
        r1 = Rf[((1 * MB + w) * KB + kb) * 64 + lane];
        r2 = Rf[((2 * MB + w) * KB + kb) * 64 + lane];
      }
      const int koff = kb * 32 + 8 * (lane >> 4);
      if constexpr (!F32) {
        const uint16_t *xt = (const uint16_t *)(smem + a.lds_x_off);
        uint4 xv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = *(const uint4 *)(xt + (16 * j + (lane & 15)) * XS + koff);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16(r0, xv[j], acc[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16(r1, xv[j], acc[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16(r2, xv[j], acc[j]);
      } else {
        const float *xt = smem + a.lds_x_off;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float *src = xt + (16 * j + (lane & 15)) * XS + koff;
          float v[8];
          const float4 u0 = *(const float4 *)src, u1 = *(const float4 *)(src + 4);
          v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
          v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
          uint4 x0, x1, x2;
          split3(v, x0, x1, x2);
          acc[j] = mfma16(r0, x0, acc[j]);
          acc[j] = mfma16(r0, x1, acc[j]);
          acc[j] = mfma16(r1, x0, acc[j]);
          acc[j] = mfma16(r0, x2, acc[j]);
          acc[j] = mfma16(r2, x0, acc[j]);
          acc[j] = mfma16(r1, x1, acc[j]);
        }
      }
    }
    // accumulators (row = coordinate, column = token) -> y tile [token][coordinate]
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ytile[(16 * j + (lane & 15)) * a.ys + 16 * w + 4 * (lane >> 4) + r] = acc[j][r];
    __syncthreads();
    // ---- quantise + pack (lane = token), chunk by chunk through the plan,
    // into the LDS word buffer.  With a small sketch (m, d_eff <= 8) wave 0
    // holds the whole signal range and adds the QJL bits and gamma itself.
    float *yrow = ytile + lane * a.ys;
    const bool qin = m > 0 && m <= 8 && d_eff <= 8 && w == 0;
    const float *sp = smem + a.lds_sp_off;
    {
      PackWin pw{0u, sbit & 31, sbit >> 5};
      int q = 0;
      if (qin) {  // the leading signal chunks, then the QJL bits and gamma
        QjlAcc qa;
#pragma unroll
        for (int j = 0; j < 8; ++j) qa.dot[j] = 0.0f;
        qa.g2 = 0.0f;
        for (; q < nsc; ++q)
          run_chunk<TG, true>(chunks[q * 4], chunks[q * 4 + 1], chunks[q * 4 + 2], chunks[q * 4 + 3],
                              yrow, trees, s_csig, pw, bwrow, dfirst, dend, sp, qa);
        uint32_t z = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) z |= (j < m && qa.dot[j] >= 0.0f ? 1u : 0u) << j;
        const int k0 = code_bits >> 5, sh = code_bits & 31;
        atomicOr(bwrow + k0, z << sh);
        if (sh + m > 32) atomicOr(bwrow + k0 + 1, z >> (32 - sh));
        atomicOr(bwrow + W - 1, half_bits_rne(sqrtf(qa.g2)) << 16);
      }
      QjlAcc no_qjl;  // unused by the chunks below
      uint4 nx[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) nx[k] = chunks[q * 4 + k];
      for (; q < nch; ++q) {
        const uint4 c0 = nx[0], c1 = nx[1], c2 = nx[2], c3 = nx[3];
#pragma unroll
        for (int k = 0; k < 4; ++k) nx[k] = chunks[(q + 1) * 4 + k];  // the plan ends with a spare chunk
        run_chunk<TG, false>(c0, c1, c2, c3, yrow, trees, s_csig, pw, bwrow, dfirst, dend, sp, no_qjl);
      }
      if (pw.fill > 0) {  // last, partial word of the range
        if (pw.kw >= dfirst && pw.kw < dend) bwrow[pw.kw] = pw.lo;
        else atomicOr(bwrow + pw.kw, pw.lo);
      }
    }
    __syncthreads();
    // ---- larger sketches: the last wave adds the QJL bits and gamma to the
    // words it owns, from the residuals, which replaced y of the signal
    // coordinates in the tile
    const bool qslow = m > 0 && !(m <= 8 && d_eff <= 8);
    for (int k = own_f; k < own_e && qslow && w == NW - 1; ++k) {
      if (k >= dfirst && k < dend) continue;
      uint32_t word = bwrow[k];
      {
        const int lo_bit = 32 * k, hi_bit = lo_bit + 32;
        const int jb = max(0, lo_bit - code_bits), je = min(m, hi_bit - code_bits);
        for (int j = jb; j < je; ++j) {
          float dot = 0.0f;
          if (a.lds_s_off >= 0) {
            for (int i = 0; i < d_eff; ++i) dot = fmaf(S_lds[j * d_eff + i], yrow[i], dot);
          } else {
            for (int i = 0; i < d_eff; ++i) dot = fmaf(S_glb[j * d_eff + i], yrow[i], dot);
          }
          word |= (dot >= 0.0f ? 1u : 0u) << (code_bits + j - lo_bit);
        }
        if (k == W - 1) {
          float g2 = 0.0f;
          for (int i = 0; i < d_eff; ++i) g2 = fmaf(yrow[i], yrow[i], g2);
          word |= half_bits_rne(sqrtf(g2)) << 16;
        }
      }
      bwrow[k] = word;
    }
    pdst = a.packed + (int64_t)b * a.ps_b + (int64_t)h * a.ps_h + ((a.token0 >> 6) + tile) * W * 64 + lofs;
    pvalid = t0 + lane < T;
    pin = t0 + lane < send;
    // The x tile was last read by the MFMAs, which every wave finished before
    // the barrier above; the y tile and the word buffer are rewritten only
    // after the barrier that follows the next x store.
  }
  if (pdst) store_prev();
}

// s_waitcnt vmcnt(n) for a wave-uniform n (the counter field is an immediate)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define SQ_VMW(k) \
  case k: __builtin_amdgcn_s_waitcnt(0x0F70 | ((k) & 15) | (((k) >> 4) << 14)); break;
#define SQ_VMW8(k) SQ_VMW(k) SQ_VMW(k + 1) SQ_VMW(k + 2) SQ_VMW(k + 3) SQ_VMW(k + 4) SQ_VMW(k + 5) SQ_VMW(k + 6) SQ_VMW(k + 7)
    SQ_VMW8(0) SQ_VMW8(8) SQ_VMW8(16) SQ_VMW8(24) SQ_VMW8(32) SQ_VMW8(40) SQ_VMW8(48) SQ_VMW8(56)
#undef SQ_VMW8
#undef SQ_VMW
    default: __builtin_amdgcn_s_waitcnt(0xCF7F); break;  // vmcnt(63): waits for more, never less
  }
}

// workgroup barrier without the memory fence of __syncthreads (the producer
// must not wait for its later loads); LDS writes of the wave are complete.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS loads (global_load_lds_dword / _dwordx4): lane l's 4 (16)
// bytes land at LDS address lds + 4l (16l).  Written as asm so that the
// compiler does not treat every later LDS read of the workgroup as a possible
// reader of these writes (it would wait for all vector memory there); the
// loads are ordered explicitly by wait_vmcnt and step_barrier.  They have no
// register results.
// Address = wave-uniform base (scalar pair) + per-lane byte offset.
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void *base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
// a wave-uniform value kept in a vector register (it is combined with
// another uniform operand in one VOP3 instruction, which takes one scalar)
__device__ __forceinline__ uint32_t to_vgpr(uint32_t x) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(x));
  return v;
}

// ------------------------------------------------------------------ compress, register quantiser
//
// Same contract as compress_kernel, for head_dim 32, 64 and 128 with at most
// 16 signal coordinates and 32 QJL rows.  A workgroup of d/16 waves serves
// one calibration head and walks 64-token tiles with one barrier per tile:
//   rotate:   wave w forms its 16 MFMA rows of y^T for the tile (16x16x32 bf16,
//             R as three bf16 terms in registers); its rows are the four
//             coordinate groups of the register plan (P2_WAVE), so lane l
//             holds in accumulator register r the values of one coordinate
//             for tokens l % 16 + 16 j.
//   quantise: straight from the accumulators: 16 descents per wave of the
//             lanes' own padded threshold trees in LDS, advancing level by
//             level together; each code is OR-ed into its record word(s) in
//             an LDS record tile [token][word], and signal residuals
//             y - C[code] go to a small float tile.
//   store:    after the barrier wave w stores record words w, w + d/16, ... as
//             coalesced 256-byte rows (lane = token) and clears them, except
//             the words with QJL bits or gamma: every wave first adds its
//             share of the QJL rows (and one wave gamma) from the residual
//             tile, and those words are stored after the next barrier.
// x tiles are double-buffered and fetched two tiles ahead; the record tile
// is triple-buffered, the residual tile double-buffered, so the barrier of
// tile t also separates tile t+1's writes from the reads of tiles t-1, t-2.

struct Compress2Args {
  const DevHead *heads;
  const uint8_t *blob;
  const void *x;
  uint32_t *packed;
  int64_t xs_b, xs_h, xs_t;
  int64_t ps_b, ps_h;
  int64_t n_tokens;
  int64_t token0;             // source token i goes to token slot token0 + i
  int first_head, cbs;
  int n_tiles, tiles_per_wg;  // workgroup (x, head, batch entry) takes tiles [x * tiles_per_wg, ...)
  int lds_tree_off, lds_csig_off, lds_s_off, lds_x_off, lds_rec_off, lds_res_off;  // floats
  int x_buf_floats;
};

constexpr int C2_RS = 20;   // residual tile row stride (floats; 16-byte rows, conflict-free)
constexpr int C2_SP = 16;   // sketch row pitch in LDS (floats, zero padded past d_eff)
constexpr int C2_WMAX = 6;  // record words stored per wave and tile (word k goes to wave k % waves)

// RS: record tile row stride in words (odd, above the record length: the
// last column is a pad), a constant so that token-block offsets are immediates
template <int D, bool F32, int RS>
__global__ __launch_bounds__(D * 4, 4) void compress2_kernel(Compress2Args a) {
  extern __shared__ float smem[];
  constexpr int NW = D / 16, KB = D / 32, MB = D / 16, NT = 64 * NW;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y, bz = blockIdx.z;
  const int tb = blockIdx.x * a.tiles_per_wg, te = min(a.n_tiles, tb + a.tiles_per_wg);
  if (tb >= te) return;  // (whole workgroup)
  const int ch = a.first_head + bz * a.cbs + h;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d_eff = hd->d_eff, m = hd->m, W = hd->W, code_bits = hd->code_bits;
  constexpr int rs = RS;
  float *trees = smem + a.lds_tree_off;
  float *csig = smem + a.lds_csig_off;
  float *Sl = smem + a.lds_s_off;  // [m][C2_SP]
  {
    const float *g = (const float *)(a.blob + hd->off_tree2);
    for (int k = threadIdx.x; k < hd->n_tree2; k += NT) trees[k] = g[k];
    const float *gc = (const float *)(a.blob + hd->off_csig2);
    for (int k = threadIdx.x; k < hd->n_csig2; k += NT) csig[k] = gc[k];
    const float *gs = (const float *)(a.blob + hd->off_S);
    for (int k = threadIdx.x; k < m * C2_SP; k += NT)
      Sl[k] = (k % C2_SP) < d_eff ? gs[(k / C2_SP) * d_eff + k % C2_SP] : 0.0f;
  }
  const SQ_CONST uint32_t *H = cptr<uint32_t>(a.blob + hd->off_p2) + w * P2_WAVE;
  const int s4 = lane >> 4;
  int dep[4];
  // per lane and register: tree base | (record word | bit shift << 8 |
  // straddles << 13) << 16; coordinate | signal-centroid base << 8 (0xFFFFFF: none)
  uint32_t tw[4], cc[4];
  {
    const uint32_t *Hv = (const uint32_t *)(a.blob + hd->off_p2) + w * P2_WAVE;  // per-lane reads
    const DevCoord *cd = (const DevCoord *)(a.blob + hd->off_coord);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dep[r] = (int)H[r];
      const uint32_t cb = Hv[20 + 4 * r + s4], c = Hv[36 + 4 * r + s4];
      cc[r] = c | ((cb == 0xFFFFFFFFu ? 0xFFFFFFu : cb) << 8);
      const int bo = cd[c].bit_off, wd = cd[c].width;
      const uint32_t wsh = (uint32_t)(bo >> 5) | ((uint32_t)(bo & 31) << 8) | ((bo & 31) + wd > 32 ? 1u << 13 : 0u);
      tw[r] = Hv[4 + 4 * r + s4] | (wsh << 16);
    }
  }
  // record words of this wave: w, w + NW, ...; qmask bit i: word w + NW i holds
  // QJL bits or gamma (stored one tile late, once every wave has added its bits)
  uint32_t qmask = 0u;
#pragma unroll
  for (int i = 0; i < C2_WMAX; ++i) {
    const int k = w + NW * i;
    if (m > 0 && k < W && ((32 * k < code_bits + m && 32 * k + 32 > code_bits) || k == W - 1)) qmask |= 1u << i;
  }
  // QJL rows of this wave (all 64 tokens): [jb, je)
  const int jb = (w * m) / NW, je = ((w + 1) * m) / NW;
  const uint4 *Rf = (const uint4 *)(a.blob + hd->off_Rfrag2);
  uint4 rf[3][KB];
#pragma unroll
  for (int sp = 0; sp < 3; ++sp)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) rf[sp][kb] = Rf[((sp * MB + w) * KB + kb) * 64 + lane];

  // x tiles go straight into LDS, 1 KB per load instruction, rows of RB
  // bytes back to back; chunk c (16 bytes) of row t sits at slot c ^ swz(t)
  // of the row, which keeps the MFMA operand reads free of bank conflicts
  // (measured: a 16-byte row pad instead doubles their LDS time).
  constexpr int ESZ = F32 ? 4 : 2;
  constexpr int RB = D * ESZ;                    // bytes of x per token
  constexpr int CPR = RB / 16;                   // 16-byte chunks per token
  constexpr int RPB = CPR >= 16 ? 1 : 16 / CPR;  // rows per 256 bytes
  constexpr int NB = CPR / NW;                   // 1 KB blocks per wave and tile
  const uint32_t lds_x = (uint32_t)(uintptr_t)(smem + a.lds_x_off);
  const uint32_t row_bytes = (uint32_t)a.xs_t * ESZ;  // 64 rows fit 32 bits (host check)
  const char *xbase = (const char *)a.x + ((int64_t)bz * a.xs_b + (int64_t)h * a.xs_h) * ESZ;
  auto dma_x = [&](int tl, int buf) __attribute__((always_inline)) {
    // rows past the end re-read the last token (a whole tile past it, which
    // only zero-fills destination words, reads nothing else)
    const int64_t t0 = min<int64_t>((int64_t)tl * 64, a.n_tokens - 1);
    const char *src = xbase + t0 * a.xs_t * ESZ;
    const int last = (int)min<int64_t>(63, a.n_tokens - 1 - t0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = w * NB + i;
      const int byte = q * 1024 + lane * 16, row = byte / RB, slot = (byte % RB) / 16;
      const int c = slot ^ ((row / RPB) & (CPR - 1));
      lds_dma16(src, (uint32_t)min(row, last) * row_bytes + (uint32_t)c * 16u,
                lds_x + (uint32_t)buf * (uint32_t)a.x_buf_floats * 4u + (uint32_t)q * 1024u);
    }
  };
  for (int k = threadIdx.x; k < 3 * 64 * rs; k += NT) smem[a.lds_rec_off + k] = 0.0f;
  // residual columns past d_eff stay zero (the QJL step reads whole rows)
  for (int k = threadIdx.x; k < 2 * 64 * C2_RS; k += NT) smem[a.lds_res_off + k] = 0.0f;
  // All set-up loads complete here, so that no wait inside the tile loop has
  // to cover them.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  dma_x(tb, 0);
  if (tb + 1 < te) dma_x(tb + 1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // the lane's operand rows are 16 j + lane % 16: their swizzle is a lane constant for bf16
  const int xsw = ((lane & 15) / RPB) & (CPR - 1);
  const uint32_t xrow = (uint32_t)(lane & 15) * RB;
  uint32_t *rec0 = (uint32_t *)(smem + a.lds_rec_off);
  // source token i lands in slot token token0 + i: lane l of a source tile
  // writes destination lane (token0 + l) % 64 of its tile or of the next;
  // lanes past the last token zero their words up to the end of the last
  // destination tile and write nothing beyond it
  uint32_t *obase = a.packed + (int64_t)bz * a.ps_b + (int64_t)h * a.ps_h + (a.token0 >> 6) * W * 64;
  const int ol = (int)(a.token0 & 63) + lane;
  const uint32_t lofs = (uint32_t)((ol >> 6) * W * 64 + (ol & 63));
  const int64_t send = ((a.token0 + a.n_tokens + 63) & ~(int64_t)63) - a.token0;
  // record words of this wave: w + NW i for i < nmine
  const int nmine = W > w ? (W - 1 - w) / NW + 1 : 0;
  int par = 0, rb = 0;
  for (int t = tb; t < te; ++t, par ^= 1, rb = rb == 2 ? 0 : rb + 1) {
    // ---- rotate: 16 rows x 64 tokens (4 blocks of 16)
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const char *xt = (const char *)(smem + a.lds_x_off + par * a.x_buf_floats) + xrow;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 r0 = rf[0][kb], r1 = rf[1][kb], r2 = rf[2][kb];
      if constexpr (!F32) {
        uint4 xv[4];  // elements kb*32 + 8*(lane/16) .. (chunk kc) of token 16j + lane%16
        const char *xc = xt + (((kb * 4 + (lane >> 4)) ^ xsw) << 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = *(const uint4 *)(xc + 16 * j * RB);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16(r0, xv[j], acc[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16(r1, xv[j], acc[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16(r2, xv[j], acc[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v[8];
          const int kc = kb * 8 + 2 * (lane >> 4), sw = ((16 * j + (lane & 15)) / RPB) & (CPR - 1);
          const float4 u0 = *(const float4 *)(xt + 16 * j * RB + ((kc ^ sw) << 4));
          const float4 u1 = *(const float4 *)(xt + 16 * j * RB + (((kc + 1) ^ sw) << 4));
          v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
          v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
          uint4 x0, x1, x2;
          split3(v, x0, x1, x2);
          acc[j] = mfma16(r0, x0, acc[j]);
          acc[j] = mfma16(r0, x1, acc[j]);
          acc[j] = mfma16(r1, x0, acc[j]);
          acc[j] = mfma16(r0, x2, acc[j]);
          acc[j] = mfma16(r2, x0, acc[j]);
          acc[j] = mfma16(r1, x1, acc[j]);
        }
      }
    }
    // ---- quantise from the accumulators: code = #{thresholds < y} by a
    // descent of the padded tree.  A NaN y codes as 0: the MFMA returns the
    // positive quiet NaN for any NaN input, and (threshold - NaN) keeps its
    // clear sign bit, so every level goes left (checked for NaN inputs of
    // either sign).  The 16
    // descents of a wave (4 registers x 4 token blocks) advance level by
    // level together, so their LDS reads overlap; the plan orders a wave's
    // registers by decreasing depth, so the registers still descending at a
    // level are a prefix.  (The descriptors are decoded per tile: hoisting the
    // decoded fields out of the loop would not fit the register budget.)
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(tw[r]), "+v"(cc[r]));
    uint32_t *rec = rec0 + rb * 64 * rs;
    float *rtile = smem + a.lds_res_off + par * 64 * C2_RS;
    uint32_t k[4][4];
    const float *tr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tr[r] = trees + (tw[r] & 0xFFFFu) - 1;  // node k at tr[k]
    }
    // level 1: the root is the same node for the lane's four token blocks
    auto first = [&](auto nr) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < decltype(nr)::value) {
          const float t = tr[r][1];
#pragma unroll
          for (int j = 0; j < 4; ++j) k[r][j] = __builtin_amdgcn_alignbit(1u, __float_as_uint(t - acc[j][r]), 31);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) k[r][j] = 1u;  // depth 0: code 0
        }
      }
    };
    auto level = [&](auto nr) __attribute__((always_inline)) {
      float t[decltype(nr)::value][4];
#pragma unroll
      for (int r = 0; r < decltype(nr)::value; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) t[r][j] = tr[r][k[r][j]];
#pragma unroll
      for (int r = 0; r < decltype(nr)::value; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          k[r][j] = __builtin_amdgcn_alignbit(k[r][j], __float_as_uint(t[r][j] - acc[j][r]), 31);
    };
    {
      if (dep[3] > 0) first(std::integral_constant<int, 4>{});
      else if (dep[2] > 0) first(std::integral_constant<int, 3>{});
      else if (dep[1] > 0) first(std::integral_constant<int, 2>{});
      else if (dep[0] > 0) first(std::integral_constant<int, 1>{});
      else first(std::integral_constant<int, 0>{});
      int l = 1;
      for (; l < dep[3]; ++l) level(std::integral_constant<int, 4>{});
      for (; l < dep[2]; ++l) level(std::integral_constant<int, 3>{});
      for (; l < dep[1]; ++l) level(std::integral_constant<int, 2>{});
      for (; l < dep[0]; ++l) level(std::integral_constant<int, 1>{});
    }
    // codes into the record tile (k - 2^depth, shifted into place)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t kw = (tw[r] >> 16) & 0xFFu, sh = (tw[r] >> 24) & 31u;
      const uint32_t top = 1u << dep[r];
      const uint32_t ntop = 0u - (top << sh);  // (k << sh) + ntop = (k - 2^depth) << sh
      uint32_t *rw = rec + (lane & 15) * rs + kw;
#pragma unroll
      for (int j = 0; j < 4; ++j) atomicOr(rw + 16 * j * rs, (k[r][j] << sh) + ntop);
      if (tw[r] & (1u << 29)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) atomicOr(rw + 16 * j * rs + 1, (k[r][j] - top) >> (32u - sh));
      }
    }
    if (m > 0) {  // signal residuals y - C[code] for the QJL sketch and gamma
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t crd = cc[r] & 0xFFu, cb = cc[r] >> 8;
        if (cb != 0xFFFFFFu) {
#pragma unroll
          for (int j = 0; j < 4; ++j)  // (a NaN y leaves a NaN residual: no QJL bit, NaN gamma)
            rtile[((lane & 15) + 16 * j) * C2_RS + crd] = acc[j][r] - csig[cb + k[r][j] - (1u << dep[r])];
        }
      }
    }
    // ---- the next tile's x has landed (this wave's loads; the barrier covers
    // every wave's); then the tile after it goes into the buffer just read
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t + 2 < te) dma_x(t + 2, par);
    // ---- record words, lane = token: this tile's words without QJL bits,
    // and the previous tile's words with QJL bits or gamma
    {
      const bool has_prev = t != tb;
      const int prb = rb == 0 ? 2 : rb - 1;
      const uint32_t lrow = (uint32_t)lane * (uint32_t)rs;
      uint32_t *ocur = obase + (int64_t)t * W * 64;
      uint32_t *oprv = obase + (int64_t)(t - 1) * W * 64;
      const bool valid = (int64_t)t * 64 + lane < a.n_tokens;
      const bool pvalid = (int64_t)(t - 1) * 64 + lane < a.n_tokens;
      const bool in = (int64_t)t * 64 + lane < send, pin = (int64_t)(t - 1) * 64 + lane < send;
      // words w + NW i, two at a time: this tile's (no QJL bits) or the
      // previous tile's; a slot past this wave's words reads and clears the
      // pad column rs - 1
      for (int i0 = 0; i0 < nmine; i0 += 2) {
        uint32_t v[2], off[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = i0 + u;
          const int kk = i < nmine ? w + NW * i : rs - 1;
          const int bi = (qmask >> i & 1u) ? prb : rb;
          off[u] = (uint32_t)(bi * 64 * rs + kk);
          v[u] = rec0[lrow + off[u]];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) rec0[lrow + off[u]] = 0u;  // for tile + 3 (two more barriers first)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = i0 + u;
          const bool q = qmask >> i & 1u;
          if (i < nmine && (!q || has_prev) && (q ? pin : in)) {
            uint32_t *o = q ? oprv : ocur;
            o[(uint32_t)(w + NW * i) * 64u + lofs] = (q ? pvalid : valid) ? v[u] : 0u;
          }
        }
      }
    }
    // ---- QJL rows [jb, je) of this tile: z_j = [(S r)_j >= 0]; the last
    // wave adds gamma = |r| as IEEE half (RNE).  The words are stored after
    // the next barrier.
    if (m > 0) {
      const float4 *rrow = (const float4 *)(rtile + lane * C2_RS);
      float rv[C2_SP];
#pragma unroll
      for (int i4 = 0; i4 < C2_SP / 4; ++i4) {
        const float4 u = rrow[i4];
        rv[4 * i4] = u.x; rv[4 * i4 + 1] = u.y; rv[4 * i4 + 2] = u.z; rv[4 * i4 + 3] = u.w;
      }
      uint32_t zb = 0u;
      for (int j = jb; j < je; ++j) {
        const float4 *srow = (const float4 *)(Sl + j * C2_SP);
        float dot = 0.0f;
#pragma unroll
        for (int i4 = 0; i4 < C2_SP / 4; ++i4) {
          const float4 s = srow[i4];
          dot = fmaf(s.x, rv[4 * i4 + 0], dot);
          dot = fmaf(s.y, rv[4 * i4 + 1], dot);
          dot = fmaf(s.z, rv[4 * i4 + 2], dot);
          dot = fmaf(s.w, rv[4 * i4 + 3], dot);
        }
        zb |= (dot >= 0.0f ? 1u : 0u) << (j - jb);
      }
      uint32_t *rrec = rec + lane * rs;
      if (je > jb) {
        const int p = code_bits + jb, pw = p >> 5, ps = p & 31;
        atomicOr(rrec + pw, zb << ps);
        if (ps + (je - jb) > 32) atomicOr(rrec + pw + 1, zb >> (32 - ps));
      }
      if (w == NW - 1) {
        float g2 = 0.0f;
#pragma unroll
        for (int i = 0; i < C2_SP; ++i) g2 = fmaf(rv[i], rv[i], g2);
        // v_sqrt_f32 (within 1 ulp of fp32) before the fp16 rounding
        atomicOr(rrec + W - 1, half_bits_rne(__builtin_amdgcn_sqrtf(g2)) << 16);
      }
    }
  }
  // ---- the last tile's words with QJL bits or gamma
  if (m > 0) {
    __syncthreads();
    uint32_t *rlast = rec0 + ((te - 1 - tb) % 3) * 64 * rs + lane * rs;
    uint32_t *dst = obase + (int64_t)(te - 1) * W * 64 + lofs;
    const bool valid = (int64_t)(te - 1) * 64 + lane < a.n_tokens;
    const bool in = (int64_t)(te - 1) * 64 + lane < send;
#pragma unroll
    for (int i = 0; i < C2_WMAX; ++i)
      if ((qmask >> i & 1u) && i < nmine && in) dst[(int64_t)(w + NW * i) * 64] = valid ? rlast[w + NW * i] : 0u;
  }
}

// ------------------------------------------------------------------ scores
//
// s_t = sum_i q~_i C_i[code_ti] + sqrt(pi/2)/m * gamma_t * sum_j w_j (2 z_tj - 1),
// q~ = R q, w = S q~[:d_eff] (SpectralQuant README, "Overview": the query is
// rotated once and scored against the codes; QJL estimator as in the QJL
// paper, section 3).
//
// A workgroup serves one (batch, KV head) and a run of 64-token tiles with 8
// consumer waves and SC_LOADERS loader waves.  The score schedule (SCHED_WORDS) cuts
// the head's coordinates into quads of 4 MFMA k-slots; the consumer waves
// are split into KS wave groups over the quads ("split-K") times TS tile
// streams (KS * TS = 8), so each wave keeps its own quads' MFMA A operands
// (q~ of 4 query heads as bf16 hi and lo parts) and their bit positions,
// masks and table addresses in registers for the whole kernel.  Per tile
// and half the lane (= token) reads its two record words, extracts the
// half's bit field and fetches the joint-table entry; per quad three
// v_mfma_f32_4x4x4_16b_bf16 (qhi*chi + qhi*clo + qlo*chi) accumulate 4 query
// heads x 64 tokens with every product exact and each term good to ~2^-16,
// software-pipelined over three quads.
// Record tiles stream from HBM into a ring of R LDS slots (TS tiles each)
// with direct-to-LDS loads issued by the loader waves, DS super-steps of NS
// slots ahead; one workgroup barrier per super-step.  The partial sums of a
// wave group meet in LDS and are added in a fixed order (deterministic) one
// super-step later, the last wave of each group adding the QJL term.

constexpr int SC_WAVES = 8;    // consumer waves per workgroup
constexpr int SC_LOADERS = 3;  // waves issuing the record loads
constexpr int SC_BLOCK = 64 * (SC_WAVES + SC_LOADERS);
// quads held in registers per consumer wave (4 or 8 query heads per MFMA row set)
__host__ __device__ constexpr int sc_qmax(int gr) { return gr == 1 ? 9 : 5; }

struct ScoresArgs {
  const DevHead *heads;
  const uint8_t *blob;
  const void *q;
  const uint32_t *kpacked;
  float *scores;
  int64_t ps_b, ps_h;
  int64_t n_tokens;
  int first_head, cbs;
  int n_q_heads, n_kv_heads, G;
  int q_f32;
  int n_tiles, tiles_per_wg;
  int ks, ts;             // wave groups over quads, tile streams (ks * ts = SC_WAVES)
  int pass;               // quads [pass * ks * sc_qmax(GR), ...) of every head
  int dma16;              // records 16-byte aligned: 1 KB direct-to-LDS loads
  int lds_lut, lds_qt, lds_wq, lds_slot, lds_pbuf;  // byte offsets
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a),
                                                __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_pair(uint16_t x) { return (uint32_t)x | ((uint32_t)x << 16); }


template <int GR, int SLOTB, int R, bool LG>
__global__ __launch_bounds__(SC_BLOCK) void scores_kernel(ScoresArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  constexpr int GP = 4 * GR;
  constexpr int SC_QMAX = sc_qmax(GR);
  constexpr int NS = SLOTB == 8192 ? 2 : 1;  // ring slots (steps of TS tiles) per barrier ("super-step")
  // In use during super-step ss: ss (consumers), ss + 1 .. ss + DS (loads in
  // flight or being issued).
  constexpr int DS = R / NS - 1;              // super-steps loaded ahead
  static_assert(R % NS == 0 && DS >= 1, "ring of whole super-steps");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int ch = a.first_head + b * a.cbs + hkv;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d, d_eff = hd->d_eff, m = hd->m, W = hd->W, code_bits = hd->code_bits;
  const int KS = a.ks, TS = a.ts, G = a.G;
  const int qp0 = a.pass * KS * SC_QMAX;
  const int nq_pass = min(hd->n_quads - qp0, KS * SC_QMAX);
  if (nq_pass <= 0) return;  // whole workgroup: this head has no quads in this pass
  const int tb = blockIdx.x * a.tiles_per_wg;
  const int te = min(a.n_tiles, tb + a.tiles_per_wg);
  const int nsteps = (te - tb + TS - 1) / TS;  // ring slots to fill, TS tiles each
  const int nsup = (nsteps + NS - 1) / NS;
  const uint32_t *slot = a.kpacked + (int64_t)b * a.ps_b + (int64_t)hkv * a.ps_h;
  const uint32_t lds0 = (uint32_t)(uintptr_t)sm;
  const bool loader = wave >= SC_WAVES;  // (a wave's own direct-to-LDS loads hold up its LDS reads)

  // Direct-to-LDS loads of super-step sp (slots sp*NS ..) are spread over the
  // loader waves: its load instructions (1 KB pieces, then 256-byte rows) are
  // numbered in order and loader l issues those with number % SC_LOADERS == l.
  // Returns how many this wave issued (wave-uniform).
  auto dma_super = [&](int sp, bool go) -> int {
    int mine = 0, base = 0;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int j = sp * NS + t;
      if (j >= nsteps) break;
      const int t0 = tb + j * TS;
      const int rows = min(TS, te - t0) * W;
      const uint32_t *src = slot + (int64_t)t0 * W * 64;
      const uint32_t dst = lds0 + a.lds_slot + (j % R) * SLOTB;
      const int n4 = a.dma16 ? rows >> 2 : 0, n1 = rows - 4 * n4;
      // ops [base, base + n4 + n1): this wave's are base + i with (base + i) % SC_LOADERS == l
      int i = (wave - SC_WAVES - base) % SC_LOADERS;
      if (i < 0) i += SC_LOADERS;
      for (; i < n4; i += SC_LOADERS) {
        if (go) lds_dma16(src + i * 256, lane * 16, dst + i * 1024);
        ++mine;
      }
      for (; i < n4 + n1; i += SC_LOADERS) {
        const int r = 4 * n4 + (i - n4);
        if (go) lds_dma4(src + r * 64, lane * 4, dst + r * 256);
        ++mine;
      }
      base += n4 + n1;
    }
    return mine;
  };

  if (loader)
    for (int sp = 0; sp < min(DS, nsup); ++sp) dma_super(sp, true);

  // ---- prologue (consumer waves): tables, q~ = R q, w = scale * S q~
  const int ct = threadIdx.x;  // < 64 * SC_WAVES for consumers
  const bool consumer = wave < SC_WAVES;
  float *qraw = (float *)(sm + a.lds_pbuf);  // scratch until the first step
  float *qt = (float *)(sm + a.lds_qt);      // [G][d]
  float *wq = (float *)(sm + a.lds_wq);      // [m][GP]
  if (consumer) {
    if constexpr (!LG) {  // joint tables: 1 KB direct-to-LDS loads (table size rounded up in the blob)
      const uint8_t *src = a.blob + hd->off_plut;
      const int nkb = (hd->n_plut * 8 + 1023) >> 10;
      for (int k = wave; k < nkb; k += SC_WAVES) lds_dma16(src + k * 1024, lane * 16, lds0 + a.lds_lut + k * 1024);
    }
    const int64_t qbase = ((int64_t)b * a.n_q_heads + (int64_t)hkv * G) * d;
    for (int k = ct; k < G * d; k += 64 * SC_WAVES)
      qraw[k] = a.q_f32 ? ((const float *)a.q)[qbase + k] : bf16_to_f32(((const uint16_t *)a.q)[qbase + k]);
  }
  __syncthreads();  // (its fence waits for every load issued so far)
  if (consumer) {
    const float *RT = (const float *)(a.blob + hd->off_RT);
    for (int k = ct; k < G * d; k += 64 * SC_WAVES) {
      const int g = k / d, i = k - g * d;
      const float *qg = qraw + g * d;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < d; j0 += 16) {  // d is a multiple of 16: 16 loads in flight
        float r[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) r[u] = RT[(size_t)(j0 + u) * d + i];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u & 3] = fmaf(r[u], qg[j0 + u], acc[u & 3]);
      }
      qt[k] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
  }
  __syncthreads();
  if (consumer && m > 0) {
    const SQ_CONST float *S = cptr<float>(a.blob + hd->off_S);
    for (int k = ct; k < m * GP; k += 64 * SC_WAVES) {
      const int j = k / GP, g = k - j * GP;
      float acc = 0.0f;
      if (g < G)
        for (int i = 0; i < d_eff; ++i) acc = fmaf(S[j * d_eff + i], qt[g * d + i], acc);
      wq[k] = hd->qjl_scale * acc;
    }
  }
  __syncthreads();  // wq complete
  float *pbuf = (float *)(sm + a.lds_pbuf);

  if (loader) {
    for (int ss = 0; ss < nsup; ++ss) {
      int pend = 0;  // this wave's loads issued after those of super-step ss
      for (int sp = ss + 1; sp <= min(ss + DS - 1, nsup - 1); ++sp) pend += dma_super(sp, false);
      wait_vmcnt(pend);
      step_barrier();
      // loads for super-step ss + DS go to the slots of ss - 1, which the
      // consumers left before this barrier
      if (ss + DS < nsup) dma_super(ss + DS, true);
    }
    step_barrier();
    return;
  }

  // ---- consumer wave (tau, kk): tile stream tau, quads [q0, q0 + nq)
  const int tau = wave / KS, kk = wave - tau * KS;
  const int nqb = nq_pass / KS, nqr = nq_pass - nqb * KS;
  const int nq = nqb + (kk < nqr ? 1 : 0);
  const int q0 = qp0 + kk * nqb + min(kk, nqr);
  // QJL term: wave kk adds it for the query heads (rows) r = kk, kk + KS, ..
  // to its own partial sum, so that every row gets it exactly once
  const bool qjl = m > 0 && a.pass == 0 && kk < min(G, GP);
  const bool qjl_fast = qjl && KS >= GP && m <= 8;  // one row per wave, weights in scalars
  uint32_t qw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    qw[j] = qjl_fast && j < m ? __float_as_uint(wq[j * GP + kk]) : 0u;  // (vector registers)
  const SQ_CONST uint32_t *sch = cptr<uint32_t>(a.blob + hd->off_sched);
  // Every wave runs SC_QMAX quads; those past its share are empty (mask 0,
  // A operands 0) so that the quads form one straight-line block.  Table
  // addresses are wave-uniform scalars; shifts and masks, also uniform, sit
  // in vector registers (the instructions using them take one scalar each),
  // word addresses per lane.  The two halves of a quad are adjacent fields
  // spanning at most 16 bits, so one pair of record words (a 64-bit window
  // starting at the word that holds the first field's bit - 3) serves both.
  uint32_t hsh[2 * SC_QMAX], hmk[2 * SC_QMAX], hlut[2 * SC_QMAX], wad[SC_QMAX];
  uint2 aqa[SC_QMAX][GR], aqb[SC_QMAX][GR], aql[SC_QMAX][GR];
  const uint32_t tile_lds = a.lds_slot + tau * W * 256 + lane * 4;  // this stream's tile in slot 0
#pragma unroll
  for (int qi = 0; qi < SC_QMAX; ++qi) {
    const bool real = qi < nq;
    const SQ_CONST uint32_t *e = sch + (size_t)(q0 + (real ? qi : 0)) * SCHED_WORDS;
    // the window starts at the word holding bit pos0 - 3 of the first field
    // (one row earlier when that field starts in the first 3 bits of a
    // word), so that (window >> (pos - 3 - 32 j)) & (mask << 3) gives
    // code * 8, the entry's byte offset; the second field starts at most
    // 8 + 31 bits in and ends below bit 64 (an empty half has mask 0)
    const int j = ((int)(e[0] & 0xFFFFu) - 3) >> 5;  // may be -1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t pw = e[hh];
      const int pos = (int)(pw & 0xFFFFu) - 3, wd = (int)(pw >> 16);
      hsh[2 * qi + hh] = to_vgpr((uint32_t)(pos - 32 * j) & 63u);
      hmk[2 * qi + hh] = to_vgpr(real ? ((1u << wd) - 1u) << 3 : 0u);
      hlut[2 * qi + hh] = (LG ? 0u : (uint32_t)a.lds_lut) + e[2 + hh] * 8u;
    }
    wad[qi] = tile_lds + (uint32_t)j * 256u;
    const uint32_t s01 = e[4], s23 = e[5];
    const uint32_t sl[4] = {s01 & 0xFFFFu, s01 >> 16, s23 & 0xFFFFu, s23 >> 16};
#pragma unroll
    for (int g = 0; g < GR; ++g) {
      const int head = 4 * g + (lane & 3);
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = (real && head < G && sl[k] != 0xFFFFu) ? qt[head * d + (int)sl[k]] : 0.0f;
        hi[k] = f32_to_bf16_rne(v);
        lo[k] = f32_to_bf16_rne(v - bf16_to_f32(hi[k]));
      }
      const uint32_t hab = (uint32_t)hi[0] | ((uint32_t)hi[1] << 16), hcd = (uint32_t)hi[2] | ((uint32_t)hi[3] << 16);
      aqa[qi][g] = make_uint2(hab, hab);
      aqb[qi][g] = make_uint2(hcd, hcd);
      aql[qi][g] = make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
    }
  }
  const uint2 *glut = (const uint2 *)(a.blob + hd->off_plut);
  const int zsh = code_bits & 31;

  // sum the wave group's partials of super-step sp (fixed order) and store
  auto reduce_k = [&](int sp, auto ksc) __attribute__((always_inline)) {
    constexpr int K = decltype(ksc)::value;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int tile = tb + (sp * NS + t) * TS + tau;
      if (tile >= te) continue;
      const float *pr = pbuf + (((sp & 1) * NS + t) * TS + tau) * K * GP * 64 + lane;
      const int64_t tok = (int64_t)tile * 64 + lane;
#pragma unroll
      for (int row0 = 0; row0 < GP; row0 += K) {
        const int row = row0 + kk;
        if (row >= GP) continue;
        float pv[K];
#pragma unroll
        for (int k2 = 0; k2 < K; ++k2) pv[k2] = pr[(k2 * GP + row) * 64];
        float v = pv[0];
#pragma unroll
        for (int k2 = 1; k2 < K; ++k2) v += pv[k2];
        if (row < G && tok < a.n_tokens) {
          float *o = a.scores + ((int64_t)b * a.n_q_heads + (int64_t)hkv * G + row) * a.n_tokens + tok;
          if (a.pass) __hip_atomic_fetch_add(o, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // one add per pass
          else *o = v;
        }
      }
    }
  };
  auto reduce = [&](int sp) __attribute__((always_inline)) {
    switch (KS) {
      case 1: reduce_k(sp, std::integral_constant<int, 1>()); break;
      case 2: reduce_k(sp, std::integral_constant<int, 2>()); break;
      case 4: reduce_k(sp, std::integral_constant<int, 4>()); break;
      default: reduce_k(sp, std::integral_constant<int, 8>()); break;
    }
  };


  for (int ss0 = 0; ss0 < nsup; ss0 += R / NS) {
#pragma unroll
    for (int u = 0; u < R / NS; ++u) {
      const int ss = ss0 + u;
      if (ss >= nsup) break;
      step_barrier();
      if (ss > 0) reduce(ss - 1);
      f32x4 acc[NS][GR];
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int g = 0; g < GR; ++g) acc[t][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      // three-stage pipeline over the quads: record words of quad it, joint
      // table entries of quad it - 1, MFMAs of quad it - 2
      uint32_t wlo[SC_QMAX][NS], whi[SC_QMAX][NS];
      uint2 ent[SC_QMAX][NS][2];
#pragma unroll
      for (int it = 0; it < SC_QMAX + 2; ++it) {
        if (it < SC_QMAX) {
#pragma unroll
          for (int t = 0; t < NS; ++t) {
            const uint32_t ad = wad[it] + ((u * NS + t) % R) * SLOTB;
            wlo[it][t] = *(const uint32_t *)(sm + ad);
            whi[it][t] = *(const uint32_t *)(sm + ad + 256);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (it >= 1 && it - 1 < SC_QMAX) {
          const int qi = it - 1;
#pragma unroll
          for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int h = 2 * qi + hh;
              // table base | code * 8 (tables are aligned to their size); the
              // first field's shift is below 32, the second's below 64
              const uint32_t win = hh == 0 ? __builtin_amdgcn_alignbit(whi[qi][t], wlo[qi][t], hsh[h])
                                           : (uint32_t)((((uint64_t)whi[qi][t] << 32) | wlo[qi][t]) >> hsh[h]);
              const uint32_t ea = (win & hmk[h]) | hlut[h];
              if constexpr (LG) {
                ent[qi][t][hh] = *(const uint2 *)((const uint8_t *)glut + ea);
              } else {  // the LDS area starts at address 0 (the launcher checks the kernel has no static LDS)
                typedef const __attribute__((address_space(3))) uint64_t lds_u64;
                const uint64_t v = *(lds_u64 *)(uintptr_t)ea;
                ent[qi][t][hh] = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
              }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (it >= 2) {
          const int qi = it - 2;
#pragma unroll
          for (int t = 0; t < NS; ++t) {
            // E = (lo_ab, hi_ab, hi_cd, lo_cd): three consecutive register pairs
            const uint4 E = make_uint4(ent[qi][t][0].x, ent[qi][t][0].y, ent[qi][t][1].x, ent[qi][t][1].y);
#pragma unroll
            for (int g = 0; g < GR; ++g) {
              acc[t][g] = mfma4(aqa[qi][g], make_uint2(E.x, E.y), acc[t][g]);
              acc[t][g] = mfma4(aqb[qi][g], make_uint2(E.z, E.w), acc[t][g]);
              acc[t][g] = mfma4(aql[qi][g], make_uint2(E.y, E.z), acc[t][g]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the stages in this order
      }
      if (qjl) {  // + gamma * sum_j w_j (2 z_j - 1), w already scaled by sqrt(pi/2)/m
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const uint32_t tl = tile_lds + (u * NS + t) * SLOTB;
          const float gm = half_bits_to_f32(*(const uint32_t *)(sm + tl + (W - 1) * 256u) >> 16);
          if (qjl_fast) {
            const uint32_t ad = tl + (code_bits >> 5) * 256u;
            const uint32_t nz = ~__builtin_amdgcn_alignbit(*(const uint32_t *)(sm + ad + 256),
                                                          *(const uint32_t *)(sm + ad), zsh);
            float qa = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)  // +w_j where z_j = 1, -w_j where z_j = 0 (w_j = 0 past m)
              qa += __uint_as_float(qw[j] ^ ((nz << (31 - j)) & 0x80000000u));
#pragma unroll
            for (int g = 0; g < GR; ++g)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                if (4 * g + rr == kk) acc[t][g][rr] = fmaf(gm, qa, acc[t][g][rr]);
          } else {
            for (int row = kk; row < min(G, GP); row += KS) {
              float qa = 0.0f;
              for (int j0 = 0; j0 < m; j0 += 32) {
                const uint32_t ad = tl + ((code_bits + j0) >> 5) * 256u;
                const uint32_t z = __builtin_amdgcn_alignbit(*(const uint32_t *)(sm + ad + 256),
                                                             *(const uint32_t *)(sm + ad), zsh);
                const int jn = min(32, m - j0);
                for (int j = 0; j < jn; ++j) {
                  const float wv = wq[(j0 + j) * GP + row];
                  qa += ((z >> j) & 1u) ? wv : -wv;
                }
              }
#pragma unroll
              for (int g = 0; g < GR; ++g)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                  if (4 * g + rr == row) acc[t][g][rr] = fmaf(gm, qa, acc[t][g][rr]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        float *pw = pbuf + ((((ss & 1) * NS + t) * TS + tau) * KS + kk) * GP * 64 + lane;
#pragma unroll
        for (int g = 0; g < GR; ++g)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) pw[(4 * g + rr) * 64] = acc[t][g][rr];
      }
    }
  }
  step_barrier();
  if (nsup > 0) reduce(nsup - 1);
}

// ------------------------------------------------------------------ attend
//
// Split-T softmax-weighted value sum in the rotated value space.  Kernel 1:
// one wave per (batch, KV head, chunk of tokens); in pass p of the
// head_dim / 64 passes a lane serves one coordinate (with column tables
// coordinate NP lane + p, so a lane's fields share their record words; else
// 64 p + lane).  Per 64-token tile the record
// words are staged straight from HBM into LDS (word-major, row stride
// ATT_RS, so lanes reading different words of one token hit different
// banks); the query group's scores give an online softmax (running max,
// rescaled sums) whose weights p are kept in LDS as bf16 hi/lo pairs, once
// for all passes.  Each lane decodes its coordinate for 4 tokens at a time into C_v[code] as
// bf16 hi/lo pairs and v_mfma_f32_4x4x4_16b_bf16 forms sum_t p_t C_v[code_t]:
// in block b, lane 4b+n supplies the 4 tokens of its coordinate (B operand),
// lane 4b+m the weights of query head m (A operand), and the accumulator of
// lane 4b+n holds head m in register m.  Three products (hi*hi + hi*lo +
// lo*hi) give each term to ~2^-16 relative.  Kernel 2: one workgroup per
// (batch, query head) combines the chunks in order (no atomics,
// deterministic) and un-rotates once: o = R_v^T o_rot / L.

// Tokens per chunk: 2048 when that still gives about two waves per CU or
// more (fewer partials to combine and table loads), else 1024.  A function of
// (batch, query heads, tokens) only, so the workspace size follows it.
static int64_t attend_chunk_tokens(int batch, int n_q_heads, int64_t n_tokens) {
  return (int64_t)batch * n_q_heads * (n_tokens / 2048) >= 4096 ? 2048 : 1024;
}
static constexpr int ATT_RS = 68;  // staged record row stride (words): 16-byte aligned, bank-spread
static constexpr int ATT_PS = 68;  // weight row stride (words): rows of different heads in different banks
static constexpr float ATT_TAU = 8.0f;  // lazy-rescale margin of the running softmax max

struct AttendArgs {
  const DevHead *heads;
  const uint8_t *blob;
  const float *scores;
  const uint32_t *vpacked;
  float *ws;
  float *out;
  int64_t ps_b, ps_h;
  int64_t n_tokens;
  float scale;
  int first_head, cbs;
  int n_q_heads, n_kv_heads;
  int n_chunks;
  int chunk_tokens;            // tokens per chunk (a multiple of 64)
  int lut_block;               // floats: stride of the 64-coordinate blocks' centroid tables
  int lds_wave_off;            // floats: per-wave areas (the centroid tables start at 0)
  int wave_floats;             // one wave's area: two staging buffers, then the weights
  int buf_floats;              // one staging buffer: [W + 2][ATT_RS] words + [G][64] scores
};

// Maximum over the 64 lanes (returned in every lane), on order-preserving
// integer keys of the floats (sign-magnitude to two's complement): rotations
// within each row of 16 (DPP), then the four row results.  A positive NaN
// wins and a negative NaN loses; either way its token's weight is NaN.
__device__ __forceinline__ float wave_max(float v) {
  int k = __float_as_int(v);
  k ^= (k >> 31) & 0x7FFFFFFF;
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x128, 0xF, 0xF, true));  // (row rotations: every lane valid)
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x124, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x122, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x121, 0xF, 0xF, true));
  int m = max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
              max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
  m ^= (m >> 31) & 0x7FFFFFFF;
  return __int_as_float(m);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// (bf16(x), bf16(x)) packed, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pair_rne(float x) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x, x}, bf16x2_t));
}

// Centroid table placement of the attend kernel: LM_COL = one column per lane
// (entry code * 64 + lane: every lane reads its own bank; widths <= 6),
// LM_PACK = a block's tables back to back with one pad entry each, LM_GLB =
// read from the table blob (tables too large for LDS).
enum { LM_COL = 0, LM_PACK = 1, LM_GLB = 2 };

// NP = 64-coordinate blocks per head (head_dim / 64, at least 1): one wave
// serves every block of its chunk, so the chunk's scores are read and its
// softmax computed once.
// WPB = waves (chunks) per workgroup, sharing the centroid tables; NBUF =
// staging buffers per wave.  Column tables: 16 single-buffered waves (four
// per SIMD) when the LDS allows, else 8 double-buffered; otherwise 4.
template <int G, int LM, int NP, int WPB, int NBUF = 2>
__global__ __launch_bounds__(64 * WPB) void attend_partial_kernel(AttendArgs a) {
  extern __shared__ float smem[];
  constexpr int GR = (G + 3) / 4, GP = 4 * GR;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // a workgroup = WPB consecutive chunks of one (batch, KV head)
  const int chunk = blockIdx.x * WPB + wv;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int ch = a.first_head + b * a.cbs + hkv;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d, W = hd->W;
  const SQ_CONST DevCoord *coords = cptr<DevCoord>(a.blob + hd->off_coord);
  uint32_t *lut = (uint32_t *)smem;
  float *stage = smem + a.lds_wave_off + wv * a.wave_floats;  // two buffers: words, then scores
  uint32_t *ph = (uint32_t *)(stage + NBUF * a.buf_floats);   // [GP][ATT_PS] bf16 hi of p, twice
  uint32_t *pl = ph + GP * ATT_PS;                             // [GP][ATT_PS] bf16 lo of p, twice
  const uint32_t *glut = (const uint32_t *)(a.blob + hd->off_lutp);
  // this lane's field in each block p: coordinate NP lane + p with column
  // tables (the lane's NP fields are adjacent in the record), else 64 p + lane
  int cb[NP], cwl[NP], cs[NP];
  uint32_t fmask[NP];
  bool straddle[NP];
  // column tables: the lane's fields are taken from one 64-bit window of
  // staged rows wrow, wrow + 1 that starts 8 bits below the first, so that
  // one shift and one and-or give each entry's byte address (field << 8 |
  // lane << 2 | block base); NP fields of at most 6 bits end below bit 64
  int wrow = 1;
  uint32_t wsh[NP], m8[NP], orv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c0 = p * 64, ci = LM == LM_COL ? NP * lane + p : c0 + lane;
    const int lut0 = c0 < d ? coords[c0].cent_base : 0;
    int width = 0, bo = 0, cbv = 0;
    if (ci < d) {
      width = coords[ci].width;
      bo = coords[ci].bit_off;
      cbv = coords[ci].cent_base - lut0;
    }
    const int n = width ? (1 << width) : 0;
    const int base = p * a.lut_block;
    if constexpr (LM == LM_COL) {
      // column lane: entry f at f * 64 + lane; a zero-width lane reads 0 at f = 0
      for (int k = wv; k < max(n, 1); k += WPB) lut[base + k * 64 + lane] = n ? glut[lut0 + cbv + k] : 0u;
      cb[p] = base + lane;
    } else if constexpr (LM == LM_PACK) {
      // coordinate c0 + j's table at offset cbv + j: lanes gathering the same
      // code from tables of equal size fall in different banks; the slot after
      // each table is 0, which a zero-width coordinate (field 0) reads
      if (ci < d) {  // lanes past the last coordinate (head_dim 32) write nothing
        for (int k = wv; k < n; k += WPB) lut[base + cbv + lane + k] = glut[lut0 + cbv + k];
        if (wv == 0) lut[base + cbv + lane + n] = 0u;
      }
      cb[p] = base + cbv + lane;
    } else {
      cb[p] = lut0 + cbv;
    }
    fmask[p] = width ? ((1u << width) - 1u) : 0u;
    cwl[p] = width ? (bo >> 5) : 0;
    cs[p] = bo & 31;
    straddle[p] = cs[p] + width > 32;
    // staged row 0 is zero (the word before word 0), row w + 1 is word w
    if (p == 0) wrow = ci < d ? ((bo - 8) >> 5) + 1 : 1;
    wsh[p] = ci < d ? (uint32_t)(bo - 8 - 32 * (wrow - 1)) & 63u : 0u;
    m8[p] = fmask[p] << 8;
    orv[p] = ((uint32_t)lane << 2) | ((uint32_t)(p * a.lut_block) << 2);
  }
  const uint32_t *lutv;
  if constexpr (LM == LM_GLB) lutv = glut;
  else lutv = lut;

  const int lsh = LM == LM_COL ? 6 : 0;  // gather index: (field << lsh) + cb
  __syncthreads();
  if (chunk >= a.n_chunks) return;  // no barrier follows

  const int64_t tb = (int64_t)chunk * a.chunk_tokens;
  const int64_t te = min(a.n_tokens, tb + a.chunk_tokens);
  const float *srow = a.scores + ((int64_t)b * a.n_q_heads + (int64_t)hkv * G) * a.n_tokens;
  const uint32_t *slot = a.vpacked + (int64_t)b * a.ps_b + (int64_t)hkv * a.ps_h;
  float mrun[G], lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    lsum[g] = 0.0f;
  }
  // per block, four independent accumulator sets (the products of a step
  // alternate among them), summed at the end
  f32x4 acc[NP][4][GR];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int r = 0; r < GR; ++r) acc[p][h][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging: the W words of the tile's records (plus one spare row, a copy
  // of the last word: the word after a field never goes past it) and its G
  // score rows go straight from HBM to LDS.  Double-buffered (NBUF 2), tile
  // i + 1 is requested before tile i is computed, so the one wait per tile
  // covers loads issued a whole tile earlier; single-buffered (NBUF 1), a
  // tile is requested when the previous one is done and the other waves of
  // the SIMD cover the wait.
  auto stage_tile = [&](int64_t t0, int buf) {
    uint32_t *rw = (uint32_t *)(stage + buf * a.buf_floats) + ATT_RS;  // row 1 = word 0
    const uint32_t *src = slot + (t0 >> 6) * W * 64 + lane;
    for (int w = 0; w <= W; ++w)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + min(w, W - 1) * 64),
                                       (__attribute__((address_space(3))) void *)(rw + w * ATT_RS), 4, 0, 0);
    float *sr = stage + buf * a.buf_floats + (W + 2) * ATT_RS;
    // pad tokens of the last tile: any in-range address (their weight is 0)
    const int64_t ts = min(t0 + lane, a.n_tokens - 1);
#pragma unroll
    for (int g = 0; g < G; ++g)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(srow + (int64_t)g * a.n_tokens + ts),
                                       (__attribute__((address_space(3))) void *)(sr + g * 64), 4, 0, 0);
  };
  // row 0 of both staging buffers: zeros (the word before word 0)
  ((uint32_t *)stage)[lane] = 0u;
  if constexpr (NBUF == 2) ((uint32_t *)(stage + a.buf_floats))[lane] = 0u;
  if constexpr (NBUF == 2) stage_tile(tb, 0);
  int buf = 0;
  for (int64_t t0 = tb; t0 < te; t0 += 64, buf ^= NBUF - 1) {
    if constexpr (NBUF == 1) stage_tile(t0, 0);  // (the last sync of the previous tile ended its reads)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this tile's staging has landed
    wave_lds_sync();
    if constexpr (NBUF == 2)
      if (t0 + 64 < te) stage_tile(t0 + 64, buf ^ 1);
    const uint32_t *rec = (const uint32_t *)(stage + buf * a.buf_floats);
    const float *sr = stage + buf * a.buf_floats + (W + 2) * ATT_RS;
    // ---- online softmax over the tile (lane = token)
    const int64_t t = t0 + lane;
    float sv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sv[g] = t < te ? a.scale * sr[g * 64 + lane] : -INFINITY;
    // The reference max moves only when a tile exceeds it by more than
    // ATT_TAU: weights stay below e^ATT_TAU and the sums are rescaled rarely.
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mx = wave_max(sv[g]);
      if (mx > mrun[g] + ATT_TAU) {  // uniform; always taken on the first tile (mrun = -inf)
        const float corr = __expf(mrun[g] - mx);
        mrun[g] = mx;
        lsum[g] *= corr;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int h = 0; h < 4; ++h) acc[p][h][g >> 2][g & 3] *= corr;
      }
      const float pv = __expf(sv[g] - mrun[g]);  // 0 for tokens past the end
      lsum[g] += pv;
      const uint32_t hp = bf16_pair_rne(pv);
      ph[g * ATT_PS + lane] = hp;
      pl[g * ATT_PS + lane] = bf16_pair_rne(pv - __uint_as_float(hp << 16));
    }
#pragma unroll
    for (int g = G; g < GP; ++g) {
      ph[g * ATT_PS + lane] = 0u;
      pl[g * ATT_PS + lane] = 0u;
    }
    wave_lds_sync();
    // ---- 8 tokens per step: the weights once, then per block decode (all
    // gathers in flight together) and the weighted sums on the MFMA.  A
    // product takes 2 tokens: the k slots of coordinate n are (hi, lo) of
    // C[code] for each token, the weights of head m are (p, p) per token, so
    // it adds p_t0 (hi0 + lo0) + p_t1 (hi1 + lo1); once with bf16(p) and once
    // with the remainder of p.
    const int m = lane & 3;
#pragma unroll 2
    for (int k = 0; k < 64; k += 8) {
      uint2 ah[GR][4], al[GR][4];
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const uint32_t *hrow = ph + (4 * r + m) * ATT_PS + k, *lrow = pl + (4 * r + m) * ATT_PS + k;
        const uint4 ah0 = *(const uint4 *)hrow, ah1 = *(const uint4 *)(hrow + 4);
        const uint4 al0 = *(const uint4 *)lrow, al1 = *(const uint4 *)(lrow + 4);
        ah[r][0] = make_uint2(ah0.x, ah0.y); ah[r][1] = make_uint2(ah0.z, ah0.w);
        ah[r][2] = make_uint2(ah1.x, ah1.y); ah[r][3] = make_uint2(ah1.z, ah1.w);
        al[r][0] = make_uint2(al0.x, al0.y); al[r][1] = make_uint2(al0.z, al0.w);
        al[r][2] = make_uint2(al1.x, al1.y); al[r][3] = make_uint2(al1.z, al1.w);
      }
      uint4 a0, a1, b0, b1;  // column tables: this lane's window rows for the 8 tokens
      if constexpr (LM == LM_COL) {
        const uint32_t *ra = rec + wrow * ATT_RS, *rb = ra + ATT_RS;
        a0 = *(const uint4 *)(ra + k); a1 = *(const uint4 *)(ra + k + 4);
        b0 = *(const uint4 *)(rb + k); b1 = *(const uint4 *)(rb + k + 4);
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        uint32_t pr[8];
        if constexpr (LM == LM_COL) {
          const uint32_t s = wsh[p], mk = m8[p], ov = orv[p];
          // the first field's shift is below 32, a later one's below 64
          auto win = [&](uint32_t hi, uint32_t lo) __attribute__((always_inline)) {
            return p == 0 ? __builtin_amdgcn_alignbit(hi, lo, s) : (uint32_t)((((uint64_t)hi << 32) | lo) >> s);
          };
          uint32_t ix[8];  // byte offsets of the entries from the start of the tables
          ix[0] = (win(b0.x, a0.x) & mk) | ov;
          ix[1] = (win(b0.y, a0.y) & mk) | ov;
          ix[2] = (win(b0.z, a0.z) & mk) | ov;
          ix[3] = (win(b0.w, a0.w) & mk) | ov;
          ix[4] = (win(b1.x, a1.x) & mk) | ov;
          ix[5] = (win(b1.y, a1.y) & mk) | ov;
          ix[6] = (win(b1.z, a1.z) & mk) | ov;
          ix[7] = (win(b1.w, a1.w) & mk) | ov;
          // the tables open the kernel's LDS (the launcher checks that the
          // kernel has no static LDS), so the offsets are LDS addresses
          typedef const __attribute__((address_space(3))) uint32_t lds_u32;
#pragma unroll
          for (int i = 0; i < 8; ++i) pr[i] = *(lds_u32 *)(uintptr_t)ix[i];
        } else {
          const uint32_t *rlo = rec + (cwl[p] + 1) * ATT_RS, *rhi = rlo + ATT_RS;
          const uint4 lo0 = *(const uint4 *)(rlo + k), lo1 = *(const uint4 *)(rlo + k + 4);
          uint4 hi0 = make_uint4(0, 0, 0, 0), hi1 = hi0;
          if (straddle[p]) {  // only lanes whose field runs into the next word read it
            hi0 = *(const uint4 *)(rhi + k);
            hi1 = *(const uint4 *)(rhi + k + 4);
          }
          const int c = cb[p], s = cs[p];
          const uint32_t fm = fmask[p];
          pr[0] = lutv[c + ((__builtin_amdgcn_alignbit(hi0.x, lo0.x, s) & fm) << lsh)];
          pr[1] = lutv[c + ((__builtin_amdgcn_alignbit(hi0.y, lo0.y, s) & fm) << lsh)];
          pr[2] = lutv[c + ((__builtin_amdgcn_alignbit(hi0.z, lo0.z, s) & fm) << lsh)];
          pr[3] = lutv[c + ((__builtin_amdgcn_alignbit(hi0.w, lo0.w, s) & fm) << lsh)];
          pr[4] = lutv[c + ((__builtin_amdgcn_alignbit(hi1.x, lo1.x, s) & fm) << lsh)];
          pr[5] = lutv[c + ((__builtin_amdgcn_alignbit(hi1.y, lo1.y, s) & fm) << lsh)];
          pr[6] = lutv[c + ((__builtin_amdgcn_alignbit(hi1.z, lo1.z, s) & fm) << lsh)];
          pr[7] = lutv[c + ((__builtin_amdgcn_alignbit(hi1.w, lo1.w, s) & fm) << lsh)];
        }
#pragma unroll
        for (int r = 0; r < GR; ++r)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint2 bv = make_uint2(pr[2 * h], pr[2 * h + 1]);
            acc[p][h][r] = mfma4(ah[r][h], bv, acc[p][h][r]);
            acc[p][h][r] = mfma4(al[r][h], bv, acc[p][h][r]);
          }
      }
    }
    wave_lds_sync();  // every read of this tile's words and weights is done
  }
  // ---- partials: o_rot for the head's coordinates, the running max and the
  // weight sum
  float *dst = a.ws + (((int64_t)b * a.n_q_heads + (int64_t)hkv * G) * a.n_chunks + chunk) * (d + 2);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int ci = LM == LM_COL ? NP * lane + p : p * 64 + lane;
    if (ci < d) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        dst[(int64_t)g * a.n_chunks * (d + 2) + 2 + ci] =
            (acc[p][0][g >> 2][g & 3] + acc[p][1][g >> 2][g & 3]) + (acc[p][2][g >> 2][g & 3] + acc[p][3][g >> 2][g & 3]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = lsum[g];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) {
      dst[(int64_t)g * a.n_chunks * (d + 2) + 0] = mrun[g];
      dst[(int64_t)g * a.n_chunks * (d + 2) + 1] = v;
    }
  }
}

__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs a) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int bq = blockIdx.x;
  const int b = bq / a.n_q_heads, hq = bq % a.n_q_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int ch = a.first_head + b * a.cbs + hq / G;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d;
  float *out = a.out + (int64_t)bq * d;
  if (a.n_tokens == 0) {
    for (int j = tid; j < d; j += blockDim.x) out[j] = 0.0f;
    return;
  }
  const float *part = a.ws + (int64_t)bq * a.n_chunks * (d + 2);
  float *wts = smem;              // [n_chunks]
  float *orot = smem + a.n_chunks;  // [d]
  float M = -INFINITY;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, part[(int64_t)c * (d + 2)]);
  float L = 0.0f;
  for (int c = 0; c < a.n_chunks; ++c) {
    const float e = expf(part[(int64_t)c * (d + 2)] - M);
    L += e * part[(int64_t)c * (d + 2) + 1];
    if (tid == 0) wts[c] = e;
  }
  __syncthreads();
  for (int i = tid; i < d; i += blockDim.x) {
    float s = 0.0f;
    for (int c = 0; c < a.n_chunks; ++c) s = fmaf(wts[c], part[(int64_t)c * (d + 2) + 2 + i], s);
    orot[i] = s / L;
  }
  __syncthreads();
  const float *R = (const float *)(a.blob + hd->off_R);
  for (int j = tid; j < d; j += blockDim.x) {
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(R[(size_t)i * d + j], orot[i], s);
    out[j] = s;
  }
}

// ------------------------------------------------------------------ dequantize
// Diagnostic: one workgroup per (batch, head, 16 tokens).  Thread = (token,
// coordinate) decodes C_i[code] (+ the QJL correction on signal coordinates),
// then x~ = R^T y^ per token.

struct DequantArgs {
  const DevHead *heads;
  const uint8_t *blob;
  const uint32_t *packed;
  float *out;
  int64_t ps_b, ps_h;
  int64_t n_tokens;
  int first_head, cbs, n_heads;
};

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  __shared__ float yb[16 * 257];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int ch = a.first_head + b * a.cbs + h;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d, W = hd->W, m = hd->m, d_eff = hd->d_eff;
  const uint32_t *slot = a.packed + (int64_t)b * a.ps_b + (int64_t)h * a.ps_h;
  const SQ_CONST DevCoord *coords = cptr<DevCoord>(a.blob + hd->off_coord);
  const float *cent = (const float *)(a.blob + hd->off_cent);
  const SQ_CONST float *S = cptr<float>(a.blob + hd->off_S);
  const float *R = (const float *)(a.blob + hd->off_R);
  const int64_t tbase = (int64_t)blockIdx.x * 16;
  auto word = [&](int64_t t, int w) -> uint32_t {
    return w < W ? slot[((t / 64) * W + w) * 64 + t % 64] : 0u;
  };
  for (int k = tid; k < 16 * d; k += blockDim.x) {
    const int tt = k / d, i = k % d;
    const int64_t t = tbase + tt;
    float v = 0.0f;
    if (t < a.n_tokens) {
      const DevCoord cd = load_coord(coords + i);
      if (cd.width) {
        const uint32_t f = __builtin_amdgcn_alignbit(word(t, (cd.bit_off >> 5) + 1), word(t, cd.bit_off >> 5),
                                                    cd.bit_off & 31) & ((1u << cd.width) - 1u);
        v = cent[cd.cent_base + f];
      }
      if (m > 0 && i < d_eff) {
        float s = 0.0f;
        for (int j = 0; j < m; ++j) {
          const int pos = hd->code_bits + j;
          const float sgn = ((word(t, pos >> 5) >> (pos & 31)) & 1u) ? 1.0f : -1.0f;
          s = fmaf(sgn, S[j * d_eff + i], s);
        }
        v += hd->qjl_scale * half_bits_to_f32(word(t, W - 1) >> 16) * s;
      }
    }
    yb[tt * 257 + i] = v;
  }
  __syncthreads();
  for (int k = tid; k < 16 * d; k += blockDim.x) {
    const int tt = k / d, j = k % d;
    const int64_t t = tbase + tt;
    if (t >= a.n_tokens) continue;
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(R[(size_t)i * d + j], yb[tt * 257 + i], s);
    a.out[(((int64_t)b * a.n_heads + h) * a.n_tokens + t) * d + j] = s;
  }
}

// ------------------------------------------------------------------ host side

static int device_lds_limit() {
  int dev = 0, v = 65536;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  return v;
}

static sq_status check_handle(const sq_calib *c, const char *fn) {
  if (!c) return fail(SQ_ERR_ARG, std::string(fn) + ": handle is NULL");
  if (!c->dev_blob) return fail(SQ_ERR_STATE, std::string(fn) + ": calibration not uploaded (call sq_calib_upload)");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev != c->device)
    return fail(SQ_ERR_STATE, std::string(fn) + ": calibration was uploaded to another device");
  return SQ_OK;
}

// calibration heads used: first_head + b*cbs + h for b < batch, h < n_heads
static sq_status check_heads(const sq_calib *c, int first_head, int n_heads, int batch, int cbs,
                             const char *fn) {
  const int64_t nh = (int64_t)c->heads.size();
  if (n_heads <= 0 || batch < 0 || cbs < 0 || first_head < 0)
    return fail(SQ_ERR_ARG, std::string(fn) + ": bad head range (need n_heads > 0, batch, cbs, first_head >= 0)");
  const int64_t last = (int64_t)first_head + (int64_t)std::max(0, batch - 1) * cbs + n_heads - 1;
  if (last >= nh) return fail(SQ_ERR_ARG, std::string(fn) + ": calibration head index out of range");
  const int d = c->heads[first_head].d;
  for (int64_t k = first_head; k <= last; ++k)
    if (c->heads[k].d != d) return fail(SQ_ERR_ARG, std::string(fn) + ": heads of different head_dim");
  return SQ_OK;
}

static sq_status check_slots(const sq_calib *c, int64_t n_tokens, int n_heads, int batch, int64_t ps_b,
                             int64_t ps_h, const char *fn) {
  const int64_t need = ((n_tokens + 63) / 64) * 64 * (int64_t)c->W_max;
  if (ps_h < need) return fail(SQ_ERR_ARG, std::string(fn) + ": ps_head smaller than sq_packed_head_words");
  if (batch > 1 && ps_b < ps_h * n_heads) return fail(SQ_ERR_ARG, std::string(fn) + ": ps_batch overlaps head slots");
  return SQ_OK;
}

static sq_status launched(const char *fn) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(fn, e);
  clear_error();
  return SQ_OK;
}

}  // namespace sq

using namespace sq;

extern "C" sq_status sq_calib_upload(sq_calib *c, sq_stream stream) {
  if (!c) return fail(SQ_ERR_ARG, "sq_calib_upload: handle is NULL");
  sq_status st = upload_tables(c, stream);
  if (st == SQ_OK) clear_error();
  return st;
}

template <int D, bool F32, bool TG>
static void launch_compress(dim3 grid, size_t lds, hipStream_t s, const CompressArgs &a) {
  hipLaunchKernelGGL((compress_kernel<D, F32, TG>), grid, dim3(4 * D), lds, s, a);
}

template <int D, bool F32>
static void launch_compress2(int rsc, dim3 grid, size_t lds, hipStream_t s, const Compress2Args &a) {
  // record strides this head size can need (at most C2_WMAX words per wave)
  if (rsc == 17) {
    hipLaunchKernelGGL((compress2_kernel<D, F32, 17>), grid, dim3(4 * D), lds, s, a);
  } else if constexpr (D >= 64) {
    if (rsc == 33) hipLaunchKernelGGL((compress2_kernel<D, F32, 33>), grid, dim3(4 * D), lds, s, a);
    else if constexpr (D == 128) hipLaunchKernelGGL((compress2_kernel<D, F32, 49>), grid, dim3(4 * D), lds, s, a);
  }
}

template <int D>
static void launch_compress_d(bool f32, bool tg, dim3 grid, size_t lds, hipStream_t s, const CompressArgs &a) {
  if (f32) tg ? launch_compress<D, true, true>(grid, lds, s, a) : launch_compress<D, true, false>(grid, lds, s, a);
  else tg ? launch_compress<D, false, true>(grid, lds, s, a) : launch_compress<D, false, false>(grid, lds, s, a);
}

static int device_cu_count() {
  int dev = 0, v = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  return v;
}

// sq_compress and sq_compress_append: source token i of x goes to token slot
// token0 + i of every head's packed slot.
static sq_status compress_impl(const char *fn, const sq_calib *c, int first_head, int n_heads, int batch,
                               int calib_batch_stride, const void *x, sq_dtype dt, int64_t n_tokens,
                               int64_t xs_batch, int64_t xs_head, int64_t xs_token, uint32_t *packed,
                               int64_t ps_batch, int64_t ps_head, int64_t token0, sq_stream stream) {
  const std::string f(fn);
  sq_status st = check_handle(c, fn);
  if (st != SQ_OK) return st;
  st = check_heads(c, first_head, n_heads, batch, calib_batch_stride, fn);
  if (st != SQ_OK) return st;
  if (n_tokens < 0) return fail(SQ_ERR_ARG, f + ": n_tokens < 0");
  if (token0 < 0) return fail(SQ_ERR_ARG, f + ": token0 < 0");
  if (dt != SQ_F32 && dt != SQ_BF16) return fail(SQ_ERR_ARG, f + ": bad dtype");
  if (n_tokens == 0 || batch == 0) { clear_error(); return SQ_OK; }
  if (!x || !packed) return fail(SQ_ERR_ARG, f + ": NULL pointer");
  if (n_tokens > ((int64_t)1 << 36) || token0 > ((int64_t)1 << 36))
    return fail(SQ_ERR_UNSUPPORTED, f + ": too many tokens");
  st = check_slots(c, token0 + n_tokens, n_heads, batch, ps_batch, ps_head, fn);
  if (st != SQ_OK) return st;
  const int esz = dt == SQ_F32 ? 4 : 2;
  if (((uintptr_t)x % 16) || (xs_token * esz) % 16 || (xs_head * esz) % 16 || (xs_batch * esz) % 16)
    return fail(SQ_ERR_ARG, f + ": x and its strides must be 16-byte aligned");
  const int d = c->heads[first_head].d;
  if (xs_token < d) return fail(SQ_ERR_ARG, f + ": xs_token < head_dim");
  // source tiles: enough to reach the end of the last destination tile (with
  // token0 % 64 != 0 the last one only zero-fills the tail of that tile)
  const int64_t send = ((token0 + n_tokens + 63) / 64) * 64 - token0;
  const int n_src_tiles = (int)((send + 63) / 64);
  // LDS: threshold trees | signal centroids | x tile | y tile | word buffer
  int max_tree = 0, max_csig = 0, max_plan = 0, max_s = 0;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_heads; ++h) {
      const int k = first_head + bb * calib_batch_stride + h;
      const DevHead &hd = c->host_desc[k];
      max_tree = std::max(max_tree, hd.n_tree);
      max_csig = std::max(max_csig, hd.n_csig);
      max_plan = std::max(max_plan, (hd.d / 16 + hd.n_chunks + 1) * PLAN_WORDS);
      max_s = std::max(max_s, hd.m * hd.d_eff);
    }
    if (calib_batch_stride == 0) break;  // every batch entry uses the same heads
  }
  // register-quantising kernel when every head has its plan and the tables fit
  {
    // (the kernel's per-lane load offsets within a 64-token tile are 32-bit;
    // each of its d/16 waves stores at most C2_WMAX record words per tile)
    bool use2 = d <= 128 && 64 * xs_token * esz < ((int64_t)1 << 32) && c->W_max <= C2_WMAX * (d / 16) &&
                n_heads <= 65535 && batch <= 65535;
    int mt = 0, mc = 0, mq = 0;
    for (int bb = 0; bb < std::max(1, batch) && use2; ++bb) {
      for (int h = 0; h < n_heads; ++h) {
        const DevHead &hd = c->host_desc[first_head + bb * calib_batch_stride + h];
        if (hd.n_p2 == 0) use2 = false;
        mt = std::max(mt, hd.n_tree2);
        mc = std::max(mc, hd.n_csig2);
        mq = std::max(mq, hd.m);
      }
      if (calib_batch_stride == 0) break;
    }
    if (use2) {
      Compress2Args b2{};
      const bool f32 = dt == SQ_F32;
      b2.lds_tree_off = 0;
      b2.lds_csig_off = (mt + 3) & ~3;
      b2.lds_s_off = b2.lds_csig_off + ((mc + 3) & ~3);
      b2.lds_x_off = (b2.lds_s_off + mq * C2_SP + 255) & ~255;  // 1 KB aligned: direct-to-LDS blocks
      b2.x_buf_floats = 16 * d * (f32 ? 4 : 2);                 // 64 rows of d elements
      b2.lds_rec_off = b2.lds_x_off + 2 * b2.x_buf_floats;
      // record tile stride: odd, above W_max (pad column)
      const int rsc = c->W_max < 17 ? 17 : c->W_max < 33 ? 33 : 49;
      b2.lds_res_off = (b2.lds_rec_off + 3 * 64 * rsc + 3) & ~3;
      const size_t lds2 = (size_t)(b2.lds_res_off + 2 * 64 * C2_RS) * 4;
      if (lds2 <= (size_t)device_lds_limit()) {
        b2.heads = c->dev_heads;
        b2.blob = (const uint8_t *)c->dev_blob;
        b2.x = x;
        b2.packed = packed;
        b2.xs_b = xs_batch; b2.xs_h = xs_head; b2.xs_t = xs_token;
        b2.ps_b = ps_batch; b2.ps_h = ps_head;
        b2.n_tokens = n_tokens;
        b2.token0 = token0;
        b2.first_head = first_head;
        b2.cbs = calib_batch_stride;
        b2.n_tiles = n_src_tiles;
        // about 4 workgroups per CU, each a run of consecutive tiles of one
        // (batch entry, head)
        const int64_t want = (int64_t)device_cu_count() * 4;
        const int64_t bh = (int64_t)n_heads * batch;
        const int64_t chunks = std::max<int64_t>(1, std::min<int64_t>(b2.n_tiles, (want + bh - 1) / bh));
        b2.tiles_per_wg = (int)((b2.n_tiles + chunks - 1) / chunks);
        dim3 grid((unsigned)((b2.n_tiles + b2.tiles_per_wg - 1) / b2.tiles_per_wg), n_heads, batch);
        hipStream_t s = (hipStream_t)stream;
        switch (d) {
          case 32: f32 ? launch_compress2<32, true>(rsc, grid, lds2, s, b2) : launch_compress2<32, false>(rsc, grid, lds2, s, b2); break;
          case 64: f32 ? launch_compress2<64, true>(rsc, grid, lds2, s, b2) : launch_compress2<64, false>(rsc, grid, lds2, s, b2); break;
          default: f32 ? launch_compress2<128, true>(rsc, grid, lds2, s, b2) : launch_compress2<128, false>(rsc, grid, lds2, s, b2); break;
        }
        return launched(fn);
      }
    }
  }
  CompressArgs a{};
  a.ys = d + 3;  // odd, and conflict-free for the MFMA-layout stores
  a.bws = (c->W_max % 2 == 0) ? c->W_max + 1 : c->W_max;
  const int xs_floats = dt == SQ_F32 ? 64 * (d + 4) : 64 * (d + 8) / 2;
  const bool s_in_lds = max_s <= 4096;  // a large sketch is read from the L1/L2 instead
  const int s_floats = s_in_lds ? ((max_s + 3) & ~3) : 0;
  const int rest = ((max_csig + 3) & ~3) + max_plan + s_floats + 64 + xs_floats + 64 * a.ys + 64 * a.bws;
  const size_t limit = (size_t)device_lds_limit();
  const size_t lds_in = (size_t)(((max_tree + 3) & ~3) + rest) * 4, lds_out = (size_t)rest * 4;
  // trees stay in LDS unless moving them out is what lets two workgroups share a CU
  const bool tg = lds_in > limit || (lds_in > limit / 2 && lds_out <= limit / 2);
  const int tree_floats = tg ? 0 : ((max_tree + 3) & ~3);
  a.lds_csig_off = tree_floats;
  a.lds_plan_off = a.lds_csig_off + ((max_csig + 3) & ~3);
  a.lds_s_off = s_in_lds ? a.lds_plan_off + max_plan : -1;
  a.lds_sp_off = a.lds_plan_off + max_plan + s_floats;
  a.lds_x_off = a.lds_sp_off + 64;
  a.lds_y_off = a.lds_x_off + xs_floats;
  a.lds_b_off = a.lds_y_off + 64 * a.ys;
  const size_t lds = (size_t)(a.lds_b_off + 64 * a.bws) * 4;
  if (lds > limit)
    return fail(SQ_ERR_UNSUPPORTED, f + ": calibration tables exceed the LDS of one workgroup");
  a.heads = c->dev_heads;
  a.blob = (const uint8_t *)c->dev_blob;
  a.x = x;
  a.packed = packed;
  a.xs_b = xs_batch; a.xs_h = xs_head; a.xs_t = xs_token;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.n_tokens = n_tokens;
  a.token0 = token0;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_tiles = n_src_tiles;
  const int gz = calib_batch_stride ? batch : 1;
  a.items = calib_batch_stride ? a.n_tiles : (int)std::min<int64_t>((int64_t)batch * a.n_tiles, INT32_MAX);
  // enough resident workgroups to keep every CU busy; each walks many tiles
  const int64_t want = (int64_t)device_cu_count() * (d >= 256 ? 1 : 2) * 2;
  int gx = (int)std::max<int64_t>(1, std::min<int64_t>(a.items, (want + (int64_t)n_heads * gz - 1) / ((int64_t)n_heads * gz)));
  dim3 grid(gx, n_heads, gz);
  if (grid.y > 65535 || grid.z > 65535) return fail(SQ_ERR_UNSUPPORTED, f + ": too many heads or batch entries");
  hipStream_t s = (hipStream_t)stream;
  const bool f32 = dt == SQ_F32;
  switch (d) {
    case 32:  launch_compress_d<32>(f32, tg, grid, lds, s, a); break;
    case 64:  launch_compress_d<64>(f32, tg, grid, lds, s, a); break;
    case 128: launch_compress_d<128>(f32, tg, grid, lds, s, a); break;
    case 256: launch_compress_d<256>(f32, tg, grid, lds, s, a); break;
    default: return fail(SQ_ERR_UNSUPPORTED, f + ": head_dim");
  }
  return launched(fn);
}

extern "C" sq_status sq_compress(const sq_calib *c, int first_head, int n_heads, int batch,
                                 int calib_batch_stride, const void *x, sq_dtype dt,
                                 int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                                 int64_t xs_token, uint32_t *packed, int64_t ps_batch,
                                 int64_t ps_head, sq_stream stream) {
  return compress_impl("sq_compress", c, first_head, n_heads, batch, calib_batch_stride, x, dt, n_tokens,
                       xs_batch, xs_head, xs_token, packed, ps_batch, ps_head, 0, stream);
}

extern "C" sq_status sq_compress_append(const sq_calib *c, int first_head, int n_heads, int batch,
                                        int calib_batch_stride, const void *x, sq_dtype dt,
                                        int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                                        int64_t xs_token, uint32_t *packed, int64_t ps_batch,
                                        int64_t ps_head, int64_t token0, sq_stream stream) {
  return compress_impl("sq_compress_append", c, first_head, n_heads, batch, calib_batch_stride, x, dt,
                       n_tokens, xs_batch, xs_head, xs_token, packed, ps_batch, ps_head, token0, stream);
}

template <int GR, int SLOTB, int R, bool LG>
static void launch_scores(dim3 grid, size_t lds, hipStream_t s, const ScoresArgs &a) {
  hipLaunchKernelGGL((scores_kernel<GR, SLOTB, R, LG>), grid, dim3(SC_BLOCK), lds, s, a);
}

// The LDS-table kernels address their tables at absolute LDS addresses: true
// when the kernel declares no static LDS (the dynamic area then starts at 0).
template <int GR>
static bool scores_lds0_ok(int slotb) {
  auto ok = [](const void *k) {
    hipFuncAttributes fa{};
    return hipFuncGetAttributes(&fa, k) == hipSuccess && fa.sharedSizeBytes == 0;
  };
  static const bool ok8 = ok(reinterpret_cast<const void *>(&scores_kernel<GR, 8192, 6, false>));
  static const bool ok16 = ok(reinterpret_cast<const void *>(&scores_kernel<GR, 16384, 3, false>));
  return slotb == 8192 ? ok8 : ok16;
}

template <int GR, bool LG>
static void launch_scores_slot(int slotb, dim3 grid, size_t lds, hipStream_t s, const ScoresArgs &a) {
  if (slotb == 8192) launch_scores<GR, 8192, 6, LG>(grid, lds, s, a);
  else launch_scores<GR, 16384, 3, LG>(grid, lds, s, a);
}

extern "C" sq_status sq_scores(const sq_calib *kc, int first_head, int calib_batch_stride, int batch,
                               int n_q_heads, int n_kv_heads, const void *q, sq_dtype qdt,
                               const uint32_t *kpacked, int64_t ps_batch, int64_t ps_head,
                               int64_t n_tokens, float *scores, sq_stream stream) {
  const char *fn = "sq_scores";
  sq_status st = check_handle(kc, fn);
  if (st != SQ_OK) return st;
  if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads)
    return fail(SQ_ERR_ARG, "sq_scores: n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G > 8) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: query group larger than 8");
  st = check_heads(kc, first_head, n_kv_heads, batch, calib_batch_stride, fn);
  if (st != SQ_OK) return st;
  if (n_tokens < 0) return fail(SQ_ERR_ARG, "sq_scores: n_tokens < 0");
  if (qdt != SQ_F32 && qdt != SQ_BF16) return fail(SQ_ERR_ARG, "sq_scores: bad dtype");
  if (n_tokens == 0 || batch == 0) { clear_error(); return SQ_OK; }
  if (!q || !kpacked || !scores) return fail(SQ_ERR_ARG, "sq_scores: NULL pointer");
  st = check_slots(kc, n_tokens, n_kv_heads, batch, ps_batch, ps_head, fn);
  if (st != SQ_OK) return st;
  if (n_tokens > ((int64_t)1 << 36)) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: too many tokens");
  const int d = kc->heads[first_head].d;
  int max_q = 1, max_plut = 1, max_m = 0, max_W = 1;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h) {
      const DevHead &D = kc->host_desc[first_head + bb * calib_batch_stride + h];
      if (D.d != d) return fail(SQ_ERR_ARG, "sq_scores: heads of one call must share head_dim");
      max_q = std::max(max_q, D.n_quads);
      max_plut = std::max(max_plut, D.n_plut);
      max_m = std::max(max_m, D.m);
      max_W = std::max(max_W, D.W);
    }
    if (calib_batch_stride == 0) break;
  }
  const int GR = (G + 3) / 4, GP = 4 * GR, QM = sc_qmax(GR);
  int ks = 1;
  while (ks < SC_WAVES && ((max_q + ks - 1) / ks > QM || (SC_WAVES / ks) * max_W * 256 + 256 > 16384)) ks *= 2;
  const int ts = SC_WAVES / ks;
  const int passes = (max_q + ks * QM - 1) / (ks * QM);
  const int need = ts * max_W * 256 + 256;  // a stream tile may read one row past its end
  int slotb;
  if (need <= 8192) slotb = 8192;
  else if (need <= 16384) slotb = 16384;
  else return fail(SQ_ERR_UNSUPPORTED, "sq_scores: records too long");
  const int R = slotb == 8192 ? 6 : 3;  // ring slots (kernel template)
  ScoresArgs a{};
  const int limit = device_lds_limit();
  auto layout = [&](bool lut_in_lds) {
    size_t off = 0;
    a.lds_lut = 0;
    off = lut_in_lds ? (((size_t)max_plut * 8 + 1023) & ~(size_t)1023) : 0;  // copied in 1 KB pieces
    a.lds_qt = (int)off;   off += (size_t)G * d * 4;
    off = (off + 15) & ~(size_t)15;
    a.lds_wq = (int)off;   off += (size_t)std::max(1, max_m) * GP * 4;
    off = (off + 1023) & ~(size_t)1023;
    a.lds_slot = (int)off; off += (size_t)R * slotb;
    a.lds_pbuf = (int)off; off += (size_t)2 * (slotb == 8192 ? 2 : 1) * SC_WAVES * GP * 64 * 4;  // parity x slots per barrier
    return off;
  };
  bool lg = false;
  size_t lds = layout(true);
  const bool lds0 = GR == 1 ? scores_lds0_ok<1>(slotb) : scores_lds0_ok<2>(slotb);
  if (lds > (size_t)limit || !lds0) {  // joint tables too large for LDS: read them through the caches
    lg = true;
    lds = layout(false);
  }
  if (lds > (size_t)limit) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: tables exceed LDS");
  a.heads = kc->dev_heads;
  a.blob = (const uint8_t *)kc->dev_blob;
  a.q = q;
  a.kpacked = kpacked;
  a.scores = scores;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.n_tokens = n_tokens;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.G = G;
  a.q_f32 = qdt == SQ_F32;
  a.ks = ks;
  a.ts = ts;
  a.dma16 = ((uintptr_t)kpacked % 16 == 0) && ps_batch % 4 == 0 && ps_head % 4 == 0;
  a.n_tiles = (int)((n_tokens + 63) / 64);
  // one workgroup per CU at a time: about two per CU over the launch
  const int64_t pairs = (int64_t)batch * n_kv_heads;
  const int64_t want = (int64_t)device_cu_count() * 2;
  const int64_t steps = (a.n_tiles + ts - 1) / ts;
  int64_t chunks = std::max<int64_t>(1, std::min<int64_t>(steps, (want + pairs - 1) / pairs));
  a.tiles_per_wg = (int)(((steps + chunks - 1) / chunks) * ts);
  chunks = (a.n_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  dim3 grid((unsigned)chunks, n_kv_heads, batch);
  if (grid.z > 65535 || grid.y > 65535) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: grid too large");
  hipStream_t s = (hipStream_t)stream;
  for (int p = 0; p < passes; ++p) {
    a.pass = p;
    if (GR == 1) {
      if (lg) launch_scores_slot<1, true>(slotb, grid, lds, s, a);
      else launch_scores_slot<1, false>(slotb, grid, lds, s, a);
    } else {
      if (lg) launch_scores_slot<2, true>(slotb, grid, lds, s, a);
      else launch_scores_slot<2, false>(slotb, grid, lds, s, a);
    }
  }
  return launched(fn);
}

extern "C" size_t sq_attend_workspace_bytes(int batch, int n_q_heads, int64_t n_tokens, int head_dim) {
  if (batch <= 0 || n_q_heads <= 0 || n_tokens <= 0 || head_dim <= 0) return 0;
  const int64_t ct = attend_chunk_tokens(batch, n_q_heads, n_tokens);
  const int64_t nch = (n_tokens + ct - 1) / ct;
  return (size_t)batch * n_q_heads * nch * (head_dim + 2) * sizeof(float);
}

// The column-table kernel addresses its tables at LDS address 0: true when
// the kernel declares no static LDS (the dynamic area then starts at 0).  The
// 16-wave kernel (at most 128 VGPRs) is taken only where it needs no scratch.
template <int G, int NP, int WPB, int NBUF = 2>
static bool attend_col_ok() {
  static const bool ok = [] {
    hipFuncAttributes fa{};
    return hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(&attend_partial_kernel<G, LM_COL, NP, WPB, NBUF>)) ==
               hipSuccess && fa.sharedSizeBytes == 0 && (WPB < 16 || fa.localSizeBytes == 0);
  }();
  return ok;
}

// lm == LM_COL with wpb 16 (single-buffered) or 8, or any placement with wpb
// 4 (the host checked that the column kernel has no static LDS before
// choosing LM_COL)
template <int G, int NP>
static void launch_attend_np(int lm, int wpb, dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a) {
  if (lm == LM_COL && wpb == 16) hipLaunchKernelGGL((attend_partial_kernel<G, LM_COL, NP, 16, 1>), grid, dim3(1024), lds, s, a);
  else if (lm == LM_COL && wpb == 8) hipLaunchKernelGGL((attend_partial_kernel<G, LM_COL, NP, 8>), grid, dim3(512), lds, s, a);
  else if (lm == LM_COL) hipLaunchKernelGGL((attend_partial_kernel<G, LM_COL, NP, 4>), grid, dim3(256), lds, s, a);
  else if (lm == LM_PACK) hipLaunchKernelGGL((attend_partial_kernel<G, LM_PACK, NP, 4>), grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((attend_partial_kernel<G, LM_GLB, NP, 4>), grid, dim3(256), lds, s, a);
}

template <int G, int NP>
static bool attend_col_ok_np(int wpb) {
  return wpb == 16 ? attend_col_ok<G, NP, 16, 1>() : wpb == 8 ? attend_col_ok<G, NP, 8>() : attend_col_ok<G, NP, 4>();
}

template <int G>
static bool attend_col_ok_g(int np, int wpb) {
  return np == 1 ? attend_col_ok_np<G, 1>(wpb) : np == 2 ? attend_col_ok_np<G, 2>(wpb) : attend_col_ok_np<G, 4>(wpb);
}

template <int G>
static void launch_attend(int lm, int np, int wpb, dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a) {
  if (np == 1) launch_attend_np<G, 1>(lm, wpb, grid, lds, s, a);
  else if (np == 2) launch_attend_np<G, 2>(lm, wpb, grid, lds, s, a);
  else launch_attend_np<G, 4>(lm, wpb, grid, lds, s, a);
}

extern "C" sq_status sq_attend(const sq_calib *vc, int first_head, int calib_batch_stride, int batch,
                               int n_q_heads, int n_kv_heads, const float *scores, float scale,
                               const uint32_t *vpacked, int64_t ps_batch, int64_t ps_head,
                               int64_t n_tokens, void *workspace, size_t ws_bytes, float *out,
                               sq_stream stream) {
  const char *fn = "sq_attend";
  sq_status st = check_handle(vc, fn);
  if (st != SQ_OK) return st;
  if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads)
    return fail(SQ_ERR_ARG, "sq_attend: n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G > 8) return fail(SQ_ERR_UNSUPPORTED, "sq_attend: query group larger than 8");
  st = check_heads(vc, first_head, n_kv_heads, batch, calib_batch_stride, fn);
  if (st != SQ_OK) return st;
  if (n_tokens < 0) return fail(SQ_ERR_ARG, "sq_attend: n_tokens < 0");
  if (batch == 0) { clear_error(); return SQ_OK; }
  if (!out) return fail(SQ_ERR_ARG, "sq_attend: out is NULL");
  const int d = vc->heads[first_head].d;
  AttendArgs a{};
  a.heads = vc->dev_heads;
  a.blob = (const uint8_t *)vc->dev_blob;
  a.scores = scores;
  a.vpacked = vpacked;
  a.out = out;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.n_tokens = n_tokens;
  a.scale = scale;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  if (n_tokens == 0) {
    a.n_chunks = 0;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * n_q_heads), dim3(256), 0, s, a);
    return launched(fn);
  }
  if (!scores || !vpacked || !workspace) return fail(SQ_ERR_ARG, "sq_attend: NULL pointer");
  st = check_slots(vc, n_tokens, n_kv_heads, batch, ps_batch, ps_head, fn);
  if (st != SQ_OK) return st;
  if (ws_bytes < sq_attend_workspace_bytes(batch, n_q_heads, n_tokens, d))
    return fail(SQ_ERR_ARG, "sq_attend: workspace too small");
  a.ws = (float *)workspace;
  a.chunk_tokens = (int)attend_chunk_tokens(batch, n_q_heads, n_tokens);
  a.n_chunks = (int)((n_tokens + a.chunk_tokens - 1) / a.chunk_tokens);
  const int np = (d + 63) / 64;  // 64-coordinate blocks, all served by one wave
  if (np != 1 && np != 2 && np != 4) return fail(SQ_ERR_UNSUPPORTED, "sq_attend: unsupported head_dim");
  // LDS: centroid tables of the blocks | ATT_WAVES x (two staging buffers, weights)
  int max_lut = 1, max_wd = 1, max_w = 0;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h) {
      const HeadCal &hc = vc->heads[first_head + bb * calib_batch_stride + h];
      max_wd = std::max(max_wd, hc.W);
      for (int pt = 0; pt < np; ++pt) {
        const int c0 = pt * 64, c1 = std::min(d, c0 + 64);
        const int lut1 = c1 < d ? hc.cent_base[c1] : hc.n_cent;
        max_lut = std::max(max_lut, lut1 - hc.cent_base[c0]);
        for (int i = c0; i < c1; ++i) max_w = std::max(max_w, hc.widths[i]);
      }
    }
    if (calib_batch_stride == 0) break;
  }
  const int GP = ((G + 3) / 4) * 4;
  const int limit = device_lds_limit();
  a.buf_floats = (max_wd + 2) * ATT_RS + G * 64;
  a.wave_floats = 2 * a.buf_floats + 2 * GP * ATT_PS;
  auto lds_for = [&](int block_floats, int wpb) {
    a.lut_block = block_floats;
    a.lds_wave_off = (np * block_floats + 3) & ~3;
    return (size_t)(a.lds_wave_off + wpb * a.wave_floats) * 4;
  };
  auto col_ok = [&](int wpb) {
    switch (G) {
      case 1: return attend_col_ok_g<1>(np, wpb);
      case 2: return attend_col_ok_g<2>(np, wpb);
      case 3: return attend_col_ok_g<3>(np, wpb);
      case 4: return attend_col_ok_g<4>(np, wpb);
      case 5: return attend_col_ok_g<5>(np, wpb);
      case 6: return attend_col_ok_g<6>(np, wpb);
      case 7: return attend_col_ok_g<7>(np, wpb);
      default: return attend_col_ok_g<8>(np, wpb);
    }
  };
  // table placement: column tables (conflict-free), shared by 16 waves with
  // one staging buffer each when that fits a CU (four waves per SIMD), else
  // by 8 double-buffered waves when that keeps as many waves per CU as
  // 4-wave workgroups would (fewer table copies); else 4-wave workgroups with
  // column tables unless packed tables let more of them share a CU
  int lm = LM_GLB, wpb = 4;
  size_t lds = 0;
  const size_t cu_lds = (size_t)limit;  // one workgroup may use all of a CU's LDS
  const size_t cap = (size_t)std::min(limit, 64 * 1024);
  const size_t lds_col = max_w <= 6 ? lds_for(64 << max_w, 4) : cap + 1;
  const size_t lds_col8 = max_w <= 6 ? lds_for(64 << max_w, 8) : cu_lds + 1;
  const size_t lds_pack = lds_for(max_lut + 64, 4);
  const int wf2 = a.wave_floats, wf1 = a.buf_floats + 2 * GP * ATT_PS;
  a.wave_floats = wf1;
  const size_t lds_col16 = max_w <= 6 ? lds_for(64 << max_w, 16) : cu_lds + 1;
  a.wave_floats = wf2;
  if (lds_col16 <= cu_lds && col_ok(16)) {
    lm = LM_COL;
    wpb = 16;
    a.wave_floats = wf1;
    lds = lds_for(64 << max_w, 16);
  } else if (lds_col8 <= cu_lds && 8 * (cu_lds / lds_col8) >= 4 * (cu_lds / std::min(lds_col, lds_pack)) && col_ok(8)) {
    lm = LM_COL;
    wpb = 8;
    lds = lds_for(64 << max_w, 8);
  } else if (lds_col <= cap && cu_lds / lds_col >= cu_lds / lds_pack && col_ok(4)) {
    lm = LM_COL;
    lds = lds_for(64 << max_w, 4);
  } else if (lds_pack <= cap) {
    lm = LM_PACK;
    lds = lds_for(max_lut + 64, 4);
  } else {
    lds = lds_for(0, 4);
  }
  if (lds > (size_t)limit) return fail(SQ_ERR_UNSUPPORTED, "sq_attend: tables exceed LDS");
  const int64_t cgroups = (a.n_chunks + wpb - 1) / wpb;
  dim3 grid((unsigned)cgroups, n_kv_heads, batch);
  if (grid.z > 65535 || grid.y > 65535 || cgroups > INT32_MAX)
    return fail(SQ_ERR_UNSUPPORTED, "sq_attend: grid too large");
  switch (G) {
    case 1: launch_attend<1>(lm, np, wpb, grid, lds, s, a); break;
    case 2: launch_attend<2>(lm, np, wpb, grid, lds, s, a); break;
    case 3: launch_attend<3>(lm, np, wpb, grid, lds, s, a); break;
    case 4: launch_attend<4>(lm, np, wpb, grid, lds, s, a); break;
    case 5: launch_attend<5>(lm, np, wpb, grid, lds, s, a); break;
    case 6: launch_attend<6>(lm, np, wpb, grid, lds, s, a); break;
    case 7: launch_attend<7>(lm, np, wpb, grid, lds, s, a); break;
    case 8: launch_attend<8>(lm, np, wpb, grid, lds, s, a); break;
  }
  sq_status s1 = launched(fn);
  if (s1 != SQ_OK) return s1;
  const size_t lds2 = (size_t)(a.n_chunks + d) * 4;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * n_q_heads), dim3(256), lds2, s, a);
  return launched(fn);
}

extern "C" sq_status sq_dequantize(const sq_calib *c, int first_head, int n_heads, int batch,
                                   int calib_batch_stride, const uint32_t *packed, int64_t ps_batch,
                                   int64_t ps_head, int64_t n_tokens, float *out, sq_stream stream) {
  const char *fn = "sq_dequantize";
  sq_status st = check_handle(c, fn);
  if (st != SQ_OK) return st;
  st = check_heads(c, first_head, n_heads, batch, calib_batch_stride, fn);
  if (st != SQ_OK) return st;
  if (n_tokens < 0) return fail(SQ_ERR_ARG, "sq_dequantize: n_tokens < 0");
  if (n_tokens == 0 || batch == 0) { clear_error(); return SQ_OK; }
  if (!packed || !out) return fail(SQ_ERR_ARG, "sq_dequantize: NULL pointer");
  st = check_slots(c, n_tokens, n_heads, batch, ps_batch, ps_head, fn);
  if (st != SQ_OK) return st;
  DequantArgs a{};
  a.heads = c->dev_heads;
  a.blob = (const uint8_t *)c->dev_blob;
  a.packed = packed;
  a.out = out;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.n_tokens = n_tokens;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_heads = n_heads;
  dim3 grid((unsigned)((n_tokens + 15) / 16), n_heads, batch), block(256);
  hipLaunchKernelGGL(dequant_kernel, grid, block, 0, (hipStream_t)stream, a);
  return launched(fn);
}
