// Upload of a calibration handle's tables to the device: the per-head
// device blob (rotation fragments, threshold trees, centroid tables, score
// schedule and joint tables, compress plans).

#include "devcommon.h"

namespace sq {

// ------------------------------------------------------------------ upload

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


// Fused decode schedule of one head (FS layout in devtypes.h).
struct FusedSched {
  std::vector<uint32_t> words;  // FS layout (devtypes.h)
  int n_groups = 0, n_ent = 0, n_qjl = 0;
};

// Empty schedule (n_groups = 0: sq_decode refuses the head) when a window
// holds more than FS_SLOTS code groups or the QJL bits do not lie in the
// record's last two words (m > 16).
static FusedSched build_fused_sched(const HeadCal &hc) {
  struct Grp { int pos, width, first, count; bool qjl; };
  std::vector<Grp> g;
  const int d = hc.d;
  for (int i = 0; i < d;) {
    if (hc.widths[i] == 0) { ++i; continue; }
    Grp cur{hc.bit_off[i], hc.widths[i], i, 1, false};
    int j = i + 1;
    // extend over following coordinates (zero-width ones add no bits)
    while (j < d && cur.width + hc.widths[j] <= FG_BITS && cur.width <= FG_BITS) {
      cur.width += hc.widths[j];
      ++j;
    }
    // trailing zero-width coordinates are not part of the group
    while (j > i + 1 && hc.widths[j - 1] == 0) --j;
    cur.count = j - i;
    g.push_back(cur);
    i = j;
  }
  const int n_code = (int)g.size();
  for (int j = 0; j < hc.m; j += FG_BITS) {
    const int n = std::min(FG_BITS, hc.m - j);
    g.push_back(Grp{hc.code_bits + j, n, j, n, true});
  }
  FusedSched F;
  const int ng = (int)g.size(), nq = ng - n_code, W = hc.W;
  if (hc.m > 16) return F;
  // tables placed largest first: each starts at a multiple of its size
  std::vector<int> order(ng);
  for (int k = 0; k < ng; ++k) order[k] = k;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return g[x].width > g[y].width; });
  std::vector<uint32_t> e0(ng);
  uint32_t ent = 0;
  for (int k : order) {
    e0[k] = ent;
    ent += 1u << g[k].width;
  }
  const size_t slots_off = ((size_t)2 * ng + nq + 15) & ~(size_t)15;
  const size_t var_words = (size_t)(W + 1) * FS_SLOTS * 2;
  F.words.assign(slots_off + 3 * var_words + 3 * (size_t)(W + 1), 0u);
  uint32_t *Q = F.words.data() + 2 * ng;
  int iq = 0;
  for (int k = 0; k < ng; ++k) {
    const Grp &q = g[k];
    F.words[2 * k] = (uint32_t)q.width | (q.qjl ? 16u : 0u) | (e0[k] << 8);
    F.words[2 * k + 1] = (uint32_t)q.first | ((uint32_t)q.count << 12);
    if (q.qjl) {
      // within words qb, qb + 1, qb = W - 2 (W - 3 when the norm shares word W - 1
      // with gamma); word -1 reads as zero
      const int qb = W - 2 - (hc.normalized ? 1 : 0);
      const int rel = q.pos - 32 * qb;
      if (rel < 0 || rel + q.width > 64) return FusedSched{};
      Q[iq++] = (uint32_t)rel | ((uint32_t)q.width << 8) | (e0[k] << 12);
    }
  }
  // window slots, for table entries of 4, 8 and 16 bytes (E = 2, 3, 4): group
  // k with field at bit pos is read from window j = (pos + 32 - E) / 32 (the
  // 64 bits of words j - 1, j starting at bit (pos + 32 - E) % 32 of word j - 1,
  // so that the field lands at bit E); slot (shift | table byte offset << 5,
  // field mask << E); unused slots read the zero entry after the tables
  for (int v = 0; v < 3; ++v) {
    const int E = 2 + v;
    uint32_t *S = F.words.data() + slots_off + v * var_words;
    std::vector<int> used(W + 1, 0);
    uint32_t *Ncnt = F.words.data() + slots_off + 3 * var_words + (size_t)v * (W + 1);
    for (int j = 0; j <= W; ++j)
      for (int u = 0; u < FS_SLOTS; ++u) S[((size_t)j * FS_SLOTS + u) * 2] = (ent << E) << 5;
    for (int k = 0; k < n_code; ++k) {
      const Grp &q = g[k];
      const int j = (q.pos + 32 - E) / 32;
      if (j > W || used[j] == FS_SLOTS) return FusedSched{};
      uint32_t *sl = S + ((size_t)j * FS_SLOTS + used[j]++) * 2;
      sl[0] = (uint32_t)((q.pos + 32 - E) & 31) | ((e0[k] << E) << 5);
      sl[1] = ((1u << q.width) - 1u) << E;
    }
    for (int j = 0; j <= W; ++j) Ncnt[j] = (uint32_t)used[j];
  }
  F.n_groups = ng;
  F.n_qjl = nq;
  F.n_ent = (int)ent;
  return F;
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
    // (the last words also hold the QJL bits, gamma or the vector norm)
    const bool tail = hc.m > 0 || hc.normalized;
    const int ecode = (w == NW - 1 && tail) ? hc.code_bits : ebit[w];
    dfirst[w] = (sbit[w] + 31) / 32;
    dend[w] = std::max(dfirst[w], ecode / 32);
    if (w == NW - 1 && !tail) dend[w] = std::max(dfirst[w], hc.W);
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
  // 16-bit tree bases, 8-bit word indices in the kernel; the normalised
  // variant goes through compress_kernel
  P.ok = P.tree.size() < 65536 && hc.W < 256 && !hc.normalized;
  return P;
}

// Grid quantiser tables (GRID_* layout).  Only for heads the register plan
// serves (d <= 128, at most 16 signal dims and 32 QJL rows); fails (ok = false) when a region has a
// zero or repeated threshold gap, a coordinate of nonzero width has zero
// variance, or the cells of all regions exceed GRID_MAX_CELLS.
static uint32_t fbits(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  return u;
}

struct GridPlan {
  std::vector<uint32_t> coord;  // [d][GRID_COORD_WORDS]
  std::vector<uint32_t> cells;  // [n][2]
  std::vector<float> csig;
  bool ok = false;
};

static GridPlan build_grid(const HeadCal &hc) {
  GridPlan G;
  const int d = hc.d;
  if (d != 32 && d != 64 && d != 128) return G;
  if (hc.m > 0 && (hc.d_eff > 16 || hc.m > 32)) return G;
  const float inf = std::numeric_limits<float>::infinity();
  G.cells = {fbits(inf), 0u};  // cell 0: zero-width coordinates
  G.coord.assign((size_t)d * GRID_COORD_WORDS, 0u);
  constexpr double MARGIN = 1.0 / 512;
  // region (regime, width) -> (first cell, C, o, h)
  struct Reg { int first = -1, C = 0; double o = 0, h = 0; };
  Reg regs[2][9];
  for (int c = 0; c < d; ++c) {
    const int b = hc.widths[c];
    uint32_t *gc = G.coord.data() + (size_t)c * GRID_COORD_WORDS;
    gc[4] = 0xFFFFFFFFu;
    const int c0 = c & ~3;
    gc[5] = (uint32_t)(hc.bit_off[c] - hc.bit_off[c0]);
    gc[6] = (uint32_t)(hc.bit_off[c0] >> 5) | ((uint32_t)(hc.bit_off[c0] & 31) << 8);
    if (b == 0) continue;  // a = b = 0, cells at 0, C - 1 = 0
    const double sig = std::sqrt(hc.lam[c]);
    if (!(sig > 0)) return G;
    Reg &R = regs[c < hc.d_eff ? 0 : 1][b];
    const int n = (1 << b) - 1;
    if (R.first < 0) {
      std::vector<double> t(n);
      for (int j = 0; j < n; ++j) t[j] = (double)hc.thr[hc.thr_base[c] + j] / sig;
      double gmin = std::numeric_limits<double>::infinity();
      for (int j = 0; j + 1 < n; ++j) gmin = std::min(gmin, t[j + 1] - t[j]);
      if (n > 1 && !(gmin > 0)) return G;
      bool found = false;
      if (n == 1) {  // one cell around the only threshold
        R.h = 1.0;
        R.o = t[0] - 0.5;
        R.C = 1;
        found = true;
      }
      for (int fi = 0; fi < 10 && !found; ++fi) {
        const double h = gmin * (0.95 - 0.05 * fi);
        for (int k = 1; k < 512 && !found; ++k) {
          const double o = t[0] - h * (k / 512.0);
          bool good = true;
          for (int j = 0; j < n && good; ++j) {
            const double p = (t[j] - o) / h, fr = p - std::floor(p);
            good = fr >= MARGIN && fr <= 1 - MARGIN;
          }
          if (good) {
            R.h = h;
            R.o = o;
            R.C = (int)std::floor((t[n - 1] - o) / h) + 1;
            found = true;
          }
        }
      }
      if (!found || R.C > GRID_MAX_CELLS) return G;
      R.first = (int)(G.cells.size() / 2);
      std::vector<uint32_t> cell((size_t)R.C * 2);
      for (int k = 0; k < R.C; ++k) {
        cell[2 * k] = fbits(inf);
        cell[2 * k + 1] = 0u;
      }
      for (int j = 0; j < n; ++j) {
        const double p = (t[j] - R.o) / R.h;
        const int k = (int)std::floor(p);
        cell[2 * k] = fbits((float)p);
      }
      // code_lo(k) = thresholds in cells before k
      uint32_t cnt = 0;
      for (int k = 0; k < R.C; ++k) {
        cell[2 * k + 1] = cnt;
        if (cell[2 * k] != fbits(inf)) ++cnt;
      }
      G.cells.insert(G.cells.end(), cell.begin(), cell.end());
      if (G.cells.size() / 2 > (size_t)GRID_MAX_CELLS) return G;
    }
    gc[0] = fbits((float)(1.0 / (sig * R.h)));
    gc[1] = fbits((float)(-R.o / R.h));
    gc[2] = (uint32_t)R.first * 8u;
    gc[3] = (uint32_t)(R.C - 1);
    if (hc.m > 0 && c < hc.d_eff) {
      gc[4] = (uint32_t)G.csig.size();
      for (int k = 0; k <= n; ++k) G.csig.push_back(hc.cent[hc.cent_base[c] + k]);
    }
  }
  if (hc.m > 0)  // signal coordinates of zero width still need a centroid (0)
    for (int c = 0; c < hc.d_eff; ++c)
      if (hc.widths[c] == 0) {
        G.coord[(size_t)c * GRID_COORD_WORDS + 4] = (uint32_t)G.csig.size();
        G.csig.push_back(0.0f);
      }
  G.ok = true;
  return G;
}

sq_status upload_tables(sq_calib *c, void *stream) {
  const int nh = (int)c->heads.size();
  std::vector<HostPlan> plans(nh);
  for (int h = 0; h < nh; ++h) plans[h] = build_plan(c->heads[h]);
  std::vector<ScoreSched> scheds(nh);
  for (int h = 0; h < nh; ++h) scheds[h] = build_score_sched(c->heads[h]);
  std::vector<HostPlan2> plans2(nh);
  std::vector<FusedSched> fsch(nh);
  for (int h = 0; h < nh; ++h) fsch[h] = build_fused_sched(c->heads[h]);
  for (int h = 0; h < nh; ++h) plans2[h] = build_plan2(c->heads[h]);
  std::vector<GridPlan> grids(nh);
  for (int h = 0; h < nh; ++h) grids[h] = build_grid(c->heads[h]);
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
    D.normalized = hc.normalized ? 1 : 0;
    D.n_tree2 = (int)P2.tree.size();
    D.n_csig2 = (int)P2.csig.size();
    D.off_p2 = off;      off = align256(off + sizeof(uint32_t) * std::max<size_t>(1, P2.words.size()));
    D.off_tree2 = off;   off = align256(off + sizeof(float) * std::max<size_t>(1, P2.tree.size()));
    D.off_csig2 = off;   off = align256(off + sizeof(float) * std::max<size_t>(1, P2.csig.size()));
    D.off_Rfrag2 = off;  off = align256(off + (P2.ok ? sizeof(uint16_t) * 3 * d * d : 1));
    D.n_fgroups = fsch[h].n_groups;
    D.n_fent = fsch[h].n_ent;
    D.n_fqjl = fsch[h].n_qjl;
    D.off_fsched = off;  off = align256(off + sizeof(uint32_t) * fsch[h].words.size());
    const GridPlan &Gp = grids[h];
    D.n_gcells = Gp.ok ? (int)(Gp.cells.size() / 2) : 0;
    D.n_gcsig = Gp.ok ? (int)Gp.csig.size() : 0;
    D.off_gcoord = off;  off = align256(off + sizeof(uint32_t) * std::max<size_t>(1, Gp.coord.size()));
    D.off_gcells = off;  off = align256(off + sizeof(uint32_t) * std::max<size_t>(1, Gp.cells.size()));
    D.off_gcsig = off;   off = align256(off + sizeof(float) * std::max<size_t>(1, Gp.csig.size()));
    D.off_Rfrag_u = off; off = align256(off + (Gp.ok ? sizeof(uint16_t) * 3 * d * d : 1));
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
    // holds R_s[mb*16 + l%16][kb*32 + 8*(l/16) + e]; row_scale multiplies row i
    // (in double, before the split) by row_scale[i]
    const int MB = d / 16, KB = d / 32;
    auto fragments = [&](uint16_t *F, const std::vector<double> *row_scale) {
      for (int mb = 0; mb < MB; ++mb)
        for (int kb = 0; kb < KB; ++kb)
          for (int l = 0; l < 64; ++l)
            for (int e = 0; e < 8; ++e) {
              const int row = mb * 16 + (l & 15), col = kb * 32 + 8 * (l >> 4) + e;
              double v = hc.R[(size_t)row * d + col] * (row_scale ? (*row_scale)[row] : 1.0);
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
    };
    fragments((uint16_t *)(img.data() + D.off_Rfrag), nullptr);
    if (grids[h].ok) {
      // rows scaled by the grid's a_i (the float the kernel would multiply
      // by); a zero-width signal row keeps scale 1 (its u is y, its code 0)
      std::vector<double> a_row(d);
      for (int i = 0; i < d; ++i) {
        float av;
        std::memcpy(&av, &grids[h].coord[(size_t)i * GRID_COORD_WORDS + 0], 4);
        a_row[i] = (hc.widths[i] == 0 && hc.m > 0 && i < hc.d_eff) ? 1.0 : (double)av;
      }
      fragments((uint16_t *)(img.data() + D.off_Rfrag_u), &a_row);
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
    if (grids[h].ok) {
      const GridPlan &Gp = grids[h];
      std::memcpy(img.data() + D.off_gcoord, Gp.coord.data(), sizeof(uint32_t) * Gp.coord.size());
      std::memcpy(img.data() + D.off_gcells, Gp.cells.data(), sizeof(uint32_t) * Gp.cells.size());
      if (!Gp.csig.empty()) std::memcpy(img.data() + D.off_gcsig, Gp.csig.data(), sizeof(float) * Gp.csig.size());
    }
    DevCoord *Cd = (DevCoord *)(img.data() + D.off_coord);
    for (int i = 0; i < d; ++i) Cd[i] = DevCoord{hc.bit_off[i], hc.widths[i], hc.thr_base[i], hc.cent_base[i]};
    std::memcpy(img.data() + D.off_sched, scheds[h].quads.data(), sizeof(uint32_t) * scheds[h].quads.size());
    std::memcpy(img.data() + D.off_fsched, fsch[h].words.data(), sizeof(uint32_t) * fsch[h].words.size());
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

}  // namespace sq

using namespace sq;

extern "C" sq_status sq_calib_upload(sq_calib *c, sq_stream stream) {
  if (!c) return fail(SQ_ERR_ARG, "sq_calib_upload: handle is NULL");
  sq_status st = upload_tables(c, stream);
  if (st == SQ_OK) clear_error();
  return st;
}
