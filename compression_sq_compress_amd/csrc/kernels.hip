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
#include <cmath>
#include <cstring>
#include <limits>
#include <string>
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

sq_status upload_tables(sq_calib *c, void *stream) {
  const int nh = (int)c->heads.size();
  std::vector<HostPlan> plans(nh);
  for (int h = 0; h < nh; ++h) plans[h] = build_plan(c->heads[h]);
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
    D.off_R = off;       off = align256(off + sizeof(float) * d * d);
    D.off_Rfrag = off;   off = align256(off + sizeof(uint16_t) * 3 * d * d);
    D.off_coord = off;   off = align256(off + sizeof(DevCoord) * d);
    D.off_tree = off;    off = align256(off + sizeof(float) * std::max<size_t>(1, P.tree.size()));
    D.off_cent = off;    off = align256(off + sizeof(float) * std::max(1, hc.n_cent));
    D.off_S = off;       off = align256(off + sizeof(float) * std::max(1, hc.m * hc.d_eff));
    D.off_plan = off;    off = align256(off + sizeof(uint32_t) * P.words.size());
    D.off_desc = off;    off = align256(off + sizeof(uint32_t) * d);
    D.off_lutp = off;    off = align256(off + sizeof(uint32_t) * std::max(1, hc.n_cent));
    D.off_csig = off;    off = align256(off + sizeof(float) * std::max<size_t>(1, P.csig.size()));
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
    DevCoord *Cd = (DevCoord *)(img.data() + D.off_coord);
    uint32_t *Dd = (uint32_t *)(img.data() + D.off_desc);
    for (int i = 0; i < d; ++i) {
      Cd[i] = DevCoord{hc.bit_off[i], hc.widths[i], hc.thr_base[i], hc.cent_base[i]};
      Dd[i] = (uint32_t)hc.bit_off[i] | ((uint32_t)hc.widths[i] << 12) | ((uint32_t)hc.cent_base[i] << 16);
    }
    if (!P.tree.empty()) std::memcpy(img.data() + D.off_tree, P.tree.data(), sizeof(float) * P.tree.size());
    if (!P.csig.empty()) std::memcpy(img.data() + D.off_csig, P.csig.data(), sizeof(float) * P.csig.size());
    std::memcpy(img.data() + D.off_plan, P.words.data(), sizeof(uint32_t) * P.words.size());
    if (hc.n_cent) std::memcpy(img.data() + D.off_cent, hc.cent.data(), sizeof(float) * hc.n_cent);
    {
      uint32_t *Pp = (uint32_t *)(img.data() + D.off_lutp);
      for (int k = 0; k < hc.n_cent; ++k) {
        const float v = hc.cent[k];
        const uint16_t hi = f32_to_bf16_rne(v);
        float vh;
        uint32_t u = (uint32_t)hi << 16;
        std::memcpy(&vh, &u, 4);
        const uint16_t lo = f32_to_bf16_rne(v - vh);
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
        float r = y[c];
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
  bool pvalid = false;
  auto store_prev = [&]() {
    for (int k = dfirst; k < dend; ++k) pdst[(int64_t)k * 64] = pvalid ? bwrow[k] : 0u;
    for (int k = own_f; k < own_e; ++k) {
      if (k >= dfirst && k < dend) continue;
      pdst[(int64_t)k * 64] = pvalid ? bwrow[k] : 0u;
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
    pdst = a.packed + (int64_t)b * a.ps_b + (int64_t)h * a.ps_h + (int64_t)tile * W * 64 + lane;
    pvalid = t0 + lane < T;
    // The x tile was last read by the MFMAs, which every wave finished before
    // the barrier above; the y tile and the word buffer are rewritten only
    // after the barrier that follows the next x store.
  }
  if (pdst) store_prev();
}

// ------------------------------------------------------------------ scores
//
// A workgroup serves one (batch, KV head) and a run of 64-token tiles; each
// of its 4 waves takes NT tiles per pass, lane = token.
// Prologue: q~ = R q for the query heads of the group (fp32), w = S q~[:d_eff]
// scaled by sqrt(pi/2)/m, and the MFMA A operands built from q~ (below); the
// head's centroid table, as bf16 hi/lo pairs, goes to LDS.
// Pass: the NT tiles' record words are staged in lane-private LDS rows.  The
// lane walks the coordinates in order (wave-uniform bit positions, a two-word
// window per tile), fetches the pair (hi, lo) of C_i[code] and feeds it to
// v_mfma_f32_4x4x4_16b_bf16 as the B operand: in block b, lane 4b+n supplies
// column n = its own token.  The A operand rows are the query heads: for a
// coordinate pair (i, i+1) the k-slots are (hi_i, lo_i, hi_i+1, lo_i+1) x
// (qhi_i, qhi_i, qhi_i+1, qhi_i+1); every four coordinates one more MFMA adds
// (hi_i..hi_i+3) x (qlo_i..qlo_i+3).  So each token's score is accumulated
// for 4 query heads per MFMA, exact to ~2^-16 relative per term, and lands
// in the token's own lane (register m = head m), where the QJL term
// gamma * sum_j w_j (2 z_j - 1) is added before one coalesced store per head.

struct ScoresArgs {
  const DevHead *heads;
  const uint8_t *blob;
  const void *q;
  const uint32_t *kpacked;
  float *scores;
  int64_t ps_b, ps_h;
  int64_t n_tokens;
  int first_head, cbs;
  int n_q_heads, n_kv_heads;
  int q_f32;
  int n_tiles, tiles_per_block;
  int lds_lut_off, lds_aq_off, lds_w_off, lds_rec_off;  // floats
  int rec_tile;                                         // words per staged tile
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a),
                                                __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_pair(uint16_t x) { return (uint32_t)x | ((uint32_t)x << 16); }

template <int G, int NT, bool LG>
__global__ __launch_bounds__(256) void scores_kernel(ScoresArgs a) {
  extern __shared__ float smem[];
  constexpr int GR = (G + 3) / 4, GP = 4 * GR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int ch = a.first_head + b * a.cbs + hkv;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d, d_eff = hd->d_eff, m = hd->m, W = hd->W, n_cent = hd->n_cent;
  const int code_bits = hd->code_bits;
  const int NP = d / 2, NQ = d / 4;
  uint32_t *lut = (uint32_t *)(smem + a.lds_lut_off);
  uint2 *aq = (uint2 *)(smem + a.lds_aq_off);
  float *wq = smem + a.lds_w_off;

  // ---- prologue (scratch aliases the record area)
  {
    float *qraw = smem + a.lds_rec_off;  // [G][d]
    float *qt = qraw + G * d;            // [GP][d]
    const int64_t qbase = ((int64_t)b * a.n_q_heads + (int64_t)hkv * G) * d;
    for (int k = threadIdx.x; k < G * d; k += blockDim.x)
      qraw[k] = a.q_f32 ? ((const float *)a.q)[qbase + k]
                        : bf16_to_f32(((const uint16_t *)a.q)[qbase + k]);
    __syncthreads();
    const float *R = (const float *)(a.blob + hd->off_R);
    for (int k = threadIdx.x; k < GP * d; k += blockDim.x) {
      const int g = k / d, i = k % d;
      float acc = 0.0f;
      if (g < G) {
        const float *Ri = R + (size_t)i * d;
        const float *qg = qraw + g * d;
        for (int j = 0; j < d; ++j) acc = fmaf(Ri[j], qg[j], acc);
      }
      qt[g * d + i] = acc;
    }
    __syncthreads();
    if (m > 0) {
      const SQ_CONST float *S = cptr<float>(a.blob + hd->off_S);
      const float sc = hd->qjl_scale;
      for (int k = threadIdx.x; k < m * GP; k += blockDim.x) {
        const int j = k / GP, g = k % GP;
        float acc = 0.0f;
        for (int i = 0; i < d_eff; ++i) acc = fmaf(S[j * d_eff + i], qt[g * d + i], acc);
        wq[k] = sc * acc;
      }
    }
    for (int k = threadIdx.x; k < GR * (NP + NQ) * 4; k += blockDim.x) {
      const int mm = k & 3, rest = k >> 2;
      const int r = rest / (NP + NQ), e = rest % (NP + NQ);
      const float *qh = qt + (4 * r + mm) * d;
      uint2 v;
      if (e < NP) {
        v.x = bf16_pair(f32_to_bf16_rne(qh[2 * e]));
        v.y = bf16_pair(f32_to_bf16_rne(qh[2 * e + 1]));
      } else {
        uint16_t lo[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x = qh[4 * (e - NP) + t];
          lo[t] = f32_to_bf16_rne(x - bf16_to_f32(f32_to_bf16_rne(x)));
        }
        v.x = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
        v.y = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
      }
      aq[k] = v;
    }
    if constexpr (!LG) {
      const uint32_t *gl = (const uint32_t *)(a.blob + hd->off_lutp);
      for (int k = threadIdx.x; k < n_cent; k += blockDim.x) lut[k] = gl[k];
    }
    __syncthreads();
  }
  // centroid pairs: LDS copy, or (tables too large for LDS) the global table
  const uint32_t *lutv;
  if constexpr (LG) lutv = (const uint32_t *)(a.blob + hd->off_lutp);
  else lutv = lut;

  const uint32_t *slot = a.kpacked + (int64_t)b * a.ps_b + (int64_t)hkv * a.ps_h;
  uint32_t *rec = (uint32_t *)(smem + a.lds_rec_off) + wave * NT * a.rec_tile;
  const int tb = blockIdx.x * a.tiles_per_block;
  const int te = min(a.n_tiles, tb + a.tiles_per_block);
  const uint2 *aqm = aq + (lane & 3);

  for (int tp = tb + wave * NT; tp < te; tp += 4 * NT) {
    const int ntl = min(NT, te - tp);
    // ---- stage the records: direct global -> LDS loads (lane l's word lands
    // in column l of row w), all issued before the first wait; row W is zero
#pragma unroll
    for (int tq = 0; tq < NT; ++tq) {
      if (tq < ntl) {
        const uint32_t *src = slot + (int64_t)(tp + tq) * W * 64 + lane;
        uint32_t *dstr = rec + tq * a.rec_tile;
        for (int w = 0; w < W; ++w)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + w * 64),
                                           (__attribute__((address_space(3))) void *)(dstr + w * 64), 4, 0, 0);
        dstr[W * 64 + lane] = 0u;
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the staged words are in LDS
    f32x4 acc[NT][GR];
#pragma unroll
    for (int tq = 0; tq < NT; ++tq)
#pragma unroll
      for (int r = 0; r < GR; ++r) acc[tq][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    int cur = -1;
    uint32_t wlo[NT], whi[NT];
#pragma unroll
    for (int tq = 0; tq < NT; ++tq) wlo[tq] = whi[tq] = 0u;
    // coordinate descriptors, 16 at a time (one scalar load), next block prefetched
    const SQ_CONST uint32_t *dsc = cptr<uint32_t>(a.blob + hd->off_desc);
    uint32_t dnext[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) dnext[c] = dsc[c];
    for (int q16 = 0; q16 < d / 16; ++q16) {
      uint32_t dcur[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) dcur[c] = dnext[c];
      if (q16 + 1 < d / 16) {
#pragma unroll
        for (int c = 0; c < 16; ++c) dnext[c] = dsc[16 * (q16 + 1) + c];
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int qd = 4 * q16 + qq;
        uint32_t dv[4][NT];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t e = dcur[4 * qq + c];
          const int bo = e & 0xFFF, wd = (e >> 12) & 0xF, cb = e >> 16;
          if (wd == 0) {
#pragma unroll
            for (int tq = 0; tq < NT; ++tq) dv[c][tq] = 0u;
            continue;
          }
          const int w = bo >> 5;
          if (w != cur) {
#pragma unroll
            for (int tq = 0; tq < NT; ++tq) {
              wlo[tq] = rec[tq * a.rec_tile + w * 64 + lane];
              whi[tq] = rec[tq * a.rec_tile + (w + 1) * 64 + lane];
            }
            cur = w;
          }
          const uint32_t mask = (1u << wd) - 1u;
#pragma unroll
          for (int tq = 0; tq < NT; ++tq) {
            const uint32_t f = __builtin_amdgcn_alignbit(whi[tq], wlo[tq], bo & 31) & mask;
            dv[c][tq] = lutv[cb + f];
          }
        }
#pragma unroll
        for (int r = 0; r < GR; ++r) {
          const uint2 a0 = aqm[(r * (NP + NQ) + 2 * qd) * 4];
          const uint2 a1 = aqm[(r * (NP + NQ) + 2 * qd + 1) * 4];
          const uint2 ac = aqm[(r * (NP + NQ) + NP + qd) * 4];
#pragma unroll
          for (int tq = 0; tq < NT; ++tq) {
            acc[tq][r] = mfma4(a0, make_uint2(dv[0][tq], dv[1][tq]), acc[tq][r]);
            acc[tq][r] = mfma4(a1, make_uint2(dv[2][tq], dv[3][tq]), acc[tq][r]);
            const uint2 bh = make_uint2(__builtin_amdgcn_perm(dv[1][tq], dv[0][tq], 0x05040100u),
                                        __builtin_amdgcn_perm(dv[3][tq], dv[2][tq], 0x05040100u));
            acc[tq][r] = mfma4(ac, bh, acc[tq][r]);
          }
        }
      }
    }
    // ---- QJL term and stores
#pragma unroll
    for (int tq = 0; tq < NT; ++tq) {
      if (tq >= ntl) continue;
      const uint32_t *rr = rec + tq * a.rec_tile + lane;
      float qa[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) qa[g] = 0.0f;
      float gm = 0.0f;
      if (m > 0) {
        for (int j = 0; j < m; ++j) {
          const int pos = code_bits + j;
          const float sgn = ((rr[(pos >> 5) * 64] >> (pos & 31)) & 1u) ? 1.0f : -1.0f;
#pragma unroll
          for (int g = 0; g < GP; g += 4) {
            const float4 wv = *(const float4 *)(wq + j * GP + g);
            qa[g] = fmaf(sgn, wv.x, qa[g]);
            qa[g + 1] = fmaf(sgn, wv.y, qa[g + 1]);
            qa[g + 2] = fmaf(sgn, wv.z, qa[g + 2]);
            qa[g + 3] = fmaf(sgn, wv.w, qa[g + 3]);
          }
        }
        gm = half_bits_to_f32(rr[(W - 1) * 64] >> 16);
      }
      const int64_t t = (int64_t)(tp + tq) * 64 + lane;
      if (t < a.n_tokens) {
#pragma unroll
        for (int r = 0; r < GR; ++r)
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            const int g = 4 * r + mm;
            if (g < G)
              a.scores[((int64_t)b * a.n_q_heads + (int64_t)hkv * G + g) * a.n_tokens + t] =
                  fmaf(gm, qa[g], acc[tq][r][mm]);
          }
      }
    }
  }
}

// ------------------------------------------------------------------ attend
//
// Split-T softmax-weighted value sum in the rotated value space.  Kernel 1:
// one wave per (batch, KV head, chunk of ATT_CHUNK tokens, block of 64
// eigen-coordinates), lane = coordinate.  Per 64-token tile the record words
// its coordinates touch are staged straight from HBM into LDS (word-major,
// row stride ATT_RS, so lanes reading different words of one token hit
// different banks); the query group's scores give an online softmax (running
// max, rescaled sums) whose weights p are kept in LDS as bf16 hi/lo pairs.
// Each lane decodes its coordinate for 4 tokens at a time into C_v[code] as
// bf16 hi/lo pairs and v_mfma_f32_4x4x4_16b_bf16 forms sum_t p_t C_v[code_t]:
// in block b, lane 4b+n supplies the 4 tokens of coordinate 4b+n (B operand),
// lane 4b+m the weights of query head m (A operand), and the accumulator of
// lane 4b+n holds head m in register m.  Three products (hi*hi + hi*lo +
// lo*hi) give each term to ~2^-16 relative.  Kernel 2: one workgroup per
// (batch, query head) combines the chunks in order (no atomics,
// deterministic) and un-rotates once: o = R_v^T o_rot / L.

static constexpr int ATT_CHUNK = 1024;
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
  int n_chunks, n_parts;
  int lds_wave_off;            // floats: per-wave areas (the centroid table starts at 0)
  int wave_floats;             // one wave's area: two staging buffers, then the weights
  int buf_floats;              // one staging buffer: [nwd][ATT_RS] words + [G][64] scores
};

// Maximum over the 64 lanes: rotations within each row of 16 (DPP), then the
// four row results (returned in every lane).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Centroid table placement of the attend kernel: LM_COL = one column per lane
// (entry code * 64 + lane: every lane reads its own bank; widths <= 6),
// LM_PACK = the block's tables back to back with one pad entry each, LM_GLB =
// read from the table blob (tables too large for LDS).
enum { LM_COL = 0, LM_PACK = 1, LM_GLB = 2 };

template <int G, int LM>
__global__ __launch_bounds__(256) void attend_partial_kernel(AttendArgs a) {
  extern __shared__ float smem[];
  constexpr int GR = (G + 3) / 4, GP = 4 * GR;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // a workgroup = 4 consecutive chunks of one (batch, KV head, coordinate block)
  const int cgrp = blockIdx.x / a.n_parts, part = blockIdx.x % a.n_parts;
  const int chunk = cgrp * 4 + wv;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int ch = a.first_head + b * a.cbs + hkv;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d, W = hd->W;
  const SQ_CONST DevCoord *coords = cptr<DevCoord>(a.blob + hd->off_coord);
  const int c0 = part * 64, c1 = min(d, c0 + 64);
  const int ci = c0 + lane;
  // the block's record words [wlo, whi] and centroid pairs [lut0, lut1)
  const int wlo = coords[c0].bit_off >> 5;
  const int whi = min(W - 1, (coords[c1 - 1].bit_off + coords[c1 - 1].width) >> 5);
  const int nwd = whi - wlo + 2;  // one spare row: the word after a field never goes past it
  const int lut0 = coords[c0].cent_base;
  uint32_t *lut = (uint32_t *)smem;
  float *stage = smem + a.lds_wave_off + wv * a.wave_floats;  // two buffers: words, then scores
  uint32_t *ph = (uint32_t *)(stage + 2 * a.buf_floats);      // [GP][ATT_PS] bf16 hi of p, twice
  uint32_t *pl = ph + GP * ATT_PS;                             // [GP][ATT_PS] bf16 lo of p, twice
  const uint32_t *glut = (const uint32_t *)(a.blob + hd->off_lutp) + lut0;
  // this lane's field
  int width = 0, bo = 0, cb = 0;
  if (ci < c1) {
    width = coords[ci].width;
    bo = coords[ci].bit_off;
    cb = coords[ci].cent_base - lut0;
  }
  const int n = width ? (1 << width) : 0;
  if constexpr (LM == LM_COL) {
    // column lane: entry f at f * 64 + lane; a zero-width lane reads 0 at f = 0
    for (int k = wv; k < max(n, 1); k += 4) lut[k * 64 + lane] = n ? glut[cb + k] : 0u;
    cb = lane;
  } else if constexpr (LM == LM_PACK) {
    // coordinate c0 + j's table at offset cb + j: lanes gathering the same code
    // from tables of equal size fall in different banks; the slot after each
    // table is 0, which a zero-width coordinate (field 0) reads
    if (ci < c1) {  // lanes past the last coordinate (head_dim 32) write nothing
      for (int k = wv; k < n; k += 4) lut[cb + lane + k] = glut[cb + k];
      if (wv == 0) lut[cb + lane + n] = 0u;
    }
    cb += lane;
  }
  const uint32_t *lutv;
  if constexpr (LM == LM_GLB) lutv = glut;
  else lutv = lut;
  const int lsh = LM == LM_COL ? 6 : 0;  // gather index: (field << lsh) + cb
  const uint32_t fmask = width ? ((1u << width) - 1u) : 0u;
  const int cwl = width ? (bo >> 5) - wlo : 0, cs = bo & 31;
  const bool straddle = cs + width > 32;
  __syncthreads();
  if (chunk >= a.n_chunks) return;  // no barrier follows

  const int64_t tb = (int64_t)chunk * ATT_CHUNK;
  const int64_t te = min(a.n_tokens, tb + ATT_CHUNK);
  const float *srow = a.scores + ((int64_t)b * a.n_q_heads + (int64_t)hkv * G) * a.n_tokens;
  const uint32_t *slot = a.vpacked + (int64_t)b * a.ps_b + (int64_t)hkv * a.ps_h;
  float mrun[G], lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    lsum[g] = 0.0f;
  }
  // four independent accumulator sets (the products of a step alternate
  // among them), summed at the end
  f32x4 acc[4][GR];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int r = 0; r < GR; ++r) acc[h][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging, double-buffered: the words [wlo, wlo + nwd) of the tile's
  // records and its G score rows go straight from HBM to LDS; tile i + 1 is
  // requested before tile i is computed, so the one wait per tile covers
  // loads issued a whole tile earlier.
  auto stage_tile = [&](int64_t t0, int buf) {
    uint32_t *rw = (uint32_t *)(stage + buf * a.buf_floats);
    const uint32_t *src = slot + (t0 >> 6) * W * 64 + lane;
    for (int w = 0; w < nwd; ++w)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + min(wlo + w, W - 1) * 64),
                                       (__attribute__((address_space(3))) void *)(rw + w * ATT_RS), 4, 0, 0);
    float *sr = stage + buf * a.buf_floats + nwd * ATT_RS;
    // pad tokens of the last tile: any in-range address (their weight is 0)
    const int64_t ts = min(t0 + lane, a.n_tokens - 1);
#pragma unroll
    for (int g = 0; g < G; ++g)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(srow + (int64_t)g * a.n_tokens + ts),
                                       (__attribute__((address_space(3))) void *)(sr + g * 64), 4, 0, 0);
  };
  stage_tile(tb, 0);
  int buf = 0;
  for (int64_t t0 = tb; t0 < te; t0 += 64, buf ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this tile's staging has landed
    wave_lds_sync();
    if (t0 + 64 < te) stage_tile(t0 + 64, buf ^ 1);
    const uint32_t *rec = (const uint32_t *)(stage + buf * a.buf_floats);
    const float *sr = stage + buf * a.buf_floats + nwd * ATT_RS;
    const uint32_t *rlo = rec + cwl * ATT_RS, *rhi = rlo + ATT_RS;
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
        for (int h = 0; h < 4; ++h) acc[h][g >> 2][g & 3] *= corr;
      }
      const float pv = __expf(sv[g] - mrun[g]);  // 0 for tokens past the end
      lsum[g] += pv;
      const uint16_t hi = f32_to_bf16_rne(pv);
      ph[g * ATT_PS + lane] = bf16_pair(hi);
      pl[g * ATT_PS + lane] = bf16_pair(f32_to_bf16_rne(pv - bf16_to_f32(hi)));
    }
#pragma unroll
    for (int g = G; g < GP; ++g) {
      ph[g * ATT_PS + lane] = 0u;
      pl[g * ATT_PS + lane] = 0u;
    }
    wave_lds_sync();
    // ---- 8 tokens per step: decode (all gathers in flight together), then
    // the weighted sums on the MFMA.  A product takes 2 tokens: the k slots
    // of coordinate n are (hi, lo) of C[code] for each token, the weights of
    // head m are (p, p) per token, so it adds p_t0 (hi0 + lo0) + p_t1 (hi1 + lo1);
    // once with bf16(p) and once with the remainder of p.
    const int m = lane & 3;
#pragma unroll 2
    for (int k = 0; k < 64; k += 8) {
      const uint4 lo0 = *(const uint4 *)(rlo + k), lo1 = *(const uint4 *)(rlo + k + 4);
      uint4 hi0 = make_uint4(0, 0, 0, 0), hi1 = hi0;
      if (straddle) {  // only lanes whose field runs into the next word read it
        hi0 = *(const uint4 *)(rhi + k);
        hi1 = *(const uint4 *)(rhi + k + 4);
      }
      uint32_t pr[8];
      pr[0] = lutv[cb + ((__builtin_amdgcn_alignbit(hi0.x, lo0.x, cs) & fmask) << lsh)];
      pr[1] = lutv[cb + ((__builtin_amdgcn_alignbit(hi0.y, lo0.y, cs) & fmask) << lsh)];
      pr[2] = lutv[cb + ((__builtin_amdgcn_alignbit(hi0.z, lo0.z, cs) & fmask) << lsh)];
      pr[3] = lutv[cb + ((__builtin_amdgcn_alignbit(hi0.w, lo0.w, cs) & fmask) << lsh)];
      pr[4] = lutv[cb + ((__builtin_amdgcn_alignbit(hi1.x, lo1.x, cs) & fmask) << lsh)];
      pr[5] = lutv[cb + ((__builtin_amdgcn_alignbit(hi1.y, lo1.y, cs) & fmask) << lsh)];
      pr[6] = lutv[cb + ((__builtin_amdgcn_alignbit(hi1.z, lo1.z, cs) & fmask) << lsh)];
      pr[7] = lutv[cb + ((__builtin_amdgcn_alignbit(hi1.w, lo1.w, cs) & fmask) << lsh)];
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const uint32_t *hrow = ph + (4 * r + m) * ATT_PS + k, *lrow = pl + (4 * r + m) * ATT_PS + k;
        const uint4 ah0 = *(const uint4 *)hrow, ah1 = *(const uint4 *)(hrow + 4);
        const uint4 al0 = *(const uint4 *)lrow, al1 = *(const uint4 *)(lrow + 4);
        const uint2 ah[4] = {make_uint2(ah0.x, ah0.y), make_uint2(ah0.z, ah0.w),
                             make_uint2(ah1.x, ah1.y), make_uint2(ah1.z, ah1.w)};
        const uint2 al[4] = {make_uint2(al0.x, al0.y), make_uint2(al0.z, al0.w),
                             make_uint2(al1.x, al1.y), make_uint2(al1.z, al1.w)};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint2 bv = make_uint2(pr[2 * h], pr[2 * h + 1]);
          acc[h][r] = mfma4(ah[h], bv, acc[h][r]);
          acc[h][r] = mfma4(al[h], bv, acc[h][r]);
        }
      }
    }
    wave_lds_sync();  // every read of this tile's words and weights is done
  }
  // ---- partials: o_rot for this block's coordinates; the running max and
  // the weight sum (block 0)
  float *dst = a.ws + (((int64_t)b * a.n_q_heads + (int64_t)hkv * G) * a.n_chunks + chunk) * (d + 2);
  if (ci < c1) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      dst[(int64_t)g * a.n_chunks * (d + 2) + 2 + ci] =
          (acc[0][g >> 2][g & 3] + acc[1][g >> 2][g & 3]) + (acc[2][g >> 2][g & 3] + acc[3][g >> 2][g & 3]);
  }
  if (part == 0) {
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

extern "C" sq_status sq_compress(const sq_calib *c, int first_head, int n_heads, int batch,
                                 int calib_batch_stride, const void *x, sq_dtype dt,
                                 int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                                 int64_t xs_token, uint32_t *packed, int64_t ps_batch,
                                 int64_t ps_head, sq_stream stream) {
  const char *fn = "sq_compress";
  sq_status st = check_handle(c, fn);
  if (st != SQ_OK) return st;
  st = check_heads(c, first_head, n_heads, batch, calib_batch_stride, fn);
  if (st != SQ_OK) return st;
  if (n_tokens < 0) return fail(SQ_ERR_ARG, "sq_compress: n_tokens < 0");
  if (dt != SQ_F32 && dt != SQ_BF16) return fail(SQ_ERR_ARG, "sq_compress: bad dtype");
  if (n_tokens == 0 || batch == 0) { clear_error(); return SQ_OK; }
  if (!x || !packed) return fail(SQ_ERR_ARG, "sq_compress: NULL pointer");
  st = check_slots(c, n_tokens, n_heads, batch, ps_batch, ps_head, fn);
  if (st != SQ_OK) return st;
  const int esz = dt == SQ_F32 ? 4 : 2;
  if (((uintptr_t)x % 16) || (xs_token * esz) % 16 || (xs_head * esz) % 16 || (xs_batch * esz) % 16)
    return fail(SQ_ERR_ARG, "sq_compress: x and its strides must be 16-byte aligned");
  const int d = c->heads[first_head].d;
  if (xs_token < d) return fail(SQ_ERR_ARG, "sq_compress: xs_token < head_dim");
  if (n_tokens > ((int64_t)1 << 36)) return fail(SQ_ERR_UNSUPPORTED, "sq_compress: too many tokens");
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
    return fail(SQ_ERR_UNSUPPORTED, "sq_compress: calibration tables exceed the LDS of one workgroup");
  a.heads = c->dev_heads;
  a.blob = (const uint8_t *)c->dev_blob;
  a.x = x;
  a.packed = packed;
  a.xs_b = xs_batch; a.xs_h = xs_head; a.xs_t = xs_token;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.n_tokens = n_tokens;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_tiles = (int)((n_tokens + 63) / 64);
  const int gz = calib_batch_stride ? batch : 1;
  a.items = calib_batch_stride ? a.n_tiles : (int)std::min<int64_t>((int64_t)batch * a.n_tiles, INT32_MAX);
  // enough resident workgroups to keep every CU busy; each walks many tiles
  const int64_t want = (int64_t)device_cu_count() * (d >= 256 ? 1 : 2) * 2;
  int gx = (int)std::max<int64_t>(1, std::min<int64_t>(a.items, (want + (int64_t)n_heads * gz - 1) / ((int64_t)n_heads * gz)));
  dim3 grid(gx, n_heads, gz);
  if (grid.y > 65535 || grid.z > 65535) return fail(SQ_ERR_UNSUPPORTED, "sq_compress: too many heads or batch entries");
  hipStream_t s = (hipStream_t)stream;
  const bool f32 = dt == SQ_F32;
  switch (d) {
    case 32:  launch_compress_d<32>(f32, tg, grid, lds, s, a); break;
    case 64:  launch_compress_d<64>(f32, tg, grid, lds, s, a); break;
    case 128: launch_compress_d<128>(f32, tg, grid, lds, s, a); break;
    case 256: launch_compress_d<256>(f32, tg, grid, lds, s, a); break;
    default: return fail(SQ_ERR_UNSUPPORTED, "sq_compress: head_dim");
  }
  return launched(fn);
}

template <int G, int NT, bool LG>
static void launch_scores(dim3 grid, size_t lds, hipStream_t s, const ScoresArgs &a) {
  hipLaunchKernelGGL((scores_kernel<G, NT, LG>), grid, dim3(256), lds, s, a);
}

template <int G>
static void launch_scores_nt(int nt, bool lg, dim3 grid, size_t lds, hipStream_t s, const ScoresArgs &a) {
  if (lg) launch_scores<G, 4, true>(grid, lds, s, a);
  else if (nt == 4) launch_scores<G, 4, false>(grid, lds, s, a);
  else if (nt == 2) launch_scores<G, 2, false>(grid, lds, s, a);
  else launch_scores<G, 1, false>(grid, lds, s, a);
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
  int max_cent = 1, max_m = 0;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h) {
      const HeadCal &hc = kc->heads[first_head + bb * calib_batch_stride + h];
      max_cent = std::max(max_cent, hc.n_cent);
      max_m = std::max(max_m, hc.m);
    }
    if (calib_batch_stride == 0) break;
  }
  const int GR = (G + 3) / 4, GP = 4 * GR;
  ScoresArgs a{};
  const int limit = device_lds_limit();
  const int scratch = (G + GP) * d;                          // prologue floats
  int nt = 4;
  bool lg = false;
  // LDS: centroid pairs | MFMA A operands | QJL weights | record tiles
  auto layout = [&](bool lut_in_lds, int n) {
    a.lds_lut_off = 0;
    a.lds_aq_off = lut_in_lds ? ((max_cent + 3) & ~3) : 0;  // 16-byte aligned
    a.lds_w_off = a.lds_aq_off + 2 * GR * (d / 2 + d / 4) * 4;
    a.lds_rec_off = a.lds_w_off + ((std::max(1, max_m) * GP + 3) & ~3);
    a.rec_tile = (kc->W_max + 1) * 64;
    return (size_t)(a.lds_rec_off + std::max(scratch, 4 * n * a.rec_tile)) * 4;
  };
  size_t lds = layout(true, nt);
  while (nt > 1 && lds > (size_t)std::min(limit, 72 * 1024)) lds = layout(true, nt >>= 1);
  if (lds > (size_t)limit) {  // centroid table too large: read it from the L1/L2
    lg = true;
    nt = 4;
    lds = layout(false, nt);
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
  a.q_f32 = qdt == SQ_F32;
  a.n_tiles = (int)((n_tokens + 63) / 64);
  // workgroups: enough to fill the chip, each a multiple of one pass (4 waves x nt tiles)
  const int64_t pairs = (int64_t)batch * n_kv_heads;
  const int64_t want = (int64_t)device_cu_count() * 8;
  int blocks_t = (int)std::min<int64_t>((a.n_tiles + 4 * nt - 1) / (4 * nt),
                                        std::max<int64_t>(1, (want + pairs - 1) / pairs));
  a.tiles_per_block = (a.n_tiles + blocks_t - 1) / blocks_t;
  a.tiles_per_block = ((a.tiles_per_block + 4 * nt - 1) / (4 * nt)) * (4 * nt);
  blocks_t = (a.n_tiles + a.tiles_per_block - 1) / a.tiles_per_block;
  dim3 grid(blocks_t, n_kv_heads, batch);
  if (grid.z > 65535 || grid.y > 65535) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: grid too large");
  hipStream_t s = (hipStream_t)stream;
  switch (G) {
    case 1: launch_scores_nt<1>(nt, lg, grid, lds, s, a); break;
    case 2: launch_scores_nt<2>(nt, lg, grid, lds, s, a); break;
    case 3: launch_scores_nt<3>(nt, lg, grid, lds, s, a); break;
    case 4: launch_scores_nt<4>(nt, lg, grid, lds, s, a); break;
    case 5: launch_scores_nt<5>(nt, lg, grid, lds, s, a); break;
    case 6: launch_scores_nt<6>(nt, lg, grid, lds, s, a); break;
    case 7: launch_scores_nt<7>(nt, lg, grid, lds, s, a); break;
    case 8: launch_scores_nt<8>(nt, lg, grid, lds, s, a); break;
  }
  return launched(fn);
}

extern "C" size_t sq_attend_workspace_bytes(int batch, int n_q_heads, int64_t n_tokens, int head_dim) {
  if (batch <= 0 || n_q_heads <= 0 || n_tokens <= 0 || head_dim <= 0) return 0;
  const int64_t nch = (n_tokens + ATT_CHUNK - 1) / ATT_CHUNK;
  return (size_t)batch * n_q_heads * nch * (head_dim + 2) * sizeof(float);
}

template <int G>
static void launch_attend(int lm, dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a) {
  if (lm == LM_COL) hipLaunchKernelGGL((attend_partial_kernel<G, LM_COL>), grid, dim3(256), lds, s, a);
  else if (lm == LM_PACK) hipLaunchKernelGGL((attend_partial_kernel<G, LM_PACK>), grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((attend_partial_kernel<G, LM_GLB>), grid, dim3(256), lds, s, a);
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
  a.n_chunks = (int)((n_tokens + ATT_CHUNK - 1) / ATT_CHUNK);
  a.n_parts = (d + 63) / 64;
  // LDS: centroid table of one 64-coordinate block | 4 x (two staging buffers, weights)
  int max_lut = 1, max_nwd = 2, max_w = 0;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h) {
      const HeadCal &hc = vc->heads[first_head + bb * calib_batch_stride + h];
      for (int pt = 0; pt < a.n_parts; ++pt) {
        const int c0 = pt * 64, c1 = std::min(d, c0 + 64);
        const int lut1 = c1 < d ? hc.cent_base[c1] : hc.n_cent;
        max_lut = std::max(max_lut, lut1 - hc.cent_base[c0]);
        const int wlo = hc.bit_off[c0] >> 5;
        const int whi = std::min(hc.W - 1, (hc.bit_off[c1 - 1] + hc.widths[c1 - 1]) >> 5);
        max_nwd = std::max(max_nwd, whi - wlo + 2);
        for (int i = c0; i < c1; ++i) max_w = std::max(max_w, hc.widths[i]);
      }
    }
    if (calib_batch_stride == 0) break;
  }
  const int GP = ((G + 3) / 4) * 4;
  const int limit = device_lds_limit();
  a.buf_floats = max_nwd * ATT_RS + G * 64;
  a.wave_floats = 2 * a.buf_floats + 2 * GP * ATT_PS;
  auto lds_for = [&](int lut_floats) {
    a.lds_wave_off = (lut_floats + 3) & ~3;
    return (size_t)(a.lds_wave_off + 4 * a.wave_floats) * 4;
  };
  int lm = LM_GLB;
  size_t lds = 0;
  if (max_w <= 6 && lds_for(64 << max_w) <= (size_t)std::min(limit, 64 * 1024)) {
    lm = LM_COL;
    lds = lds_for(64 << max_w);
  } else if (lds_for(max_lut + 64) <= (size_t)std::min(limit, 64 * 1024)) {
    lm = LM_PACK;
    lds = lds_for(max_lut + 64);
  } else {
    lds = lds_for(0);
  }
  if (lds > (size_t)limit) return fail(SQ_ERR_UNSUPPORTED, "sq_attend: tables exceed LDS");
  const int64_t cgroups = (a.n_chunks + 3) / 4;
  dim3 grid((unsigned)(cgroups * a.n_parts), n_kv_heads, batch);
  if (grid.z > 65535 || grid.y > 65535 || cgroups * a.n_parts > INT32_MAX)
    return fail(SQ_ERR_UNSUPPORTED, "sq_attend: grid too large");
  switch (G) {
    case 1: launch_attend<1>(lm, grid, lds, s, a); break;
    case 2: launch_attend<2>(lm, grid, lds, s, a); break;
    case 3: launch_attend<3>(lm, grid, lds, s, a); break;
    case 4: launch_attend<4>(lm, grid, lds, s, a); break;
    case 5: launch_attend<5>(lm, grid, lds, s, a); break;
    case 6: launch_attend<6>(lm, grid, lds, s, a); break;
    case 7: launch_attend<7>(lm, grid, lds, s, a); break;
    case 8: launch_attend<8>(lm, grid, lds, s, a); break;
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
