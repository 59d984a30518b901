// Attend kernels shared by sq_attend (scores from device memory) and
// sq_decode (scores computed in the kernel from the packed keys).
#pragma once

#include "devcommon.h"

namespace sq {

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

// Tokens per chunk: the largest of 2048, 1024, ..., 128 that still gives
// batch x query heads x chunks >= 4096 partials (about two waves per CU or
// more; longer chunks mean fewer partials to combine and fewer table loads),
// else 64 (one tile: short caches are spread over as many waves as they
// have tiles).  A function of (batch, query heads, tokens) only, so the
// workspace size follows it.
static inline int64_t attend_chunk_tokens(int batch, int n_q_heads, int64_t n_tokens) {
  const int64_t bh = (int64_t)batch * n_q_heads;
  for (int64_t ct = 2048; ct >= 128; ct /= 2)
    if (bh * ((n_tokens + ct - 1) / ct) >= 4096) return ct;
  return 64;
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
  int g0, G_full;              // query heads g0 .. g0 + G - 1 of each KV head's group of G_full
  // sq_decode only: the keys' calibration and records and the queries
  const DevHead *kheads;
  const uint8_t *kblob;
  const uint32_t *kpacked;
  const void *q;
  int64_t kps_b, kps_h;
  int q_f32;
  int lds_ktab;                // bytes: the keys' score tables, [n_fent][GQ] floats
  PageArgs vpg, kpg;           // paged values / keys (table == nullptr: contiguous slots)
};

// How sq_attend launches for a given call (see plan_attend).
struct AttendPlan {
  AttendArgs a;        // everything but the data pointers, scale and workspace
  int lm = 0, np = 1, wpb = 4, max_width = 0;
  size_t lds = 0;
  dim3 grid;
};
sq_status plan_attend(const sq_calib *vc, int first_head, int calib_batch_stride, int batch, int n_q_heads,
                      int n_kv_heads, int64_t n_tokens, AttendPlan &P);

// How sq_decode launches for a given call (see plan_decode).
struct DecodePlan {
  AttendArgs a;        // everything but the data pointers, scale, workspace and g0
  int gsub = 4;        // query heads per launch (the last launch may take fewer)
  int launches = 1, lm = 0, np = 1, wpb = 4;
  size_t lds = 0;
  dim3 grid;
};
sq_status plan_decode(const sq_calib *kc, const sq_calib *vc, int first_head, int cbs, int batch, int n_q_heads,
                      int n_kv_heads, int64_t n_tokens, DecodePlan &P);


// Centroid table placement of the attend kernel: LM_COL = one column per lane
// (entry code * 64 + lane: every lane reads its own bank; widths <= 6),
// LM_PACK = a block's tables back to back with one pad entry each, LM_GLB =
// read from the table blob (tables too large for LDS).
enum { LM_COL = 0, LM_PACK = 1, LM_GLB = 2 };

// ---- scores inside the attend kernel (sq_decode)
//
// The keys' record fields are cut into groups of adjacent fields (FS layout in
// devtypes.h).  Per workgroup the query group's tables are built once in LDS:
// entry v of a code group holds, for each of the GQ query heads, the sum over
// the group's coordinates of q~_i C_i[field of i in v] (fp32, each product
// and sum rounded once); entry v of a QJL group holds sqrt(pi/2)/m sum_j w_j
// (2 v_j - 1) with w = S q~[0:d_eff].  A token's score is then the sum over
// groups of one table entry each, the QJL groups' sum scaled by gamma: the
// same value as sum_i q~_i C_i[code_i] + sqrt(pi/2)/m gamma sum_j w_j (2 z_j - 1)
// (SpectralQuant README "Overview": the query is rotated once and scored
// from the codes; QJL estimator, TurboQuant reference-implementation page,
// "Project Structure").
constexpr int DEC_KW = 32;  // record words of a key held in registers (lane = token)

// Build the score tables of query heads g0 .. g0 + G - 1 of KV head hkv (batch
// b) in LDS at byte offset a.lds_ktab of smem.  All waves of the workgroup
// take part; ends with a barrier.  scratch: at least G * (d + m) floats of LDS
// not otherwise in use yet.
template <int G, int GQ, int NT>
__device__ __forceinline__ void build_score_tables(const AttendArgs &a, int b, int hkv, int ch,
                                                   float *smem, float *scratch) {
  const SQ_CONST DevHead *kh = cptr<DevHead>(a.kheads) + ch;
  const int d = kh->d, km = kh->m, kd_eff = kh->d_eff, kW = kh->W, ng = kh->n_fgroups;
  float *qt = scratch;          // [G][d] rotated queries q~ = R q
  float *wq = scratch + G * d;  // [G][m] sqrt(pi/2)/m S q~[0:d_eff]
  const int64_t qbase = ((int64_t)b * a.n_q_heads + (int64_t)hkv * a.G_full + a.g0) * d;
  const float *RT = (const float *)(a.kblob + kh->off_RT);  // RT[j d + i] = R[i][j]
  for (int k = threadIdx.x; k < G * d; k += NT) {
    const int g = k / d, i = k - g * d;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < d; j0 += 8) {
      float r[8], qv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        r[u] = RT[(size_t)(j0 + u) * d + i];
        const int64_t qi = qbase + (int64_t)g * d + j0 + u;
        qv[u] = a.q_f32 ? ((const float *)a.q)[qi] : bf16_to_f32(((const uint16_t *)a.q)[qi]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u & 3] = fmaf(r[u], qv[u], acc[u & 3]);
    }
    qt[k] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  __syncthreads();
  if (km > 0) {
    const SQ_CONST float *S = cptr<float>(a.kblob + kh->off_S);
    for (int k = threadIdx.x; k < G * km; k += NT) {
      const int g = k / km, j = k - g * km;
      float acc = 0.0f;
      for (int i = 0; i < kd_eff; ++i) acc = fmaf(S[j * kd_eff + i], qt[g * d + i], acc);
      wq[k] = kh->qjl_scale * acc;
    }
    __syncthreads();
  }
  const SQ_CONST uint32_t *fs = cptr<uint32_t>(a.kblob + kh->off_fsched);
  const SQ_CONST DevCoord *kc = cptr<DevCoord>(a.kblob + kh->off_coord);
  const float *kcent = (const float *)(a.kblob + kh->off_cent);
  float *tab = smem + a.lds_ktab / 4;
  // one group per wave at a time, its entries over the wave's lanes
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int grp = wv; grp < ng; grp += NT / 64) {
    const uint32_t fw = fs[2 * grp], bw = fs[2 * grp + 1];
    const int width = (int)(fw & 15u);
    const bool qj = (fw >> 4) & 1u;
    const uint32_t e0 = fw >> 8;
    const int first = (int)(bw & 4095u), cnt = (int)((bw >> 12) & 255u);
    if (qj) {
      for (int k = lane; k < (GQ << width); k += 64) {
        const int v = k / GQ, g = k - v * GQ;
        float e = 0.0f;
        if (g < G)
          for (int c = 0; c < cnt; ++c) {
            const float w = wq[g * km + first + c];
            e += ((v >> c) & 1) ? w : -w;
          }
        tab[(size_t)(e0 + v) * GQ + g] = e;
      }
      continue;
    }
    // code group: a lane per entry v and every head at once; the centroids of
    // the group's first CMAX coordinates are loaded together (one load each
    // for all heads), then each head's sum runs over the coordinates in order
    constexpr int CMAX = 8;
    for (int v = lane; v < (1 << width); v += 64) {
      float cv[CMAX];
      int sh = 0;
#pragma unroll
      for (int c = 0; c < CMAX; ++c) {
        cv[c] = 0.0f;
        if (c < cnt) {
          const DevCoord cd = load_coord(kc + first + c);
          if (cd.width) {
            cv[c] = kcent[cd.cent_base + ((v >> sh) & ((1 << cd.width) - 1))];
            sh += cd.width;
          }
        }
      }
      float e[GQ];
#pragma unroll
      for (int g = 0; g < GQ; ++g) e[g] = 0.0f;
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < cnt && kc[first + c].width)
#pragma unroll
          for (int g = 0; g < G; ++g) e[g] = fmaf(qt[g * d + first + c], cv[c], e[g]);
      for (int c = CMAX; c < cnt; ++c) {  // (longer groups: zero-width coordinates among the fields)
        const DevCoord cd = load_coord(kc + first + c);
        if (cd.width) {
          const float x = kcent[cd.cent_base + ((v >> sh) & ((1 << cd.width) - 1))];
          sh += cd.width;
#pragma unroll
          for (int g = 0; g < G; ++g) e[g] = fmaf(qt[g * d + first + c], x, e[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GQ; ++g) tab[(size_t)(e0 + v) * GQ + g] = e[g];
    }
  }
  if (threadIdx.x < GQ) tab[(size_t)kh->n_fent * GQ + threadIdx.x] = 0.0f;  // the zero entry of unused slots
  __syncthreads();
}

// NP = 64-coordinate blocks per head (head_dim / 64, at least 1): one wave
// serves every block of its chunk, so the chunk's scores are read and its
// softmax computed once.
// WPB = waves (chunks) per workgroup, sharing the centroid tables; NBUF =
// staging buffers per wave.  Column tables: 16 single-buffered waves (four
// per SIMD) when the LDS allows, else 8 double-buffered; otherwise 4.
// FUSED (sq_decode): the scores of each tile are computed here from the
// packed keys (lane = token, the key record in registers) instead of being
// read from device memory; G <= 4 query heads per launch.
// FM: 0 sq_attend (scores from device memory), 1 sq_decode (scores built from
// the key records), 2 sq_decode over paged key and value pools
template <int G, int LM, int NP, int WPB, int NBUF = 2, int FM = 0>
__global__ __launch_bounds__(64 * WPB) void attend_partial_kernel(AttendArgs a) {
  constexpr bool FUSED = FM != 0, PAGED = FM == 2;
  extern __shared__ float smem[];
  constexpr int GR = (G + 3) / 4, GP = 4 * GR;
  constexpr int GQ = G == 3 ? 4 : G;  // floats per score-table entry
  static_assert(!FUSED || G <= 4, "sq_decode serves at most 4 query heads per launch");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // a workgroup = WPB consecutive chunks of one (batch, KV head)
  const int chunk = blockIdx.x * WPB + wv;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int ch = a.first_head + b * a.cbs + hkv;
  const SQ_CONST DevHead *hd = cptr<DevHead>(a.heads) + ch;
  const int d = hd->d, W = hd->W;
  const bool vnorm = hd->normalized != 0;
  const int vm = hd->m;
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
  // sq_decode: the score tables of this KV head's query group
  int kW = 0, km = 0, knq = 0, knorm = 0;
  const SQ_CONST uint32_t *kslots = nullptr, *kqslots = nullptr, *kscnt = nullptr;
  const uint32_t *kslot = nullptr;
  if constexpr (FUSED) {
    build_score_tables<G, GQ, 64 * WPB>(a, b, hkv, ch, smem, smem + a.lds_wave_off);
    const SQ_CONST DevHead *kh = cptr<DevHead>(a.kheads) + ch;
    kW = kh->W;
    km = kh->m;
    knq = kh->n_fqjl;
    knorm = kh->normalized;
    const int ng = kh->n_fgroups;
    constexpr int E = GQ == 4 ? 4 : GQ == 2 ? 3 : 2;  // log2 of an entry's bytes
    const SQ_CONST uint32_t *fs = cptr<uint32_t>(a.kblob + kh->off_fsched);
    kqslots = fs + 2 * ng;
    const SQ_CONST uint32_t *sbase = fs + ((2 * ng + knq + 15) & ~15);
    kslots = sbase + (size_t)(E - 2) * (kW + 1) * FS_SLOTS * 2;
    kscnt = sbase + (size_t)3 * (kW + 1) * FS_SLOTS * 2 + (size_t)(E - 2) * (kW + 1);
    kslot = PAGED ? a.kpacked : a.kpacked + (int64_t)b * a.kps_b + (int64_t)hkv * a.kps_h;
  }
  __syncthreads();
  if (chunk >= a.n_chunks) return;  // no barrier follows

  const int64_t tb = (int64_t)chunk * a.chunk_tokens;
  const int64_t te = min(a.n_tokens, tb + a.chunk_tokens);
  const float *srow = FUSED ? nullptr : a.scores + ((int64_t)b * a.n_q_heads + (int64_t)hkv * a.G_full + a.g0) * a.n_tokens;
  const uint32_t *slot = PAGED ? a.vpacked : a.vpacked + (int64_t)b * a.ps_b + (int64_t)hkv * a.ps_h;
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
    const uint32_t *src = (PAGED ? page_tile(a.vpg, slot, b, hkv, t0 >> 6, W) : slot + (t0 >> 6) * W * 64) + lane;
    for (int w = 0; w <= W; ++w)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + min(w, W - 1) * 64),
                                       (__attribute__((address_space(3))) void *)(rw + w * ATT_RS), 4, 0, 0);
    if constexpr (!FUSED) {
      float *sr = stage + buf * a.buf_floats + (W + 2) * ATT_RS;
      // pad tokens of the last tile: any in-range address (their weight is 0)
      const int64_t ts = min(t0 + lane, a.n_tokens - 1);
#pragma unroll
      for (int g = 0; g < G; ++g)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(srow + (int64_t)g * a.n_tokens + ts),
                                         (__attribute__((address_space(3))) void *)(sr + g * 64), 4, 0, 0);
    }
  };
  // sq_decode: the key record of this lane's token, word k in kw[k + 1]
  // (kw[0] = 0 is the word before the record); the words qb, qb + 1 holding
  // the QJL bits again in qlo, qhi and the last word (gamma, the norm) in
  // wlast; pad tokens of the last tile hold all-zero records
  uint32_t kw[FUSED ? DEC_KW + 2 : 1];
  uint32_t qlo = 0u, qhi = 0u, wlast = 0u;
  auto load_keys = [&](int64_t t0) {
    if constexpr (FUSED) {
      const uint32_t *src =
          (PAGED ? page_tile(a.kpg, kslot, b, hkv, t0 >> 6, kW) : kslot + (t0 >> 6) * (int64_t)kW * 64) + lane;
      kw[0] = 0u;
#pragma unroll
      for (int k = 0; k < DEC_KW; ++k) kw[k + 1] = k < kW ? src[k * 64] : 0u;
      kw[DEC_KW + 1] = 0u;
      if (km > 0 || knorm) wlast = src[(kW - 1) * 64];
      if (km > 0) {
        const int qb = kW - 2 - knorm;
        qhi = qb + 1 >= 0 ? src[(qb + 1) * 64] : 0u;
        qlo = qb >= 0 ? src[qb * 64] : 0u;
      }
    }
  };
  // row 0 of both staging buffers: zeros (the word before word 0)
  ((uint32_t *)stage)[lane] = 0u;
  if constexpr (NBUF == 2) ((uint32_t *)(stage + a.buf_floats))[lane] = 0u;
  if constexpr (NBUF == 2) stage_tile(tb, 0);
  int buf = 0;
  for (int64_t t0 = tb; t0 < te; t0 += 64, buf ^= NBUF - 1) {
    if constexpr (NBUF == 1) stage_tile(t0, 0);  // (the last sync of the previous tile ended its reads)
    load_keys(t0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this tile's staging has landed
    wave_lds_sync();
    if constexpr (NBUF == 2)
      if (t0 + 64 < te) stage_tile(t0 + 64, buf ^ 1);
    const uint32_t *rec = (const uint32_t *)(stage + buf * a.buf_floats);
    const float *sr = stage + buf * a.buf_floats + (W + 2) * ATT_RS;
    // ---- online softmax over the tile (lane = token)
    const int64_t t = t0 + lane;
    float sv[G];
    if constexpr (FUSED) {
      // the tile's scores: per window j (record words j - 1, j), FS_SLOTS
      // table reads, all issued before they are summed; then the QJL groups
      // from the last two words, scaled by gamma
      float s4[GQ], q4[GQ];
#pragma unroll
      for (int g = 0; g < GQ; ++g) s4[g] = q4[g] = 0.0f;
      typedef const __attribute__((address_space(3))) float lds_f32;
      typedef const __attribute__((address_space(3))) f32x2_t lds_f2;
      typedef const __attribute__((address_space(3))) f32x4 lds_f4;
      auto entry = [&](uint32_t ad, float *e) __attribute__((always_inline)) {
        if constexpr (GQ == 4) {
          const f32x4 v = *(lds_f4 *)(uintptr_t)ad;
          e[0] = v[0]; e[1] = v[1]; e[2] = v[2]; e[3] = v[3];
        } else if constexpr (GQ == 2) {
          const f32x2_t v = *(lds_f2 *)(uintptr_t)ad;
          e[0] = v[0]; e[1] = v[1];
        } else {
          e[0] = *(lds_f32 *)(uintptr_t)ad;
        }
      };
#pragma unroll
      for (int j = 0; j <= DEC_KW; ++j) {
        if (j <= kW) {
          // every slot of the window: its slot words in one scalar load before
          // the first table read (a scalar load waited for between two table
          // reads would also wait for every table read in flight); unused
          // slots read the zero entry
          const SQ_CONST uint32_t *sl = kslots + j * FS_SLOTS * 2;
          float e[FS_SLOTS][GQ];
#pragma unroll
          for (int u = 0; u < FS_SLOTS; ++u) {
            const uint32_t d0 = sl[2 * u], d1 = sl[2 * u + 1];
            const uint32_t win = __builtin_amdgcn_alignbit(kw[j + 1], kw[j], d0);  // (shift = d0 mod 32)
            entry((win & d1) | ((d0 >> 5) + (uint32_t)a.lds_ktab), e[u]);
          }
#pragma unroll
          for (int u = 0; u < FS_SLOTS; ++u)
#pragma unroll
            for (int g = 0; g < GQ; ++g) s4[g] += e[u][g];
        }
      }
      float gm = 0.0f;
      if (km > 0) {
        constexpr int E = GQ == 4 ? 4 : GQ == 2 ? 3 : 2;
        for (int u = 0; u < knq; ++u) {
          const uint32_t qd = kqslots[u];
          const uint32_t f = (uint32_t)((((uint64_t)qhi << 32) | qlo) >> (qd & 255u)) & ((1u << ((qd >> 8) & 15u)) - 1u);
          float e[GQ];
          entry(((qd >> 12) << E) + (f << E) + (uint32_t)a.lds_ktab, e);
#pragma unroll
          for (int g = 0; g < GQ; ++g) q4[g] += e[g];
        }
        gm = half_bits_to_f32(wlast >> 16);  // gamma: top half of the last word
      }
      // normalised keys: the score is nu times the unit vector's
      const float knu = knorm ? half_bits_to_f32(km > 0 ? (wlast & 0xFFFFu) : (wlast >> 16)) : 1.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) sv[g] = t < te ? a.scale * (knu * fmaf(gm, q4[g], s4[g])) : -INFINITY;
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) sv[g] = t < te ? a.scale * sr[g * 64 + lane] : -INFINITY;
    }
    // normalised values: the token's value is nu_t times its unit-vector
    // reconstruction, so its weight in the sum (not in the normaliser) is p nu
    float vnu = 1.0f;
    if (vnorm) {
      const uint32_t wl = rec[W * ATT_RS + lane];  // staged row W = word W - 1
      vnu = half_bits_to_f32(vm > 0 ? (wl & 0xFFFFu) : (wl >> 16));
    }
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
      const float pw = pv * vnu;  // the value's norm (normalised values), else 1
      const uint32_t hp = bf16_pair_rne(pw);
      ph[g * ATT_PS + lane] = hp;
      pl[g * ATT_PS + lane] = bf16_pair_rne(pw - __uint_as_float(hp << 16));
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
  float *dst = a.ws + (((int64_t)b * a.n_q_heads + (int64_t)hkv * a.G_full + a.g0) * a.n_chunks + chunk) * (d + 2);
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

// Ordered combine of the chunks' partials and the un-rotation, one workgroup
// per (batch, query head) (attend.hip); enqueued by launch_attend_combine.
void launch_attend_combine(const AttendArgs &a, int batch, int d, hipStream_t s);


}  // namespace sq
