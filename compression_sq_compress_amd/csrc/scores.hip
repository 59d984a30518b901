// sq_scores: q.k scores read straight from the packed keys (gfx950).

#include "devcommon.h"

namespace sq {

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
// super-step later by the wave that owns the query head's row, which adds
// the QJL term too (gamma times one or two reads of per-query tables over the
// sign-bit patterns, built in the prologue; sketches longer than 16 rows are
// summed bit by bit into a wave's partial instead).

constexpr int SC_WAVES = 8;    // consumer waves per workgroup
constexpr int SC_LOADERS = 3;  // waves issuing the record loads
constexpr int SC_BLOCK = 64 * (SC_WAVES + SC_LOADERS);
// quads held in registers per consumer wave (4 or 8 query heads per MFMA row set)
__host__ __device__ constexpr int sc_qmax(int gr) { return gr == 1 ? 9 : 5; }
// QJL term by table lookup for sketches of at most SC_QTAB_MAX_M rows: the
// sign bits split into a chunk of the first min(m, 8) bits and one of the
// rest, and each chunk gets a table over its bit patterns holding, per query
// row, sum_j w_j (2 z_j - 1) over the chunk's rows.  Entries of both chunks:
constexpr int SC_QTAB_MAX_M = 16;
__host__ __device__ constexpr int sc_qtab_entries(int m) {
  return m <= 0 || m > SC_QTAB_MAX_M ? 0 : (1 << (m < 8 ? m : 8)) + (m > 8 ? (1 << (m - 8)) : 0);
}

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
  int lds_lut, lds_qt, lds_wq, lds_qtab, lds_slot, lds_pbuf;  // byte offsets
};

// How sq_scores launches for a given call (see plan_scores).
struct ScorePlan {
  ScoresArgs a;       // everything but the data pointers, dtype flags and pass
  int passes = 0, max_quads = 0, slotb = 0, GR = 1;
  bool lg = false;    // joint tables read through the caches instead of LDS
  size_t lds = 0;
  dim3 grid;
};
sq_status plan_scores(const sq_calib *kc, int first_head, int calib_batch_stride, int batch, int n_q_heads,
                      int n_kv_heads, int64_t n_tokens, ScorePlan &P);



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
  const bool knorm = hd->normalized != 0;  // (read once: the loop's barriers keep loads in place)
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
  // QJL tables [entry][GP] (chunk 0's 2^min(m,8) entries, then chunk 1's)
  const bool qtab = m > 0 && m <= SC_QTAB_MAX_M;
  const int qn0 = 1 << min(m, 8);
  const float *qtb = (const float *)(sm + a.lds_qtab);
  if (qtab) {
    if (consumer) {
      float *qo = (float *)(sm + a.lds_qtab);
      const int ne = sc_qtab_entries(m);
      for (int k = ct; k < ne * GP; k += 64 * SC_WAVES) {
        const int e = k / GP, g = k - e * GP;
        const bool c1 = e >= qn0;
        const int z = c1 ? e - qn0 : e, j0 = c1 ? 8 : 0, nb = c1 ? m - 8 : min(m, 8);
        float acc = 0.0f;
        for (int j = 0; j < nb; ++j) {
          const float wv = wq[(j0 + j) * GP + g];
          acc += ((z >> j) & 1) ? wv : -wv;
        }
        qo[k] = acc;
      }
    }
    __syncthreads();
  }
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
  // QJL term: the wave that sums the partials of query head (row) r =
  // kk + j KS adds it for that row, so that every row gets it exactly once:
  // from the tables (qv, carried to the reduction one super-step later), or
  // for longer sketches bit by bit into the wave's own partial sum
  const bool qjl = m > 0 && a.pass == 0 && kk < min(G, GP);
  const bool qjl_tab = qjl && qtab;
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
      hlut[2 * qi + hh] = to_vgpr((LG ? 0u : (uint32_t)a.lds_lut) + e[2 + hh] * 8u);
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

  // QJL terms of the rows this wave sums, per tile of the super-step
  float qv[NS][GP];
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int j = 0; j < GP; ++j) qv[t][j] = 0.0f;
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
        if (qjl_tab) v += qv[t][row0 / K];
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
      if (qjl_tab) {  // gamma * sum_j w_j (2 z_j - 1) per row (w scaled by sqrt(pi/2)/m), times nu if normalised
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const uint32_t tl = tile_lds + (u * NS + t) * SLOTB;
          const uint32_t wl = *(const uint32_t *)(sm + tl + (W - 1) * 256u);
          float gm = half_bits_to_f32(wl >> 16);
          if (knorm) gm *= half_bits_to_f32(wl & 0xFFFFu);
          const uint32_t ad = tl + (code_bits >> 5) * 256u;
          const uint32_t z = __builtin_amdgcn_alignbit(*(const uint32_t *)(sm + ad + 256),
                                                       *(const uint32_t *)(sm + ad), zsh);
          const float *t0 = qtb + (z & (uint32_t)(qn0 - 1)) * GP;
          const float *t1 = qtb + (qn0 + ((z >> 8) & ((1u << max(m - 8, 0)) - 1u))) * GP;  // used when m > 8 (qn0 = 256)
#pragma unroll
          for (int j = 0; j < GP; ++j) {
            const int row = kk + j * KS;
            if (row < min(G, GP)) {
              float v = t0[row];
              if (m > 8) v += t1[row];
              qv[t][j] = gm * v;
            }
          }
        }
      } else if (qjl) {  // longer sketches: + gamma * sum_j w_j (2 z_j - 1) into this wave's partial
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const uint32_t tl = tile_lds + (u * NS + t) * SLOTB;
          const float gm = half_bits_to_f32(*(const uint32_t *)(sm + tl + (W - 1) * 256u) >> 16);
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
      if (knorm) {  // normalised keys: s = nu * (...), each partial scaled (linear)
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const uint32_t tl = tile_lds + (u * NS + t) * SLOTB;
          const uint32_t wl = *(const uint32_t *)(sm + tl + (W - 1) * 256u);
          const float nu = half_bits_to_f32(m > 0 ? (wl & 0xFFFFu) : (wl >> 16));
#pragma unroll
          for (int g = 0; g < GR; ++g)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[t][g][rr] *= nu;
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

}  // namespace sq

using namespace sq;

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

// Launch plan of sq_scores for a set of heads: wave groups over the quads,
// passes over them, ring slots, LDS layout and grid (every field of the
// kernel arguments except the data pointers and the pass index).
namespace sq {
sq_status plan_scores(const sq_calib *kc, int first_head, int calib_batch_stride, int batch, int n_q_heads,
                      int n_kv_heads, int64_t n_tokens, ScorePlan &P) {
  const int G = n_q_heads / n_kv_heads;
  const int d = kc->heads[first_head].d;
  int max_q = 1, max_plut = 1, max_m = 0, max_W = 1, max_qe = 0;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h) {
      const DevHead &D = kc->host_desc[first_head + bb * calib_batch_stride + h];
      if (D.d != d) return fail(SQ_ERR_ARG, "sq_scores: heads of one call must share head_dim");
      max_q = std::max(max_q, D.n_quads);
      max_plut = std::max(max_plut, D.n_plut);
      max_m = std::max(max_m, D.m);
      max_qe = std::max(max_qe, sc_qtab_entries(D.m));
      max_W = std::max(max_W, D.W);
    }
    if (calib_batch_stride == 0) break;
  }
  const int GR = (G + 3) / 4, GP = 4 * GR, QM = sc_qmax(GR);
  int ks = 1;
  while (ks < SC_WAVES && ((max_q + ks - 1) / ks > QM || (SC_WAVES / ks) * max_W * 256 + 256 > 16384)) ks *= 2;
  const int ts = SC_WAVES / ks;
  P.passes = (max_q + ks * QM - 1) / (ks * QM);
  P.max_quads = max_q;
  const int need = ts * max_W * 256 + 256;  // a stream tile may read one row past its end
  if (need <= 8192) P.slotb = 8192;
  else if (need <= 16384) P.slotb = 16384;
  else return fail(SQ_ERR_UNSUPPORTED, "sq_scores: records too long");
  const int R = P.slotb == 8192 ? 6 : 3;  // ring slots (kernel template)
  ScoresArgs &a = P.a;
  a = ScoresArgs{};
  const int limit = device_lds_limit();
  auto layout = [&](bool lut_in_lds) {
    size_t off = 0;
    a.lds_lut = 0;
    off = lut_in_lds ? (((size_t)max_plut * 8 + 1023) & ~(size_t)1023) : 0;  // copied in 1 KB pieces
    a.lds_qt = (int)off;   off += (size_t)G * d * 4;
    off = (off + 15) & ~(size_t)15;
    a.lds_wq = (int)off;   off += (size_t)std::max(1, max_m) * GP * 4;
    a.lds_qtab = (int)off; off += (size_t)max_qe * GP * 4;
    off = (off + 1023) & ~(size_t)1023;
    a.lds_slot = (int)off; off += (size_t)R * P.slotb;
    a.lds_pbuf = (int)off; off += (size_t)2 * (P.slotb == 8192 ? 2 : 1) * SC_WAVES * GP * 64 * 4;  // parity x slots per barrier
    return off;
  };
  P.lg = false;
  P.lds = layout(true);
  const bool lds0 = GR == 1 ? scores_lds0_ok<1>(P.slotb) : scores_lds0_ok<2>(P.slotb);
  if (P.lds > (size_t)limit || !lds0) {  // joint tables too large for LDS: read them through the caches
    P.lg = true;
    P.lds = layout(false);
  }
  if (P.lds > (size_t)limit) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: tables exceed LDS");
  P.GR = GR;
  a.heads = kc->dev_heads;
  a.blob = (const uint8_t *)kc->dev_blob;
  a.n_tokens = n_tokens;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.G = G;
  a.ks = ks;
  a.ts = ts;
  a.n_tiles = (int)((n_tokens + 63) / 64);
  // one workgroup per CU at a time: about two per CU over the launch
  const int64_t pairs = (int64_t)batch * n_kv_heads;
  const int64_t want = (int64_t)device_cu_count() * 2;
  const int64_t steps = (a.n_tiles + ts - 1) / ts;
  int64_t chunks = std::max<int64_t>(1, std::min<int64_t>(steps, (want + pairs - 1) / pairs));
  a.tiles_per_wg = (int)(((steps + chunks - 1) / chunks) * ts);
  chunks = (a.n_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  P.grid = dim3((unsigned)chunks, n_kv_heads, batch);
  if (P.grid.z > 65535 || P.grid.y > 65535) return fail(SQ_ERR_UNSUPPORTED, "sq_scores: grid too large");
  return SQ_OK;
}
}  // namespace sq

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
  ScorePlan P;
  st = plan_scores(kc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens, P);
  if (st != SQ_OK) return st;
  ScoresArgs a = P.a;
  a.q = q;
  a.kpacked = kpacked;
  a.scores = scores;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.q_f32 = qdt == SQ_F32;
  a.dma16 = ((uintptr_t)kpacked % 16 == 0) && ps_batch % 4 == 0 && ps_head % 4 == 0;
  hipStream_t s = (hipStream_t)stream;
  for (int p = 0; p < P.passes; ++p) {
    a.pass = p;
    if (P.GR == 1) {
      if (P.lg) launch_scores_slot<1, true>(P.slotb, P.grid, P.lds, s, a);
      else launch_scores_slot<1, false>(P.slotb, P.grid, P.lds, s, a);
    } else {
      if (P.lg) launch_scores_slot<2, true>(P.slotb, P.grid, P.lds, s, a);
      else launch_scores_slot<2, false>(P.slotb, P.grid, P.lds, s, a);
    }
  }
  return launched(fn);
}

namespace sq {
sq_status score_plan_summary(const sq_calib *kc, int first_head, int calib_batch_stride, int batch,
                             int n_q_heads, int n_kv_heads, int64_t n_tokens, int *passes, int *max_quads,
                             int *wave_groups) {
  ScorePlan P;
  sq_status st = plan_scores(kc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens, P);
  if (st != SQ_OK) return st;
  *passes = P.passes;
  *max_quads = P.max_quads;
  *wave_groups = P.a.ks;
  return SQ_OK;
}
}  // namespace sq
