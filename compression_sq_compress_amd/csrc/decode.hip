// sq_decode: the fused decode step -- scores, online softmax and the value sum
// in one pass over the packed keys and values, with no score tensor in device
// memory (gfx950).

#include "attend_kernel.h"

using namespace sq;

namespace sq {
// defined, per instance, in the decode_g*.hip units
template <int G, int FM>
bool dispatch_g(bool run, int lm, int np, int wpb, dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a);
}  // namespace sq

namespace {

template <int FM>
bool dispatch_fm(bool run, int gsub, int lm, int np, int wpb, dim3 grid, size_t lds, hipStream_t s,
                 const AttendArgs &a) {
  switch (gsub) {
    case 1: return dispatch_g<1, FM>(run, lm, np, wpb, grid, lds, s, a);
    case 2: return dispatch_g<2, FM>(run, lm, np, wpb, grid, lds, s, a);
    case 3: return dispatch_g<3, FM>(run, lm, np, wpb, grid, lds, s, a);
    default: return dispatch_g<4, FM>(run, lm, np, wpb, grid, lds, s, a);
  }
}

// run == false: only report whether that kernel exists without scratch;
// paged: the instance reading paged key and value pools
bool dispatch(bool run, int gsub, int lm, int np, int wpb, dim3 grid, size_t lds, hipStream_t s,
              const AttendArgs &a, bool paged = false) {
  return paged ? dispatch_fm<2>(run, gsub, lm, np, wpb, grid, lds, s, a)
               : dispatch_fm<1>(run, gsub, lm, np, wpb, grid, lds, s, a);
}

}  // namespace

namespace sq {

// Launch plan of sq_decode: the value side as in sq_attend (chunking, centroid
// table placement), then the keys' score tables after the value tables
// (4 KB-aligned, so that a table of up to 256 entries of 16 bytes starts at
// a multiple of its size), then one single staging buffer and the weights per
// wave.  The query group is served in launches of at most 4 query heads.
// Fills every field of the kernel arguments except the data pointers.
sq_status plan_decode(const sq_calib *kc, const sq_calib *vc, int first_head, int cbs, int batch, int n_q_heads,
                      int n_kv_heads, int64_t n_tokens, DecodePlan &P) {
  AttendPlan V;
  sq_status st = plan_attend(vc, first_head, cbs, batch, n_q_heads, n_kv_heads, n_tokens, V);
  if (st != SQ_OK) return st;
  const int G = n_q_heads / n_kv_heads;
  const int d = vc->heads[first_head].d;
  if (kc->heads[first_head].d != d) return fail(SQ_ERR_ARG, "sq_decode: keys and values of different head_dim");
  int max_ent = 0, max_groups = 0, max_kw = 0, max_km = 0, max_vw = 0;
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h) {
      const DevHead &K = kc->host_desc[first_head + bb * cbs + h];
      if (K.d != d) return fail(SQ_ERR_ARG, "sq_decode: heads of one call must share head_dim");
      max_ent = std::max(max_ent, K.n_fent);
      max_groups = std::max(max_groups, K.n_fgroups);
      max_kw = std::max(max_kw, K.W);
      max_km = std::max(max_km, K.m);
      max_vw = std::max(max_vw, vc->heads[first_head + bb * cbs + h].W);
    }
    if (cbs == 0) break;
  }
  if (max_kw > DEC_KW) return fail(SQ_ERR_UNSUPPORTED, "sq_decode: key records longer than 32 words");
  for (int bb = 0; bb < std::max(1, batch); ++bb) {
    for (int h = 0; h < n_kv_heads; ++h)
      if (kc->host_desc[first_head + bb * cbs + h].n_fgroups == 0)
        return fail(SQ_ERR_UNSUPPORTED, "sq_decode: a key head has more than 16 QJL bits or a record word "
                                        "with more than 8 field groups (use sq_scores + sq_attend)");
    if (cbs == 0) break;
  }
  P.gsub = std::min(G, 4);
  const int GQ = P.gsub == 3 ? 4 : P.gsub;
  AttendArgs &a = P.a;
  a = V.a;
  a.buf_floats = (max_vw + 2) * ATT_RS;  // record rows only: the scores are computed in the kernel
  const int GP = 4;
  a.wave_floats = a.buf_floats + 2 * GP * ATT_PS;
  const size_t vtab_bytes = (size_t)a.lds_wave_off * 4;  // the value side's tables (plan_attend's layout)
  a.lds_ktab = (int)((vtab_bytes + 4095) & ~(size_t)4095);
  const size_t ktab_bytes = (size_t)(max_ent + 1) * GQ * 4;  // and the zero entry
  const int wave_off_bytes = (int)((a.lds_ktab + ktab_bytes + 15) & ~(size_t)15);
  a.lds_wave_off = wave_off_bytes / 4;
  const size_t limit = (size_t)device_lds_limit();
  const int cand_col[3] = {16, 12, 8}, cand_other[2] = {8, 4};
  const int *cand = V.lm == LM_COL ? cand_col : cand_other;
  const int ncand = V.lm == LM_COL ? 3 : 2;
  P.wpb = 0;
  for (int k = 0; k < ncand; ++k) {
    const int wpb = cand[k];
    const size_t lds = (size_t)wave_off_bytes + (size_t)wpb * a.wave_floats * 4;
    // the table build uses the wave areas as scratch for q~ and w
    const size_t scratch = (size_t)P.gsub * (d + max_km) * 4;
    if (lds > limit || (size_t)wpb * a.wave_floats * 4 < scratch) continue;
    if (!dispatch(false, P.gsub, V.lm, V.np, wpb, dim3(), 0, nullptr, a)) continue;
    P.wpb = wpb;
    P.lds = lds;
    break;
  }
  if (!P.wpb) return fail(SQ_ERR_UNSUPPORTED, "sq_decode: key score tables and staging exceed the LDS");
  // chunks: a whole number of workgroups per (batch, KV head) where the
  // value side's chunking allows (never more chunks than sq_attend uses, so
  // its workspace size holds)
  const int64_t k_wg = V.a.n_chunks / P.wpb;
  if (k_wg >= 1) {
    const int64_t ct = ((n_tokens + k_wg * P.wpb - 1) / (k_wg * P.wpb) + 63) / 64 * 64;
    a.chunk_tokens = (int)ct;
    a.n_chunks = (int)((n_tokens + ct - 1) / ct);
  }
  P.lm = V.lm;
  P.np = V.np;
  P.launches = (G + P.gsub - 1) / P.gsub;
  const int64_t cgroups = (a.n_chunks + P.wpb - 1) / P.wpb;
  P.grid = dim3((unsigned)cgroups, n_kv_heads, batch);
  a.heads = vc->dev_heads;
  a.blob = (const uint8_t *)vc->dev_blob;
  a.kheads = kc->dev_heads;
  a.kblob = (const uint8_t *)kc->dev_blob;
  a.G_full = G;
  return SQ_OK;
}

}  // namespace sq

static sq_status decode_impl(const char *fn, const sq_calib *kc, const sq_calib *vc, int first_head,
                             int calib_batch_stride, int batch, int n_q_heads, int n_kv_heads, const void *q,
                             sq_dtype qdt, const uint32_t *kpacked, int64_t kps_batch, int64_t kps_head,
                             const uint32_t *vpacked, int64_t vps_batch, int64_t vps_head, int64_t n_tokens,
                             float scale, void *workspace, size_t ws_bytes, float *out, sq_stream stream,
                             const sq_paged *paged) {
  sq_status st = check_handle(kc, fn);
  if (st != SQ_OK) return st;
  st = check_handle(vc, fn);
  if (st != SQ_OK) return st;
  if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads)
    return fail(SQ_ERR_ARG, "sq_decode: n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G > 8) return fail(SQ_ERR_UNSUPPORTED, "sq_decode: query group larger than 8");
  if ((st = check_heads(kc, first_head, n_kv_heads, batch, calib_batch_stride, fn)) != SQ_OK) return st;
  if ((st = check_heads(vc, first_head, n_kv_heads, batch, calib_batch_stride, fn)) != SQ_OK) return st;
  if (n_tokens < 0) return fail(SQ_ERR_ARG, "sq_decode: n_tokens < 0");
  if (qdt != SQ_F32 && qdt != SQ_BF16) return fail(SQ_ERR_ARG, "sq_decode: bad dtype");
  if (batch == 0) { clear_error(); return SQ_OK; }
  if (!out) return fail(SQ_ERR_ARG, "sq_decode: out is NULL");
  const int d = vc->heads[first_head].d;
  hipStream_t s = (hipStream_t)stream;
  if (n_tokens == 0) {  // softmax over no tokens: zeros, as sq_attend
    AttendArgs a{};
    a.heads = vc->dev_heads;
    a.blob = (const uint8_t *)vc->dev_blob;
    a.out = out;
    a.first_head = first_head;
    a.cbs = calib_batch_stride;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.n_chunks = 0;
    launch_attend_combine(a, batch, d, s);
    return launched(fn);
  }
  if (!q || !kpacked || !vpacked || !workspace) return fail(SQ_ERR_ARG, "sq_decode: NULL pointer");
  PageArgs kpg{}, vpg{};
  if (paged) {
    if ((st = check_paged(kc, paged, n_tokens, n_kv_heads, fn, kpg)) != SQ_OK) return st;
    if ((st = check_paged(vc, paged, n_tokens, n_kv_heads, fn, vpg)) != SQ_OK) return st;
  } else {
    if ((st = check_slots(kc, n_tokens, n_kv_heads, batch, kps_batch, kps_head, fn)) != SQ_OK) return st;
    if ((st = check_slots(vc, n_tokens, n_kv_heads, batch, vps_batch, vps_head, fn)) != SQ_OK) return st;
  }
  if (n_tokens > ((int64_t)1 << 36)) return fail(SQ_ERR_UNSUPPORTED, "sq_decode: too many tokens");
  if (ws_bytes < sq_attend_workspace_bytes(batch, n_q_heads, n_tokens, d))
    return fail(SQ_ERR_ARG, "sq_decode: workspace too small (sq_attend_workspace_bytes)");
  DecodePlan P;
  if ((st = plan_decode(kc, vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens, P)) != SQ_OK)
    return st;
  if (paged)
    for (int g0 = 0; g0 < G; g0 += P.gsub)
      if (!dispatch(false, std::min(P.gsub, G - g0), P.lm, P.np, P.wpb, dim3(), 0, nullptr, P.a, true))
        return fail(SQ_ERR_UNSUPPORTED, std::string(fn) + ": no paged kernel instance without scratch for this shape");
  AttendArgs a = P.a;
  a.vpacked = vpacked;
  a.ps_b = vps_batch;
  a.ps_h = vps_head;
  a.kpacked = kpacked;
  a.kps_b = kps_batch;
  a.kps_h = kps_head;
  a.q = q;
  a.q_f32 = qdt == SQ_F32;
  a.scale = scale;
  a.ws = (float *)workspace;
  a.out = out;
  a.kpg = kpg;
  a.vpg = vpg;
  for (int g0 = 0; g0 < G; g0 += P.gsub) {
    a.g0 = g0;
    const int gn = std::min(P.gsub, G - g0);
    // a remainder smaller than the launch size takes its own instance
    dispatch(true, gn, P.lm, P.np, P.wpb, P.grid, P.lds, s, a, paged != nullptr);
    if ((st = launched(fn)) != SQ_OK) return st;
  }
  launch_attend_combine(a, batch, d, s);
  return launched(fn);
}

extern "C" sq_status sq_decode(const sq_calib *kc, const sq_calib *vc, int first_head, int calib_batch_stride,
                               int batch, int n_q_heads, int n_kv_heads, const void *q, sq_dtype qdt,
                               const uint32_t *kpacked, int64_t kps_batch, int64_t kps_head,
                               const uint32_t *vpacked, int64_t vps_batch, int64_t vps_head, int64_t n_tokens,
                               float scale, void *workspace, size_t ws_bytes, float *out, sq_stream stream) {
  return decode_impl("sq_decode", kc, vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, q, qdt,
                     kpacked, kps_batch, kps_head, vpacked, vps_batch, vps_head, n_tokens, scale, workspace,
                     ws_bytes, out, stream, nullptr);
}

extern "C" sq_status sq_decode_paged(const sq_calib *kc, const sq_calib *vc, int first_head,
                                     int calib_batch_stride, int batch, int n_q_heads, int n_kv_heads,
                                     const void *q, sq_dtype qdt, const uint32_t *kpool, const uint32_t *vpool,
                                     const sq_paged *pg, int64_t n_tokens, float scale, void *workspace,
                                     size_t ws_bytes, float *out, sq_stream stream) {
  if (!pg) return fail(SQ_ERR_ARG, "sq_decode_paged: pg is NULL");
  return decode_impl("sq_decode_paged", kc, vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, q,
                     qdt, kpool, 0, 0, vpool, 0, 0, n_tokens, scale, workspace, ws_bytes, out, stream, pg);
}
