// sq_attend: softmax-weighted value sum over the packed values (gfx950).

#include <mutex>

#include "attend_kernel.h"

namespace sq {

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

void launch_attend_combine(const AttendArgs &a, int batch, int d, hipStream_t s) {
  const size_t lds = a.n_chunks > 0 ? (size_t)(a.n_chunks + d) * 4 : 0;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * a.n_q_heads), dim3(256), lds, s, a);
}

}  // namespace sq


using namespace sq;

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

// Launch plan of sq_attend for a set of heads: chunk size, table placement
// (column / packed / global), waves per workgroup, LDS layout and grid.
// Fills every field of the kernel arguments except the data pointers.
namespace sq {
sq_status plan_attend(const sq_calib *vc, int first_head, int calib_batch_stride, int batch, int n_q_heads,
                      int n_kv_heads, int64_t n_tokens, AttendPlan &P) {
  const int G = n_q_heads / n_kv_heads;
  const int d = vc->heads[first_head].d;
  AttendArgs &a = P.a;
  a = AttendArgs{};
  a.heads = vc->dev_heads;
  a.blob = (const uint8_t *)vc->dev_blob;
  a.n_tokens = n_tokens;
  a.first_head = first_head;
  a.cbs = calib_batch_stride;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.g0 = 0;
  a.G_full = G;
  a.chunk_tokens = (int)attend_chunk_tokens(batch, n_q_heads, n_tokens);
  a.n_chunks = (int)((n_tokens + a.chunk_tokens - 1) / a.chunk_tokens);
  const int np = (d + 63) / 64;  // 64-coordinate blocks, all served by one wave
  if (np != 1 && np != 2 && np != 4) return fail(SQ_ERR_UNSUPPORTED, "sq_attend: unsupported head_dim");
  P.np = np;
  // LDS: centroid tables of the blocks | waves x (staging buffers, weights)
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
  P.max_width = max_w;
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
  // Column tables take one 64-bit window of record rows starting 8 bits below
  // a lane's first field for all its np fields: 8 + np * max_w bits, plus up
  // to 31 bits of offset inside the first row, must stay within 64.
  const bool col_fits = max_w <= 6 && 39 + np * max_w <= 64;
  // table placement: column tables (conflict-free), shared by 16 waves with
  // one staging buffer each when that fits a CU (four waves per SIMD), else
  // by 8 double-buffered waves when that keeps as many waves per CU as
  // 4-wave workgroups would (fewer table copies); else 4-wave workgroups with
  // column tables unless packed tables let more of them share a CU
  int lm = LM_GLB, wpb = 4;
  size_t lds = 0;
  const size_t cu_lds = (size_t)limit;  // one workgroup may use all of a CU's LDS
  const size_t cap = (size_t)std::min(limit, 64 * 1024);
  const size_t lds_col = col_fits ? lds_for(64 << max_w, 4) : cap + 1;
  const size_t lds_col8 = col_fits ? lds_for(64 << max_w, 8) : cu_lds + 1;
  const size_t lds_pack = lds_for(max_lut + 64, 4);
  const int wf2 = a.wave_floats, wf1 = a.buf_floats + 2 * GP * ATT_PS;
  a.wave_floats = wf1;
  const size_t lds_col16 = col_fits ? lds_for(64 << max_w, 16) : cu_lds + 1;
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
  P.grid = dim3((unsigned)cgroups, n_kv_heads, batch);
  if (P.grid.z > 65535 || P.grid.y > 65535 || cgroups > INT32_MAX)
    return fail(SQ_ERR_UNSUPPORTED, "sq_attend: grid too large");
  P.lm = lm;
  P.wpb = wpb;
  P.lds = lds;
  return SQ_OK;
}
}  // namespace sq

// Fixed device scratch of sq_attend_noalloc (the split-T partials), one copy
// per GPU for the life of the process.  In host code `scratch` names a
// host-side stand-in, never the device array: its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.  Every chunk's partials are written
// in full before the combine reads them, so nothing needs clearing between
// calls; calls that overlap on one GPU share the array and race.
namespace sq {
__device__ __align__(256) float scratch[SQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];
}  // namespace sq
static std::mutex g_scratch_mu;
static void *g_scratch_addr[64] = {};

static sq_status scratch_for_current_device(const char *fn, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= 64) return fail(SQ_ERR_UNSUPPORTED, std::string(fn) + ": device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(sq::scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (!p) return fail(SQ_ERR_HIP, std::string(fn) + ": no device address for the scratch array");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SQ_OK;
}

// sq_attend and sq_attend_noalloc.  With scratch_ok the partials go to the
// library's fixed device scratch (workspace == nullptr on entry): its address
// is taken only after every argument has been validated.
static sq_status attend_impl(const char *fn, const sq_calib *vc, int first_head, int calib_batch_stride,
                             int batch, int n_q_heads, int n_kv_heads, const float *scores, float scale,
                             const uint32_t *vpacked, int64_t ps_batch, int64_t ps_head, int64_t n_tokens,
                             void *workspace, size_t ws_bytes, float *out, sq_stream stream,
                             bool scratch_ok) {
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
  hipStream_t s = (hipStream_t)stream;
  if (n_tokens == 0) {
    AttendArgs a{};
    a.heads = vc->dev_heads;
    a.blob = (const uint8_t *)vc->dev_blob;
    a.out = out;
    a.first_head = first_head;
    a.cbs = calib_batch_stride;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.n_chunks = 0;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * n_q_heads), dim3(256), 0, s, a);
    return launched(fn);
  }
  if (!scores || !vpacked || (!workspace && !scratch_ok)) return fail(SQ_ERR_ARG, "sq_attend: NULL pointer");
  st = check_slots(vc, n_tokens, n_kv_heads, batch, ps_batch, ps_head, fn);
  if (st != SQ_OK) return st;
  const size_t ws_need = sq_attend_workspace_bytes(batch, n_q_heads, n_tokens, d);
  if (scratch_ok) {
    if (ws_need > SQ_NOALLOC_SCRATCH_BYTES)
      return fail(SQ_ERR_UNSUPPORTED, std::string(fn) + ": the partials need " + std::to_string(ws_need) +
                                          " bytes, more than the library's fixed scratch of " +
                                          std::to_string((size_t)SQ_NOALLOC_SCRATCH_BYTES) + " bytes");
    st = scratch_for_current_device(fn, &workspace);
    if (st != SQ_OK) return st;
    ws_bytes = SQ_NOALLOC_SCRATCH_BYTES;
  }
  if (ws_bytes < ws_need) return fail(SQ_ERR_ARG, "sq_attend: workspace too small");
  AttendPlan P;
  st = plan_attend(vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens, P);
  if (st != SQ_OK) return st;
  AttendArgs a = P.a;
  a.scores = scores;
  a.vpacked = vpacked;
  a.out = out;
  a.ps_b = ps_batch; a.ps_h = ps_head;
  a.scale = scale;
  a.ws = (float *)workspace;
  switch (G) {
    case 1: launch_attend<1>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 2: launch_attend<2>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 3: launch_attend<3>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 4: launch_attend<4>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 5: launch_attend<5>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 6: launch_attend<6>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 7: launch_attend<7>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
    case 8: launch_attend<8>(P.lm, P.np, P.wpb, P.grid, P.lds, s, a); break;
  }
  sq_status s1 = launched(fn);
  if (s1 != SQ_OK) return s1;
  const size_t lds2 = (size_t)(a.n_chunks + d) * 4;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * n_q_heads), dim3(256), lds2, s, a);
  return launched(fn);
}

extern "C" sq_status sq_attend(const sq_calib *vc, int first_head, int calib_batch_stride, int batch,
                               int n_q_heads, int n_kv_heads, const float *scores, float scale,
                               const uint32_t *vpacked, int64_t ps_batch, int64_t ps_head,
                               int64_t n_tokens, void *workspace, size_t ws_bytes, float *out,
                               sq_stream stream) {
  return attend_impl("sq_attend", vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, scores,
                     scale, vpacked, ps_batch, ps_head, n_tokens, workspace, ws_bytes, out, stream, false);
}

extern "C" sq_status sq_attend_noalloc(const sq_calib *vc, int first_head, int calib_batch_stride,
                                       int batch, int n_q_heads, int n_kv_heads, const float *scores,
                                       float scale, const uint32_t *vpacked, int64_t ps_batch,
                                       int64_t ps_head, int64_t n_tokens, float *out, sq_stream stream) {
  return attend_impl("sq_attend_noalloc", vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads,
                     scores, scale, vpacked, ps_batch, ps_head, n_tokens, nullptr, 0, out, stream, true);
}

// Diagnostic: how sq_scores and sq_attend launch for these arguments.
extern "C" sq_status sq_plan_decode(const sq_calib *kc, const sq_calib *vc, int first_head,
                                    int calib_batch_stride, int batch, int n_q_heads, int n_kv_heads,
                                    int64_t n_tokens, sq_decode_plan *out) {
  const char *fn = "sq_plan_decode";
  if (!out) return fail(SQ_ERR_ARG, "sq_plan_decode: out is NULL");
  std::memset(out, 0, sizeof(*out));
  if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads || n_q_heads / n_kv_heads > 8)
    return fail(SQ_ERR_ARG, "sq_plan_decode: bad head counts");
  if (batch <= 0 || n_tokens <= 0) return fail(SQ_ERR_ARG, "sq_plan_decode: batch and n_tokens must be > 0");
  sq_status st;
  if (kc) {
    if ((st = check_handle(kc, fn)) != SQ_OK) return st;
    if ((st = check_heads(kc, first_head, n_kv_heads, batch, calib_batch_stride, fn)) != SQ_OK) return st;
    if ((st = score_plan_summary(kc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens,
                                 &out->score_passes, &out->score_quads, &out->score_wave_groups)) != SQ_OK)
      return st;
  }
  if (vc) {
    if ((st = check_handle(vc, fn)) != SQ_OK) return st;
    if ((st = check_heads(vc, first_head, n_kv_heads, batch, calib_batch_stride, fn)) != SQ_OK) return st;
    AttendPlan P;
    if ((st = plan_attend(vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens, P)) != SQ_OK)
      return st;
    out->attend_placement = P.lm;
    out->attend_waves = P.wpb;
    out->attend_blocks = P.np;
    out->attend_chunks = P.a.n_chunks;
  }
  if (kc && vc) {
    DecodePlan D;
    if ((st = plan_decode(kc, vc, first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads, n_tokens, D)) ==
        SQ_OK) {
      out->decode_launches = D.launches;
      out->decode_waves = D.wpb;
      out->decode_lds_bytes = (int)D.lds;
    } else {
      out->decode_launches = 0;  // sq_decode would refuse these arguments (message in sq_last_error)
      return st;
    }
  }
  clear_error();
  return SQ_OK;
}
