// sq_dequantize: diagnostic reconstruction of packed vectors (gfx950).

#include "devcommon.h"

namespace sq {

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
      if (hd->normalized) {  // normalised variant: times the stored vector norm
        const uint32_t wl = word(t, W - 1);
        v *= half_bits_to_f32(m > 0 ? (wl & 0xFFFFu) : (wl >> 16));
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


}  // namespace sq

using namespace sq;

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
