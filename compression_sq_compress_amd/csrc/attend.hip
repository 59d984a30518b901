// sq_attend: softmax-weighted value sum over the packed values (gfx950).

#include <mutex>

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

// How sq_attend launches for a given call (see plan_attend).
struct AttendPlan {
  AttendArgs a;        // everything but the data pointers, scale and workspace
  int lm = 0, np = 1, wpb = 4, max_width = 0;
  size_t lds = 0;
  dim3 grid;
};


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
  clear_error();
  return SQ_OK;
}
