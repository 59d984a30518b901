// sq_compress and sq_compress_append: rotation, quantisation, selective QJL
// and packing of K/V vectors (gfx950).

#include <cstdlib>
#include <cstring>

#include "compress_common.h"
#include "compress2_kernel.h"

namespace sq {

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
  PageArgs pg;          // paged destination (pg.table == nullptr: contiguous slots)
};

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
// PG: records go to a paged pool through the block table (else contiguous slots)
template <int D, bool F32, bool TG, bool PG>
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
  uint32_t *pdst = nullptr;  // this lane's destination of the previous tile's records
  bool pvalid = false, pin = false, have_prev = false;
  // Source token i lands in slot token token0 + i: lane l of a source tile
  // writes destination lane (token0 + l) % 64 of its tile or of the next.
  // Lanes past the last token zero their words up to the end of the last
  // destination tile and write nothing beyond it.
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
    if (have_prev) store_prev();
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
    if (hd->normalized) {
      // normalised variant: the vector's norm nu = |y| (= |x|) goes into the
      // record as a half and the unit vector y / nu is quantised (a zero
      // vector stays zero; a NaN one stays NaN)
      if (w == 0) {
        float s2 = 0.0f;
        for (int i = 0; i < D; ++i) s2 = fmaf(yrow[i], yrow[i], s2);
        const float nu = __builtin_amdgcn_sqrtf(s2);
        const float inv = nu > 0.0f ? 1.0f / nu : 0.0f;
        for (int i = 0; i < D; ++i) yrow[i] *= inv;
        atomicOr(bwrow + (W - 1), half_bits_rne(nu) << (m > 0 ? 0 : 16));
      }
      __syncthreads();
    }
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
    // ---- larger sketches: every wave takes m / NW of the QJL rows (16 at a
    // time, the lane's residuals read 16 at a time) and ORs their bits into
    // the word buffer; the last wave adds gamma.  A barrier then separates
    // these ORs from the stores of the words at the top of the next tile.
    const bool qslow = m > 0 && !(m <= 8 && d_eff <= 8);
    if (qslow) {
      const int jb = (w * m) / NW, je = ((w + 1) * m) / NW;
      const float *Sb = a.lds_s_off >= 0 ? S_lds : (const float *)S_glb;
      for (int j0 = jb; j0 < je; j0 += 16) {
        const int nj = min(16, je - j0);
        float dot[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) dot[jj] = 0.0f;
        for (int i0 = 0; i0 < d_eff; i0 += 16) {
          const int ni = min(16, d_eff - i0);
          float yv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) yv[u] = u < ni ? yrow[i0 + u] : 0.0f;
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            if (jj < nj) {
              const float *srow = Sb + (size_t)(j0 + jj) * d_eff + i0;
              float acc = dot[jj];
#pragma unroll
              for (int u = 0; u < 16; ++u)
                if (u < ni) acc = fmaf(srow[u], yv[u], acc);
              dot[jj] = acc;
            }
          }
        }
        uint32_t zb = 0u;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          if (jj < nj) zb |= (dot[jj] >= 0.0f ? 1u : 0u) << jj;
        const int pbit = code_bits + j0;
        const uint64_t v = (uint64_t)zb << (pbit & 31);
        atomicOr(bwrow + (pbit >> 5), (uint32_t)v);
        if ((uint32_t)(v >> 32)) atomicOr(bwrow + (pbit >> 5) + 1, (uint32_t)(v >> 32));
      }
      if (w == NW - 1) {
        float g2 = 0.0f;
        for (int i = 0; i < d_eff; ++i) g2 = fmaf(yrow[i], yrow[i], g2);
        atomicOr(bwrow + W - 1, half_bits_rne(sqrtf(g2)) << 16);
      }
      __syncthreads();
    }
    pvalid = t0 + lane < T;
    pin = t0 + lane < send;
    // destination of this lane's token (contiguous slot or its block; nullptr: dropped)
    if constexpr (PG) {
      uint32_t *p = page_token_tile(a.pg, a.packed, b, h, a.token0, tile, lane, (a.token0 + T - 1) >> 6, W);
      pdst = pin ? p : nullptr;
    } else {
      const int ol = (int)(a.token0 & 63) + lane;
      pdst = a.packed + (int64_t)b * a.ps_b + (int64_t)h * a.ps_h + ((a.token0 >> 6) + tile) * W * 64 +
             (int64_t)(ol >> 6) * W * 64 + (ol & 63);
    }
    pin = pin && pdst != nullptr;
    have_prev = true;
    // The x tile was last read by the MFMAs, which every wave finished before
    // the barrier above; the y tile and the word buffer are rewritten only
    // after the barrier that follows the next x store.
  }
  if (have_prev) store_prev();
}


// compress2 instances live in compress2_contig.hip and compress2_paged.hip
extern template void launch_compress2_pg<false>(int, bool, bool, int, dim3, size_t, hipStream_t, const Compress2Args &);
extern template void launch_compress2_pg<true>(int, bool, bool, int, dim3, size_t, hipStream_t, const Compress2Args &);

}  // namespace sq

using namespace sq;

template <int D, bool F32, bool TG>
static void launch_compress(bool pg, dim3 grid, size_t lds, hipStream_t s, const CompressArgs &a) {
  if (pg) hipLaunchKernelGGL((compress_kernel<D, F32, TG, true>), grid, dim3(4 * D), lds, s, a);
  else hipLaunchKernelGGL((compress_kernel<D, F32, TG, false>), grid, dim3(4 * D), lds, s, a);
}

template <int D>
static void launch_compress_d(bool f32, bool tg, dim3 grid, size_t lds, hipStream_t s, const CompressArgs &a) {
  const bool pg = a.pg.table != nullptr;
  if (f32) tg ? launch_compress<D, true, true>(pg, grid, lds, s, a) : launch_compress<D, true, false>(pg, grid, lds, s, a);
  else tg ? launch_compress<D, false, true>(pg, grid, lds, s, a) : launch_compress<D, false, false>(pg, grid, lds, s, a);
}


// sq_compress and sq_compress_append: source token i of x goes to token slot
// token0 + i of every head's packed slot.
static sq_status compress_impl(const char *fn, const sq_calib *c, int first_head, int n_heads, int batch,
                               int calib_batch_stride, const void *x, sq_dtype dt, int64_t n_tokens,
                               int64_t xs_batch, int64_t xs_head, int64_t xs_token, uint32_t *packed,
                               int64_t ps_batch, int64_t ps_head, int64_t token0, sq_stream stream,
                               const sq_paged *paged = nullptr) {
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
  PageArgs pga{};
  if (paged) {
    if ((st = check_paged(c, paged, token0 + n_tokens, n_heads, fn, pga)) != SQ_OK) return st;
  } else {
    st = check_slots(c, token0 + n_tokens, n_heads, batch, ps_batch, ps_head, fn);
    if (st != SQ_OK) return st;
  }
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
    // (normalised heads have no tree plan, n_p2 = 0: they take the grid tables)
    bool use2 = d <= 128 && 64 * xs_token * esz < ((int64_t)1 << 32) && c->W_max <= C2_WMAX * (d / 16) &&
                n_heads <= 65535 && batch <= 65535;
    // quantiser: the grid tables when every head has them, else the padded
    // trees (the environment variable SQ_QUANTISER = "tree" forces the trees)
    const char *qenv = std::getenv("SQ_QUANTISER");
    bool gridq = use2 && !(qenv && std::strcmp(qenv, "tree") == 0);
    bool treeq = use2;
    int mt = 0, mc = 0, mq = 0, mg = 0, mgc = 0, n_norm = 0, n_seen = 0;
    for (int bb = 0; bb < std::max(1, batch) && use2; ++bb) {
      for (int h = 0; h < n_heads; ++h) {
        const DevHead &hd = c->host_desc[first_head + bb * calib_batch_stride + h];
        n_norm += hd.normalized ? 1 : 0;
        n_seen += 1;
        if (hd.n_p2 == 0) treeq = false;
        if (hd.n_gcells == 0) gridq = false;
        mt = std::max(mt, hd.n_tree2);
        mc = std::max(mc, hd.n_csig2);
        mq = std::max(mq, hd.m);
        mg = std::max(mg, 2 * hd.n_gcells);
        mgc = std::max(mgc, hd.n_gcsig);
      }
      if (calib_batch_stride == 0) break;
    }
    // normalised heads: the grid kernel's NORM instances (bf16 input,
    // contiguous slots, every head of the call normalised)
    const bool norm = n_norm > 0;
    if (norm && (n_norm != n_seen || dt != SQ_BF16 || paged)) gridq = false;
    if (norm) treeq = false;
    use2 = gridq || treeq;
    if (gridq) {
      mt = mg;
      mc = mgc;
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
      b2.lds_nrm_off = b2.lds_res_off + 2 * 64 * C2_RS;
      const size_t lds2 = (size_t)(b2.lds_nrm_off + (norm ? 64 * 8 : 0)) * 4;
      if (lds2 <= (size_t)device_lds_limit()) {
        b2.heads = c->dev_heads;
        b2.blob = (const uint8_t *)c->dev_blob;
        b2.x = x;
        b2.packed = packed;
        b2.pg = pga;
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
        if (norm) launch_compress2_norm(d, rsc, grid, lds2, s, b2);
        else if (b2.pg.table) launch_compress2_pg<true>(d, f32, gridq, rsc, grid, lds2, s, b2);
        else launch_compress2_pg<false>(d, f32, gridq, rsc, grid, lds2, s, b2);
        return launched(fn);
      }
    }
  }
  CompressArgs a{};
  a.ys = d + 3;  // odd, and conflict-free for the MFMA-layout stores
  a.bws = (c->W_max % 2 == 0) ? c->W_max + 1 : c->W_max;
  const int xs_floats = dt == SQ_F32 ? 64 * (d + 4) : 64 * (d + 8) / 2;
  const size_t limit = (size_t)device_lds_limit();
  // the sketch goes to LDS when the workgroup still fits (else it is read
  // through the L1/L2)
  const int rest_no_s = ((max_csig + 3) & ~3) + max_plan + 64 + xs_floats + 64 * a.ys + 64 * a.bws;
  const bool s_in_lds = (size_t)(rest_no_s + ((max_s + 3) & ~3)) * 4 <= limit;
  const int s_floats = s_in_lds ? ((max_s + 3) & ~3) : 0;
  const int rest = rest_no_s + s_floats;
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
  a.pg = pga;
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

extern "C" sq_status sq_compress_append_paged(const sq_calib *c, int first_head, int n_heads, int batch,
                                              int calib_batch_stride, const void *x, sq_dtype dt,
                                              int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                                              int64_t xs_token, uint32_t *pool, const sq_paged *pg,
                                              int64_t token0, sq_stream stream) {
  if (!pg) return fail(SQ_ERR_ARG, "sq_compress_append_paged: pg is NULL");
  return compress_impl("sq_compress_append_paged", c, first_head, n_heads, batch, calib_batch_stride, x, dt,
                       n_tokens, xs_batch, xs_head, xs_token, pool, 0, 0, token0, stream, pg);
}

extern "C" sq_status sq_compress_append(const sq_calib *c, int first_head, int n_heads, int batch,
                                        int calib_batch_stride, const void *x, sq_dtype dt,
                                        int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                                        int64_t xs_token, uint32_t *packed, int64_t ps_batch,
                                        int64_t ps_head, int64_t token0, sq_stream stream) {
  return compress_impl("sq_compress_append", c, first_head, n_heads, batch, calib_batch_stride, x, dt,
                       n_tokens, xs_batch, xs_head, xs_token, packed, ps_batch, ps_head, token0, stream);
}
