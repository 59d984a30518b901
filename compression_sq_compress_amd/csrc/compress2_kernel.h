// The register-quantising compress kernel (compress2) and its launchers.
// Its instances are compiled in compress2_contig.hip (records to contiguous
// slots) and compress2_paged.hip (records to a paged pool), in parallel.
#pragma once
#include "compress_common.h"

namespace sq {

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
// With GRID the quantise step reads instead one grid cell per value (code =
// cells' count left of it + one compare with the cell's threshold), the MFMA
// rows are the coordinates in natural order (R fragments of compress_kernel;
// for plain heads pre-scaled by the grid's a_i, the accumulators starting at
// b_i, so that the MFMAs return the grid coordinate u = a_i y_i + b_i),
// and a lane's four codes (coordinates 16 w + 4 s .. + 3, adjacent fields) are
// combined in registers and OR-ed into the record tile as one 64-bit window.
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
  int lds_nrm_off;            // floats: per-wave partial norms [64 tokens][8 waves] (normalised heads)
  int x_buf_floats;
  PageArgs pg;                // paged destination (pg.table == nullptr: contiguous slots)
};

constexpr int C2_RS = 20;   // residual tile row stride (floats; 16-byte rows, conflict-free)
constexpr int C2_SP = 16;   // sketch row pitch in LDS (floats, zero padded past d_eff)
constexpr int C2_WMAX = 6;  // record words stored per wave and tile (word k goes to wave k % waves)

// RS: record tile row stride in words (odd, above the record length: the
// last column is a pad), a constant so that token-block offsets are immediates
// GRID: quantise with the grid tables (one cell read per value, codes of a
// lane's four registers combined before one pair of record-tile ORs; MFMA
// rows in natural coordinate order) instead of the padded trees.
// NORM (grid quantiser only): normalised heads -- each token's norm nu = |y|
// (= |x|, R orthogonal) from the accumulators, summed over the waves in a
// fixed order through LDS (one extra barrier per tile); the unit vector
// y / nu is quantised and its residual sketched, and nu goes into the record
// as an IEEE half.
template <int D, bool F32, int RS, bool GRID, bool PG, bool NORM = false>
__global__ __launch_bounds__(D * 4, 4) void compress2_kernel(Compress2Args a) {
  static_assert(!NORM || GRID, "normalised heads use the grid quantiser");
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
    if constexpr (GRID) {
      const uint32_t *g = (const uint32_t *)(a.blob + hd->off_gcells);
      for (int k = threadIdx.x; k < 2 * hd->n_gcells; k += NT) ((uint32_t *)trees)[k] = g[k];
      const float *gc = (const float *)(a.blob + hd->off_gcsig);
      for (int k = threadIdx.x; k < hd->n_gcsig; k += NT) csig[k] = gc[k];
    } else {
      const float *g = (const float *)(a.blob + hd->off_tree2);
      for (int k = threadIdx.x; k < hd->n_tree2; k += NT) trees[k] = g[k];
      const float *gc = (const float *)(a.blob + hd->off_csig2);
      for (int k = threadIdx.x; k < hd->n_csig2; k += NT) csig[k] = gc[k];
    }
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
  // grid quantiser, per lane and register (coordinate 16 w + 4 s + r): u = y a + b,
  // its region's cells (LDS byte address) and last cell, signal-centroid base,
  // field shift; the lane's run of four fields: record word | bit shift << 8
  // (UQ: R rows pre-scaled by a_i, the MFMAs start at b_i and give u; ga then
  // holds 1 / a_i for the signal residuals, 1 for a zero-width row)
  constexpr bool UQ = GRID && !NORM;
  float ga[4], gcmf[4];
  f32x4 gbv = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t gtab[4], gfs[4], gpos = 0;  // gfs: field shift | signal-centroid base << 8 (0xFFFFFF: none)
  if constexpr (GRID) {
    const uint32_t cells0 = (uint32_t)(uintptr_t)trees;
    const uint4 *GC = (const uint4 *)(a.blob + hd->off_gcoord);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 16 * w + 4 * s4 + r;
      const uint4 v0 = GC[2 * c], v1 = GC[2 * c + 1];
      const float av = __uint_as_float(v0.x);
      ga[r] = !UQ ? av : av != 0.0f ? 1.0f / av : 1.0f;
      gbv[r] = __uint_as_float(v0.y);
      gtab[r] = cells0 + v0.z;
      gcmf[r] = (float)v0.w;
      gfs[r] = v1.y | ((v1.x == 0xFFFFFFFFu ? 0xFFFFFFu : v1.x) << 8);
      if (r == 0) gpos = v1.z;
      dep[r] = 0;
      tw[r] = cc[r] = 0u;
    }
  } else {
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
  // Grid quantiser, plain heads: R with row i scaled by a_i and the
  // accumulators started at b_i, so the MFMAs give u = a_i y_i + b_i directly
  // (signal residuals take y = (u - b_i) / a_i).
  const uint4 *Rf = (const uint4 *)(a.blob + (GRID ? (UQ ? hd->off_Rfrag_u : hd->off_Rfrag) : hd->off_Rfrag2));
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
  // (the x-fetch offsets are formed at each use from an opaque copy of the
  // lane index: hoisted out of the tile loop they are spilled, and the
  // reloads cost more than forming them again -- measured)
  auto lane_now = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto dma_x = [&](int tl, int buf) __attribute__((always_inline)) {
    // rows past the end re-read the last token (a whole tile past it, which
    // only zero-fills destination words, reads nothing else)
    const int64_t t0 = min<int64_t>((int64_t)tl * 64, a.n_tokens - 1);
    const char *src = xbase + t0 * a.xs_t * ESZ;
    const uint32_t last = (uint32_t)min<int64_t>(63, a.n_tokens - 1 - t0);
    const uint32_t ln = (uint32_t)lane_now();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // unsigned, so that the divisions by the power-of-two row size are shifts
      const uint32_t q = (uint32_t)(w * NB + i);
      const uint32_t byte = q * 1024u + ln * 16u, row = byte / RB, slot = (byte % RB) / 16u;
      const uint32_t c = slot ^ ((row / RPB) & (CPR - 1));
      lds_dma16(src, min(row, last) * row_bytes + c * 16u,
                lds_x + (uint32_t)buf * (uint32_t)a.x_buf_floats * 4u + q * 1024u);
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
  uint32_t *oslot = PG ? a.packed : a.packed + (int64_t)bz * a.ps_b + (int64_t)h * a.ps_h;
  const int64_t send = ((a.token0 + a.n_tokens + 63) & ~(int64_t)63) - a.token0;
  // source token i lands in slot token token0 + i: lane l of a source tile
  // writes destination lane (token0 + l) % 64 of its tile or of the next
  // word 0 of this lane's destination token for source tile tl (contiguous
  // slot: a uniform tile offset plus the lane's; paged: through the block
  // table), nullptr when the lane writes nothing
  auto dst_of = [&](int tl) __attribute__((always_inline)) -> uint32_t * {
    const int ln = lane;
    const int64_t st = (int64_t)tl * 64 + ln;
    if constexpr (!PG) {
      const int ol = (int)(a.token0 & 63) + ln;
      const uint32_t lofs = (uint32_t)((ol >> 6) * W * 64 + (ol & 63));
      return st >= send ? nullptr : oslot + ((a.token0 >> 6) + tl) * (int64_t)W * 64 + lofs;
    } else {
      // (the block lookups are wave-uniform: taken before the lane test)
      uint32_t *p = page_token_tile(a.pg, oslot, bz, h, a.token0, tl, ln, (a.token0 + a.n_tokens - 1) >> 6, W);
      return st >= send ? nullptr : p;
    }
  };
  // record words of this wave: w + NW i for i < nmine
  const int nmine = W > w ? (W - 1 - w) / NW + 1 : 0;
  int par = 0, rb = 0;
  for (int t = tb; t < te; ++t, par ^= 1, rb = rb == 2 ? 0 : rb + 1) {
    // ---- rotate: 16 rows x 64 tokens (4 blocks of 16)
    f32x4 acc[4];
    const f32x4 acc0 = UQ ? gbv : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = acc0;
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
    uint32_t *rec = rec0 + rb * 64 * rs;
    float *rtile = smem + a.lds_res_off + par * 64 * C2_RS;
    // normalised heads: 1 / nu of tokens 16 j + lane % 16 (0 for a zero vector)
    float inv_nu[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (NORM) {
      float *nrm = smem + a.lds_nrm_off;  // [token][wave]
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = acc[j][0] * acc[j][0];
#pragma unroll
        for (int r = 1; r < 4; ++r) p[j] = fmaf(acc[j][r], acc[j][r], p[j]);
        p[j] += __shfl_xor(p[j], 16);  // rows of the four lane groups
        p[j] += __shfl_xor(p[j], 32);
      }
      if (s4 == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) nrm[(16 * j + (lane & 15)) * 8 + w] = p[j];
      }
      __syncthreads();
      auto norm_of = [&](int tok) __attribute__((always_inline)) {
        float t = nrm[tok * 8];  // the NW waves' partials in a fixed order: every wave gets the same nu
#pragma unroll
        for (int i = 1; i < NW; ++i) t += nrm[tok * 8 + i];
        return __builtin_amdgcn_sqrtf(t);
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float nu = norm_of(16 * j + (lane & 15));
        inv_nu[j] = nu > 0.0f ? 1.0f / nu : 0.0f;
      }
      if (w == NW - 1)  // nu of token = lane into word W - 1 (low half after QJL bits, else high)
        atomicOr(rec + lane * rs + W - 1, half_bits_rne(norm_of(lane)) << (m > 0 ? 0 : 16));
    }
    if constexpr (GRID) {
      // one cell read per value; the lane's four codes (adjacent fields) are
      // combined, then OR-ed into the record tile as one 64-bit window
      typedef const __attribute__((address_space(3))) uint64_t lds_u64;
      uint32_t F[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t code[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // a NaN u converts to cell 0 and fails the compare: code 0
          // (v_med3_f32 returns 0 for a NaN first operand; +-inf clamp to the ends)
          const float u = UQ ? acc[j][r] : fmaf(acc[j][r] * inv_nu[j], ga[r], gbv[r]);
          const int cell = (int)__builtin_amdgcn_fmed3f(u, 0.0f, gcmf[r]);
          const uint64_t e = *(lds_u64 *)(uintptr_t)(gtab[r] + (uint32_t)cell * 8u);
          code[j] = (uint32_t)(e >> 32) + (u > __uint_as_float((uint32_t)e) ? 1u : 0u);
          F[j] |= code[j] << (gfs[r] & 31u);
        }
        const uint32_t gcb = gfs[r] >> 8;
        if (m > 0 && gcb != 0xFFFFFFu) {
          const int crd = 16 * w + 4 * s4 + r;  // < d_eff <= 16
          // y = (u - b) / a (ga holds 1 / a here; 1 and b = 0 for zero-width rows)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            rtile[((lane & 15) + 16 * j) * C2_RS + crd] =
                (UQ ? (acc[j][r] - gbv[r]) * ga[r] : acc[j][r] * inv_nu[j]) - csig[gcb + code[j]];
        }
      }
      uint32_t *rw = rec + (lane & 15) * rs + (gpos & 0xFFu);
      const uint32_t sh = gpos >> 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint64_t v = (uint64_t)F[j] << sh;
        atomicOr(rw + 16 * j * rs, (uint32_t)v);
        atomicOr(rw + 16 * j * rs + 1, (uint32_t)(v >> 32));
      }
    } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(tw[r]), "+v"(cc[r]));
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
      uint32_t *ocur = dst_of(t);
      uint32_t *oprv = has_prev ? dst_of(t - 1) : nullptr;
      const bool valid = (int64_t)t * 64 + lane < a.n_tokens;
      const bool pvalid = (int64_t)(t - 1) * 64 + lane < a.n_tokens;
      const bool in = ocur != nullptr, pin = oprv != nullptr;
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
            o[(uint32_t)(w + NW * i) * 64u] = (q ? pvalid : valid) ? v[u] : 0u;
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
    uint32_t *dst = dst_of(te - 1);
    const bool valid = (int64_t)(te - 1) * 64 + lane < a.n_tokens;
    const bool in = dst != nullptr;
#pragma unroll
    for (int i = 0; i < C2_WMAX; ++i)
      if ((qmask >> i & 1u) && i < nmine && in) dst[(int64_t)(w + NW * i) * 64] = valid ? rlast[w + NW * i] : 0u;
  }
}

template <int D, bool F32, bool GRID, bool PG, bool NORM = false>
void launch_compress2_g(int rsc, dim3 grid, size_t lds, hipStream_t s, const Compress2Args &a) {
  // record strides this head size can need (at most C2_WMAX words per wave)
  if (rsc == 17) {
    hipLaunchKernelGGL((compress2_kernel<D, F32, 17, GRID, PG, NORM>), grid, dim3(4 * D), lds, s, a);
  } else if constexpr (D >= 64) {
    if (rsc == 33) hipLaunchKernelGGL((compress2_kernel<D, F32, 33, GRID, PG, NORM>), grid, dim3(4 * D), lds, s, a);
    else if constexpr (D == 128) hipLaunchKernelGGL((compress2_kernel<D, F32, 49, GRID, PG, NORM>), grid, dim3(4 * D), lds, s, a);
  }
}

// normalised heads: bf16 input, contiguous slots, grid quantiser
void launch_compress2_norm(int d, int rsc, dim3 grid, size_t lds, hipStream_t s, const Compress2Args &a);

// every instance of one destination kind (PG), by head size, input dtype and quantiser
template <bool PG>
void launch_compress2_pg(int d, bool f32, bool gridq, int rsc, dim3 grid, size_t lds, hipStream_t s,
                         const Compress2Args &a) {
  auto by_d = [&](auto dc, auto fc) {
    constexpr int DD = decltype(dc)::value;
    constexpr bool FF = decltype(fc)::value;
    if (gridq) launch_compress2_g<DD, FF, true, PG>(rsc, grid, lds, s, a);
    else launch_compress2_g<DD, FF, false, PG>(rsc, grid, lds, s, a);
  };
  using T = std::true_type;
  using F = std::false_type;
  switch (d) {
    case 32: f32 ? by_d(std::integral_constant<int, 32>(), T()) : by_d(std::integral_constant<int, 32>(), F()); break;
    case 64: f32 ? by_d(std::integral_constant<int, 64>(), T()) : by_d(std::integral_constant<int, 64>(), F()); break;
    default: f32 ? by_d(std::integral_constant<int, 128>(), T()) : by_d(std::integral_constant<int, 128>(), F()); break;
  }
}

}  // namespace sq
