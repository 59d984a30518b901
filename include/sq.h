/*
 * sq.h -- C ABI of libsq, an MI355X (gfx950) implementation of the SpectralQuant
 * KV-cache compression hot path.
 *
 * SpectralQuant (README "Overview", "Repository Structure"; ossradar.top summary,
 * "core capabilities") rotates each key/value vector of an attention head into an
 * eigenbasis calibrated once per head, quantises every rotated coordinate with a
 * Lloyd-Max codebook at a bit width chosen by reverse water-filling over the
 * eigenvalues, and corrects only the few "signal" coordinates of keys (the top
 * d_eff, d_eff = rounded participation ratio) with a 1-bit QJL sign sketch of the
 * quantisation residual.  Decode-time scoring rotates the query once and reads
 * q.k directly from the packed codes plus the QJL term; the value side
 * dequantises codes for the softmax-weighted sum.
 *
 * Conventions for every call:
 *   - Return value: SQ_OK (0) or an sq_status error.  On error nothing was
 *     enqueued on the stream and sq_last_error() returns a message for the
 *     calling thread.
 *   - Device calls enqueue work on the caller's HIP stream (hipStream_t passed
 *     as sq_stream; NULL = the legacy default stream) and return at once.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - "DEVICE" pointers are device memory owned by the caller (e.g. torch
 *     tensors); "HOST" pointers are host memory owned by the caller.  Nothing
 *     is allocated on the hot path (sq_compress, sq_scores, sq_attend,
 *     sq_dequantize).
 *   - A calibration handle is immutable after sq_calib_upload; concurrent calls
 *     on different streams that share it are safe.  Calls that write the same
 *     output buffer from different streams race.
 *   - NaN inputs are not checked on the hot path: a NaN coordinate compares
 *     false against every threshold and gets code 0.  A NaN entry of x makes
 *     every rotated coordinate of that vector NaN: all codes 0, for keys no
 *     QJL bit set and a NaN gamma.
 *
 * Packed record layout (one record per (head, token); identical in the CPU
 * oracle, which implements it independently):
 *   - W 32-bit words, bit p = bit (p % 32) of word (p / 32);
 *   - code fields of coordinates i = 0..d-1 in eigen order, b_i bits each,
 *     back to back from bit 0 (fields may straddle words);
 *   - then the m QJL bits z_0..z_{m-1};
 *   - if m > 0: gamma (residual norm) as IEEE half in bits [32W-16, 32W);
 *   - normalised calibrations: the vector norm nu as IEEE half in bits
 *     [32W-32, 32W-16) if m > 0, else in bits [32W-16, 32W);
 *   - W = max(1, ceil((sum b_i + m + 16*[m>0] + 16*[normalised]) / 32));
 *     unused bits are zero;
 *   - word w of token t lives at 32-bit element ((t/64)*W + w)*64 + t%64 of the
 *     head's slot, so one wavefront reads word w of 64 tokens as one coalesced
 *     256-byte access.  T is padded to a multiple of 64 with all-zero records.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SQ_OK = 0,
  SQ_ERR_ARG = 1,          /* bad argument (null pointer, bad size, bad head range) */
  SQ_ERR_UNSUPPORTED = 2,  /* valid but outside this build's limits (head_dim, LDS) */
  SQ_ERR_NUMERIC = 3,      /* non-finite calibration samples, fewer than 2 samples */
  SQ_ERR_HIP = 4,          /* a HIP runtime call failed (message holds hipGetErrorString) */
  SQ_ERR_ALLOC = 5,        /* host or device allocation failed (calibration only) */
  SQ_ERR_IO = 6,           /* save/load failure or malformed file */
  SQ_ERR_STATE = 7         /* handle not uploaded before a device call */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_BF16 = 1 } sq_dtype;

typedef void *sq_stream; /* a hipStream_t */

typedef struct {
  int head_dim;                 /* 32, 64, 128 or 256 */
  double avg_bits;              /* code-bit budget per coordinate; round(avg_bits*d) bits */
  int qjl_bits_per_signal_dim;  /* QJL rows per signal dim: 1 for keys, 0 for values */
  int max_bits;                 /* widest code field, 1..8 */
  int lloyd_max_iters;          /* cap of the per-region Lloyd-Max iteration */
  int n_threads;                /* host threads used by sq_calibrate; 0 = hardware count */
  int normalize;                /* 1: normalised variant -- samples divided by their norms
                                   before calibration; each record stores its vector's
                                   norm (IEEE half) and the unit vector is quantised */
  double deff_cumvar;           /* d_eff rule.  0: rounded participation ratio (default).
                                   In (0, 1]: the smallest k whose k leading eigenvalues
                                   hold at least this fraction of their sum (the README's
                                   "participation ratio vs cumvar" sweep; its threshold is
                                   not given there, so the caller chooses it) */
} sq_calib_opts;

typedef struct sq_calib sq_calib; /* opaque, library-owned */

typedef struct {
  int head_dim;
  int d_eff;           /* rounded participation ratio, clamped to [1, d] */
  int m;               /* QJL rows = qjl_bits_per_signal_dim * d_eff (0 for values) */
  int code_bits;       /* sum of widths */
  int record_words;    /* W */
  int n_thresholds;    /* sum over coordinates of 2^b_i - 1 */
  int n_centroids;     /* sum over coordinates of 2^b_i (b_i > 0) */
  int n_regions;       /* (regime, width) codebooks fitted */
  int lloyd_unconverged; /* regions that hit the iteration cap */
  double participation_ratio;
  double kappa;        /* lambda[d_eff-1] / lambda[d_eff]; +inf if d_eff == d */
  int normalized;      /* records carry the vector norm (normalised variant) */
} sq_head_info;

/* Defaults: avg_bits 3, qjl 1 (keys), max_bits 8, 200 Lloyd-Max iterations,
 * unnormalised, d_eff by the rounded participation ratio. */
sq_status sq_calib_default_opts(sq_calib_opts *opts, int head_dim);

/*
 * sq_calibrate -- host-side, one-time calibration of n_heads independent heads.
 * README "Repository Structure" (calibration: PCA, d_eff, kappa; Lloyd-Max with
 * per-regime codebooks) and the repository's tests/conftest.py fixture
 * pre_computed_calibration (uncentered X^T X / n, eigh reversed to descending,
 * d_eff = round(PR), kappa).  Per head, in double precision:
 *   1. C = X^T X / n; Jacobi eigendecomposition; eigenvalues descending
 *      (clamped at 0); each eigenvector signed so its largest-magnitude entry
 *      is positive; R = rows of eigenvectors.
 *   2. d_eff = round-half-even(PR), PR = (sum l)^2 / sum l^2 (or, with
 *      opts->deff_cumvar > 0, the smallest k with l_0 + .. + l_{k-1} >=
 *      deff_cumvar * sum l); kappa = l[d_eff-1] / l[d_eff].
 *   3. widths: greedy reverse water-filling of round(avg_bits*d) bits, one bit
 *      at a time to argmax l_i * 4^-b_i (ties to the lower index), b_i <= max_bits.
 *   4. regions (signal = i < d_eff | noise, width); per region a Lloyd-Max
 *      codebook fitted on the pooled standardised samples (R x)_i / sqrt(l_i),
 *      started at the (j+1/2)/L sample quantiles, iterated until the partition
 *      repeats or lloyd_max_iters; tables scaled by sqrt(l_i) per coordinate.
 *   5. QJL matrix S = qjl_gauss[h][0:m][0:d_eff] (m = qjl_bits * d_eff).
 * samples   HOST float [n_heads][n_samples][head_dim], read only.
 * qjl_gauss HOST float [n_heads][qjl_bits*head_dim][head_dim] standard-normal
 *           draws supplied by the caller (NULL allowed when qjl_bits == 0).
 * out       receives a new handle (free with sq_calib_destroy).
 * Errors: SQ_ERR_ARG (null/size), SQ_ERR_UNSUPPORTED (head_dim),
 *         SQ_ERR_NUMERIC (n_samples < 2, non-finite sample), SQ_ERR_ALLOC.
 */
sq_status sq_calibrate(const float *samples, int n_heads, int64_t n_samples,
                       const sq_calib_opts *opts, const float *qjl_gauss,
                       sq_calib **out);

/*
 * sq_calibrate_device -- the same calibration with its dense steps on the
 * GPU (README "Overview": a one-time calibration pass; "Repository
 * Structure": calibration by PCA, d_eff, kappa).  On `stream`, in fp64: the
 * per-sample norms (normalised variant), C = X^T X / n, a parallel cyclic
 * Jacobi eigendecomposition of every head (one workgroup per head; rotations
 * of the same 2 x 2 Schur form as sq_calibrate's solver, applied to the d/2
 * disjoint pairs of a round-robin step at once), and the rotated samples
 * Y = X R^T.  The host then applies the eigen-order and sign rule, d_eff,
 * widths, the per-region Lloyd-Max fits and the QJL rows exactly as
 * sq_calibrate does, on opts->n_threads threads.  Results equal
 * sq_calibrate's up to rounding order: eigenvalues and the eigenvectors of
 * well-separated eigenvalues to ~1e-12 relative, codebooks to ~1e-6.
 * samples   DEVICE float [n_heads][n_samples][head_dim] (read only).
 * qjl_gauss HOST float, as for sq_calibrate.
 * Allocates device scratch of 24 d^2 n_heads bytes (+ 8 n_samples n_heads
 * when normalising) and at most 512 MiB of rotated samples per chunk of
 * heads (also on the host); returns after the stream work is complete.
 * Errors: as sq_calibrate; SQ_ERR_UNSUPPORTED for more than 65535 heads or
 * more than 2^30 samples, or when one head's rotated samples exceed 512 MiB;
 * SQ_ERR_HIP on a failed launch or copy.
 */
sq_status sq_calibrate_device(const float *samples, int n_heads, int64_t n_samples,
                              const sq_calib_opts *opts, const float *qjl_gauss,
                              sq_stream stream, sq_calib **out);

/*
 * sq_calibrate_tq -- the TurboQuant-style baseline (random rotation, per-vector
 * norm, Gaussian Lloyd-Max codebook of the rotated unit vector's coordinates,
 * QJL over all dims for keys) as a calibration handle that the same device
 * calls run (TurboQuant reference-implementation page, "Project Structure":
 * the MSE quantiser, and the Prod quantiser = (b-1)-bit MSE stage + 1-bit QJL
 * of the residual; "Key Findings" 2: Prod for keys, MSE for values).  No data
 * is needed.  Per head: R = rotation[h] (rows: y = R x, orthogonal);
 * normalised records; every coordinate at width b - 1 (keys:
 * opts->qjl_bits_per_signal_dim == 1, then m = d QJL rows S = qjl_gauss[h]
 * over all d coordinates) or b (values: qjl_bits_per_signal_dim == 0), with
 * b = opts->avg_bits (an integer 1..8 for values, 2..9 for keys, minus the
 * QJL bit at most 8); codebook: the Lloyd-Max quantiser of N(0, 1) (Max,
 * 1960) scaled by 1/sqrt(d), the same for every coordinate.
 * rotation  HOST float [n_heads][head_dim][head_dim].
 * qjl_gauss HOST float [n_heads][head_dim][head_dim] (keys), else NULL.
 * Errors: SQ_ERR_ARG (null, bits out of range), SQ_ERR_UNSUPPORTED (head_dim).
 */
sq_status sq_calibrate_tq(const float *rotation, const float *qjl_gauss, int n_heads,
                          const sq_calib_opts *opts, sq_calib **out);

/* Copy the handle's tables to the current HIP device (enqueued on `stream`,
 * which is synchronised before return).  Device memory is owned by the handle.
 * Must be called before any device call that uses the handle. */
sq_status sq_calib_upload(sq_calib *c, sq_stream stream);

int sq_calib_n_heads(const sq_calib *c);
sq_status sq_calib_info(const sq_calib *c, int head, sq_head_info *info);

/* Export one head's artifact to HOST buffers (any pointer may be NULL):
 * eigenvalues double[d], rotation double[d*d] (row i = eigenvector i),
 * widths int32[d], thresholds float[n_thresholds] and centroids
 * float[n_centroids] (concatenated in coordinate order, ascending within a
 * coordinate, already scaled by sqrt(l_i)), qjl float[m*d_eff] row-major. */
sq_status sq_calib_export(const sq_calib *c, int head, double *eigenvalues,
                          double *rotation, int32_t *widths, float *thresholds,
                          float *centroids, float *qjl);

/* Versioned little-endian file of the whole handle (host tables only). */
sq_status sq_calib_save(const sq_calib *c, const char *path);
sq_status sq_calib_load(const char *path, sq_calib **out);
void sq_calib_destroy(sq_calib *c);

/* Minimum per-head slot size, in 32-bit words, for n_tokens tokens: the
 * largest W over the handle's heads times n_tokens rounded up to 64. */
int64_t sq_packed_head_words(const sq_calib *c, int64_t n_tokens);

/*
 * sq_compress -- spectral rotation, per-coordinate Lloyd-Max quantisation,
 * selective QJL on the signal dims (keys) and bit-dense packing
 * (README "Repository Structure": spectral_rotation, nonuniform_quantization,
 * selective_qjl).  Vector (b, h, t), h in [0, n_heads), uses calibration head
 * first_head + b*calib_batch_stride + h.
 * x       DEVICE, dtype dt, element (b,h,t,i) at b*xs_batch + h*xs_head +
 *         t*xs_token + i (strides in elements; the last dim is contiguous).
 * packed  DEVICE uint32, slot of (b,h) at b*ps_batch + h*ps_head (words);
 *         ps_head >= sq_packed_head_words(c, n_tokens).  Every word of the
 *         ceil(T/64)*64-token range is written (pad tokens as zeros).
 * n_tokens == 0 or batch == 0 is a no-op.
 * Quantiser: code = #{thresholds < y} by a uniform-grid table per region
 * (one cell read and one compare per value) when the calibration's grid
 * tables exist (head_dim <= 128, at most 16 signal dims and 32 QJL rows, at
 * most 6144 cells per head), else by a descent of padded threshold trees;
 * both give the same codes.  Normalised calibrations take the grid path for
 * bf16 input into contiguous slots, the general kernel otherwise.
 * The environment variable SQ_QUANTISER=tree forces the trees (a test hook).
 */
sq_status sq_compress(const sq_calib *c, int first_head, int n_heads, int batch,
                      int calib_batch_stride, const void *x, sq_dtype dt,
                      int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                      int64_t xs_token, uint32_t *packed, int64_t ps_batch,
                      int64_t ps_head, sq_stream stream);

/*
 * Paged packed cache (the decode-time cache layout of serving engines: the
 * sequences of a batch share a pool of fixed-size blocks handed out as they
 * grow).  A block holds block_tiles 64-token tiles of every head of a call;
 * logical block j of batch row b (its tiles j*block_tiles ..) is physical
 * block block_table[b * table_stride + j] of the pool, whose head h (0 <= h <
 * n_heads of the call) takes the words [(block * n_heads + h) * block_words,
 * + block_words) with block_words = sq_paged_block_words(c, block_tiles);
 * tile i of a block starts i * 64 * W words in, in the word-interleaved
 * record layout of the contiguous slots.  Block ids are the caller's; an id
 * outside [0, n_blocks) is never dereferenced (its writes are dropped, its
 * reads take the first or last block instead).
 */
typedef struct {
  const int32_t *block_table;  /* DEVICE int32 [batch][table_stride] */
  int64_t table_stride;        /* >= the logical blocks a call touches */
  int32_t block_tiles;         /* 64-token tiles per block, >= 1 */
  int32_t n_blocks;            /* physical blocks in the pool, >= 1 */
} sq_paged;

/* Words per (block, head) of a pool for this handle: block_tiles * 64 * W_max. */
int64_t sq_paged_block_words(const sq_calib *c, int block_tiles);

/*
 * sq_compress_append -- sq_compress of n_tokens new vectors into token slots
 * token0 .. token0 + n_tokens - 1 of an existing packed cache: the decode-time
 * producer of the compressed cache (SpectralQuant README "Overview": the
 * method compresses the KV cache during inference; TurboQuant reference
 * implementation page, "Key Findings" 5, "Compressed Storage": records are
 * kept compressed, not simulated).  The record of a token depends only on
 * its own vector, so appending in pieces gives the same words as one
 * sq_compress over the whole sequence.
 * x       DEVICE, as in sq_compress; token i of x is cache token token0 + i.
 * packed  DEVICE, as in sq_compress; ps_head >=
 *         sq_packed_head_words(c, token0 + n_tokens).  Written: the words of
 *         tokens token0 .. token0 + n_tokens - 1, and zeros for the tokens
 *         after them up to the end of their 64-token tile.  Tokens below
 *         token0 and tiles past the last one are not touched.
 * token0  >= 0, any alignment.  token0 == 0 is exactly sq_compress.
 * Errors: token0 < 0 -> SQ_ERR_ARG; otherwise as sq_compress.
 */
sq_status sq_compress_append(const sq_calib *c, int first_head, int n_heads,
                             int batch, int calib_batch_stride, const void *x,
                             sq_dtype dt, int64_t n_tokens, int64_t xs_batch,
                             int64_t xs_head, int64_t xs_token,
                             uint32_t *packed, int64_t ps_batch,
                             int64_t ps_head, int64_t token0,
                             sq_stream stream);

/*
 * sq_compress_append_paged -- sq_compress_append into a paged cache (layout
 * above): the words of tokens token0 .. token0 + n_tokens - 1 of batch row b,
 * head h go to their tiles' blocks, with the same zero fill to the end of
 * the last tile.  The record words equal those of sq_compress_append.
 * pool    DEVICE uint32, n_blocks * n_heads * sq_paged_block_words(c, block_tiles) words.
 * pg      HOST pointer to the block table description (the table is DEVICE).
 * Errors: as sq_compress_append; SQ_ERR_ARG for a NULL pg, table or pool,
 * block_tiles or n_blocks < 1, or table_stride below the logical blocks of
 * token0 + n_tokens tokens.
 */
sq_status sq_compress_append_paged(const sq_calib *c, int first_head, int n_heads,
                                   int batch, int calib_batch_stride, const void *x,
                                   sq_dtype dt, int64_t n_tokens, int64_t xs_batch,
                                   int64_t xs_head, int64_t xs_token, uint32_t *pool,
                                   const sq_paged *pg, int64_t token0, sq_stream stream);

/*
 * sq_scores -- raw q.k scores read from the packed keys (no softmax scale).
 * SpectralQuant README "Overview" (decode-time attention reads the compressed
 * keys: the query is rotated into the calibrated basis once and scored against
 * the codes) and "Repository Structure" (selective_qjl: the QJL correction on
 * the signal dims); the sign-sketch inner-product estimator with factor
 * sqrt(pi/2)/m is the QJL estimator (TurboQuant reference-implementation page,
 * "Project Structure", the Prod quantiser's QJL stage).
 * The query of each query head is rotated once, q~ = R q; then
 *   s_t = sum_i q~_i C_i[code_ti] + sqrt(pi/2)/m * gamma_t * sum_j w_j (2 z_tj - 1),
 * w = S q~[0:d_eff].  Query head hq of batch b reads KV head
 * hq / (n_q_heads / n_kv_heads) of batch b (contiguous GQA groups).
 * q       DEVICE [batch][n_q_heads][head_dim], dtype qdt, contiguous.
 * kpacked DEVICE slots as in sq_compress (ps_batch, ps_head in words).
 * scores  DEVICE float [batch][n_q_heads][n_tokens].
 * Errors: n_q_heads % n_kv_heads != 0, group size > 8 -> SQ_ERR_ARG / UNSUPPORTED.
 */
sq_status sq_scores(const sq_calib *kc, int first_head, int calib_batch_stride,
                    int batch, int n_q_heads, int n_kv_heads, const void *q,
                    sq_dtype qdt, const uint32_t *kpacked, int64_t ps_batch,
                    int64_t ps_head, int64_t n_tokens, float *scores,
                    sq_stream stream);

/* Workspace bytes sq_attend needs for these sizes. */
size_t sq_attend_workspace_bytes(int batch, int n_q_heads, int64_t n_tokens,
                                 int head_dim);

/*
 * sq_attend -- o = sum_t softmax(scale * s)_t * v~_t for every (b, hq), where v~
 * is the dequantised value (R_v^T C[code]).  SpectralQuant README "Overview"
 * (values are dequantised for the attention-weighted sum; no QJL on values:
 * TurboQuant reference-implementation page, "Key Findings" 2, MSE quantiser
 * for values).  Softmax is max-subtracted; the sum is formed in the rotated
 * value space and un-rotated once (R_v^T is linear).  Split over token chunks with
 * (max, sum exp, partial sum) partials in `workspace`, then an ordered
 * (deterministic) combine and one un-rotation per (b, hq).
 * scores  DEVICE float [batch][n_q_heads][n_tokens] (e.g. from sq_scores).
 * vpacked DEVICE value slots as in sq_compress.
 * workspace DEVICE, ws_bytes >= sq_attend_workspace_bytes(...).
 * out     DEVICE float [batch][n_q_heads][head_dim].
 * n_tokens == 0 writes zeros.
 */
sq_status sq_attend(const sq_calib *vc, int first_head, int calib_batch_stride,
                    int batch, int n_q_heads, int n_kv_heads, const float *scores,
                    float scale, const uint32_t *vpacked, int64_t ps_batch,
                    int64_t ps_head, int64_t n_tokens, void *workspace,
                    size_t ws_bytes, float *out, sq_stream stream);

/*
 * sq_decode -- the fused decode step: for every (b, hq),
 *   o = sum_t softmax(scale * s)_t v~_t,  s_t the score sq_scores gives,
 * computed in one pass over the packed keys and values with no score tensor
 * in device memory (SpectralQuant README "Overview": decode-time attention
 * over the compressed cache; "Headline Results": the per-step decode
 * latency).  Each key record is read once by the lane of its token; its
 * code fields are cut into groups of at most 6 bits (a wider field alone),
 * and per (batch, KV head) the query group's tables of every group's
 * contribution (sum of q~_i C_i[code] over the group's coordinates, and the
 * QJL term sqrt(pi/2)/m sum_j w_j (2 z_j - 1) of the sign bits) are built
 * once in LDS in fp32, so a score costs one table read per group.  Then the
 * online softmax and the value sum of sq_attend; split over token chunks with
 * the same (max, sum exp, partial sum) partials and ordered combine.
 * q        DEVICE [batch][n_q_heads][head_dim], dtype qdt, contiguous.
 * kpacked  DEVICE key slots (kps_batch, kps_head words), as from sq_compress
 *          with kc; vpacked likewise for vc.  Head (b, h) of both handles is
 *          first_head + b * calib_batch_stride + h.
 * workspace DEVICE, ws_bytes >= sq_attend_workspace_bytes(batch, n_q_heads,
 *          n_tokens, head_dim).
 * out      DEVICE float [batch][n_q_heads][head_dim].  n_tokens == 0 writes zeros.
 * Errors: as sq_scores and sq_attend; SQ_ERR_UNSUPPORTED (nothing enqueued;
 * use sq_scores + sq_attend then) when a key record exceeds 32 words, a key
 * head has more than 16 QJL bits (e.g. the TurboQuant-style keys, m = d) or a
 * record word in which more than 8 code groups start, the query group is
 * larger than 8, or the score tables and staging do not fit the LDS.
 */
sq_status sq_decode(const sq_calib *kc, const sq_calib *vc, int first_head,
                    int calib_batch_stride, int batch, int n_q_heads, int n_kv_heads,
                    const void *q, sq_dtype qdt, const uint32_t *kpacked,
                    int64_t kps_batch, int64_t kps_head, const uint32_t *vpacked,
                    int64_t vps_batch, int64_t vps_head, int64_t n_tokens, float scale,
                    void *workspace, size_t ws_bytes, float *out, sq_stream stream);

/*
 * sq_decode_paged -- sq_decode over paged key and value caches that share
 * one block table (layout above; kpool's block_words from kc, vpool's from
 * vc).  The result equals sq_decode's over the same records in contiguous
 * slots, bit for bit.
 * Errors: as sq_decode; SQ_ERR_ARG for a NULL pg, table or pool, block_tiles
 * or n_blocks < 1, or table_stride below the logical blocks of n_tokens.
 */
sq_status sq_decode_paged(const sq_calib *kc, const sq_calib *vc, int first_head,
                          int calib_batch_stride, int batch, int n_q_heads, int n_kv_heads,
                          const void *q, sq_dtype qdt, const uint32_t *kpool,
                          const uint32_t *vpool, const sq_paged *pg, int64_t n_tokens,
                          float scale, void *workspace, size_t ws_bytes, float *out,
                          sq_stream stream);

/*
 * sq_attend_noalloc -- sq_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same result, with the split-T
 * partials in the library's fixed device scratch instead of a caller
 * workspace.  The scratch is a SQ_NOALLOC_SCRATCH_BYTES (32 MiB) array that
 * each GPU the library runs on holds until the process ends; calls that need
 * more (sq_attend_workspace_bytes of the same sizes above the limit) fail
 * with SQ_ERR_UNSUPPORTED before anything is enqueued.  The call allocates
 * nothing.  All calls on one GPU share its array, so calls that overlap in
 * time on one GPU (different streams) race; calls in stream order do not.
 * Arguments, layout and errors otherwise as sq_attend.
 */
#define SQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
sq_status sq_attend_noalloc(const sq_calib *vc, int first_head, int calib_batch_stride,
                            int batch, int n_q_heads, int n_kv_heads, const float *scores,
                            float scale, const uint32_t *vpacked, int64_t ps_batch,
                            int64_t ps_head, int64_t n_tokens, float *out, sq_stream stream);

/*
 * sq_plan_decode -- diagnostic: how sq_scores (keys handle kc) and sq_attend
 * (values handle vc) would launch for these arguments on the current device,
 * without launching anything.  Either handle may be NULL (its fields stay 0).
 *   score_passes       launches of the scores kernel (passes over the quads of
 *                      4 coordinates; passes after the first add into scores)
 *   score_quads        the largest number of quads of one head
 *   score_wave_groups  wave groups the quads are split over
 *   attend_placement   centroid tables: 0 one column per lane in LDS, 1 packed
 *                      in LDS, 2 read from device memory
 *   attend_waves       waves (token chunks) per workgroup
 *   attend_blocks      64-coordinate blocks each wave serves (head_dim / 64)
 *   attend_chunks      token chunks per (batch, query head)
 *   decode_launches    launches of the fused kernel (query heads served four
 *                      at a time), decode_waves its waves per workgroup,
 *                      decode_lds_bytes its LDS per workgroup
 * Errors: as sq_scores / sq_attend for the head range; SQ_ERR_STATE when a
 * handle is not uploaded.
 */
typedef struct {
  int score_passes, score_quads, score_wave_groups;
  int attend_placement, attend_waves, attend_blocks, attend_chunks;
  int decode_launches, decode_waves, decode_lds_bytes;  /* sq_decode (both handles given) */
} sq_decode_plan;
sq_status sq_plan_decode(const sq_calib *kc, const sq_calib *vc, int first_head,
                         int calib_batch_stride, int batch, int n_q_heads, int n_kv_heads,
                         int64_t n_tokens, sq_decode_plan *out);

/*
 * sq_dequantize -- diagnostic: x~ = R^T (C[code] + pad_d(sqrt(pi/2)/m * gamma *
 * S^T (2z-1))) for every packed vector: the reconstruction the scores see
 * (SpectralQuant README "Headline Results": per-vector cosine similarity of
 * the reconstruction; "Repository Structure", metrics.py).
 * out DEVICE float [batch][n_heads][n_tokens][head_dim].
 */
sq_status sq_dequantize(const sq_calib *c, int first_head, int n_heads, int batch,
                        int calib_batch_stride, const uint32_t *packed,
                        int64_t ps_batch, int64_t ps_head, int64_t n_tokens,
                        float *out, sq_stream stream);

/*
 * sq_unpack -- HOST decode of one head's slot (for tests and tools).
 * packed HOST uint32 slot of calibration head `head`; codes uint8 [T][d],
 * qjl uint8 [T][m] (may be NULL when m == 0), gamma float [T] (may be NULL),
 * nu float [T] (vector norms of a normalised calibration, else 0; may be NULL).
 */
sq_status sq_unpack(const sq_calib *c, int head, const uint32_t *packed,
                    int64_t n_tokens, uint8_t *codes, uint8_t *qjl, float *gamma,
                    float *nu);

/* Message of the last error on the calling thread ("" if none). */
const char *sq_last_error(void);

/* Digest of the sources this library was built from (16 hex digits of a
 * SHA-256 over the library's source files and this header); the Python
 * binding refuses a library whose digest differs from its sources. */
const char *sq_build_digest(void);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
