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
 *   - W = max(1, ceil((sum b_i + m + 16*[m>0]) / 32)); unused bits are zero;
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
} sq_head_info;

/* Defaults: avg_bits 3, qjl 1 (keys), max_bits 8, 200 Lloyd-Max iterations. */
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
 *   2. d_eff = round-half-even(PR), PR = (sum l)^2 / sum l^2; kappa.
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
 */
sq_status sq_compress(const sq_calib *c, int first_head, int n_heads, int batch,
                      int calib_batch_stride, const void *x, sq_dtype dt,
                      int64_t n_tokens, int64_t xs_batch, int64_t xs_head,
                      int64_t xs_token, uint32_t *packed, int64_t ps_batch,
                      int64_t ps_head, sq_stream stream);

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
 * sq_scores -- raw q.k scores read from the packed keys (no softmax scale).
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
 * is the dequantised value (R_v^T C[code]).  Split over token chunks with
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
 * sq_dequantize -- diagnostic: x~ = R^T (C[code] + pad_d(sqrt(pi/2)/m * gamma *
 * S^T (2z-1))) for every packed vector.
 * out DEVICE float [batch][n_heads][n_tokens][head_dim].
 */
sq_status sq_dequantize(const sq_calib *c, int first_head, int n_heads, int batch,
                        int calib_batch_stride, const uint32_t *packed,
                        int64_t ps_batch, int64_t ps_head, int64_t n_tokens,
                        float *out, sq_stream stream);

/*
 * sq_unpack -- HOST decode of one head's slot (for tests and tools).
 * packed HOST uint32 slot of calibration head `head`; codes uint8 [T][d],
 * qjl uint8 [T][m] (may be NULL when m == 0), gamma float [T] (may be NULL).
 */
sq_status sq_unpack(const sq_calib *c, int head, const uint32_t *packed,
                    int64_t n_tokens, uint8_t *codes, uint8_t *qjl, float *gamma);

/* Message of the last error on the calling thread ("" if none). */
const char *sq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
