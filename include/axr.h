/*
 * axr.h -- C ABI of the AXELRAM-style LUT attention-scoring library for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638),
 * Abstract.  Keys are transformed once on write by an orthogonal transform
 * (a seeded sign pattern followed by a normalised Walsh-Hadamard transform)
 * and scalar-quantized against a design-time codebook that depends only on
 * the head dimension d and bit width b; queries are scored on read by table
 * lookup, with no inverse transform.
 *
 * Conventions shared by every call
 *   - All functions have C linkage, return an axr_status (0 = success) and
 *     never throw.  On failure axr_last_error() returns a message describing
 *     the most recent failure on the calling thread.
 *   - Arguments are validated before any HIP call, so a rejected call leaves
 *     the device untouched.
 *   - Device buffers are allocated, owned and freed by the caller.  The
 *     library allocates no device memory; it keeps only a process-wide cache
 *     of codebooks keyed by (d, b).
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t cast
 *     to void*; NULL means the default stream).  Launch failures are reported
 *     as AXR_EHIP; faults during execution surface at the caller's next
 *     synchronisation.  The library never synchronises.
 *   - Sign pattern: `sign_bits` is a HOST array of d/32 uint32 words; bit
 *     (j % 32) of word (j / 32) set means s_j = -1, clear means s_j = +1.
 *     The words are copied into kernel arguments; the array may be reused as
 *     soon as the call returns.
 *   - Packed index record of one key: d*b bits, little-endian bit stream:
 *     bit r of idx_j is record bit j*b + r, record bit m is bit (m % 32) of
 *     32-bit word (m / 32).  W = d*b/32 words per key, keys contiguous.
 *   - Supported: d in {128, 256, 512}, b in {2, 3, 4} (axr_codebook also
 *     accepts b = 1 and any d >= 1).
 */
#ifndef AXR_H
#define AXR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum axr_status {
  AXR_OK = 0,
  AXR_EINVAL = -1,       /* null pointer, negative size, inconsistent shape   */
  AXR_EUNSUPPORTED = -2, /* d, b, dtype or head layout outside what is built  */
  AXR_EALIGN = -3,       /* a device pointer is not aligned as required       */
  AXR_EHIP = -4          /* the HIP runtime reported an error                 */
} axr_status;

typedef enum axr_dtype { AXR_F32 = 0, AXR_F16 = 1, AXR_BF16 = 2 } axr_dtype;

/* Library version, as major*10000 + minor*100 + patch. */
int axr_version(void);

/* Message for the last non-OK return on the calling thread ("" if none).
 * The pointer stays valid until the next axr_* call on that thread. */
const char* axr_last_error(void);

/*
 * Design-time codebook (AXELRAM, Abstract: the optimal quantizer depends only
 * on d and b).  Host only, no HIP call.  Computes the Lloyd-Max quantizer for
 * the density N(0, 1/d): 2^b centroids and 2^b - 1 thresholds, each threshold
 * the midpoint of its neighbouring centroids and each centroid the mean of
 * N(0, 1/d) over its cell.  The quantizer is symmetric; the middle threshold
 * is exactly 0.
 *   centroids  : host double[2^b], written ascending
 *   thresholds : host double[2^b - 1], written ascending
 * Errors: AXR_EINVAL for d < 1, b outside [1, 4] or a null pointer.
 */
int axr_codebook(int d, int b, double* centroids, double* thresholds);

/*
 * Write path (AXELRAM, Abstract: transform on write, quantize once).
 * For each of the n keys k (rows of `keys`):
 *   ||k|| is stored in norms[i] (fp32, accumulated in fp32; a key whose
 *   squared entries underflow or overflow fp32 takes it from its
 *   transformed coordinates scaled by 2^64 or 2^-64, so keys keep full
 *   precision from fp32 denormal entries up to ~1e36);
 *   y = H_d (s * k) / (sqrt(d) ||k||)       (y = 0 for a zero key);
 *   idx_j = number of codebook thresholds strictly below y_j, in [0, 2^b);
 *   the indices are packed into packed[i*W .. i*W + W) as described above.
 *   keys   : device, n x d elements of `dtype`, row-major, 16-byte aligned
 *   packed : device uint32 [n][W], 16-byte aligned
 *   norms  : device float [n], 4-byte aligned
 * n = 0 is a no-op.  Keys of a [B][Hkv][T][d] cache are simply n = B*Hkv*T
 * consecutive rows.  Errors: AXR_EINVAL, AXR_EUNSUPPORTED, AXR_EALIGN,
 * AXR_EHIP.  Decisions are taken in fp32: a coordinate whose exact value lies
 * within ~1e-7 (relative) of a threshold may fall in the neighbouring cell.
 */
int axr_quantize_keys(const void* keys, int dtype, int64_t n, int d, int b,
                      const uint32_t* sign_bits, uint32_t* packed, float* norms,
                      void* stream);

/*
 * Read path (AXELRAM, Abstract: table lookup on read, no inverse transform).
 * For batch bi, query head h (KV head kvh = h / (Hq / Hkv)) and token t < T:
 *   q' = H_d (s * q[bi][h]) / sqrt(d)                 (queries not normalised)
 *   LUT[j][c] = q'_j * centroid_c
 *   scores[bi][h][t] = norms[r] * sum_j LUT[j][idx_j(r)],  r = (bi*Hkv + kvh)*t_cap + t
 * Table entries hold the summed products of a group of coordinates: two
 * (four for b = 2 at d = 128; one where the pair table would not fit in
 * LDS: b = 4 at d = 256 and 512).  Their sum
 * is taken exactly in 32-bit fixed point, each coordinate term rounded to a
 * unit of a per-head scale that puts sum_j |q'_j| max_c |centroid_c| in
 * [2^30, 2^31) units: the error is at most d/2 units, i.e. at most
 * (d/2) * 1.0001 * (max|c| / min|c|) / 2^30 of norms * sum_j |LUT[j][idx_j]|
 * (max|c| / min|c| = 3.34, 8.78, 21.3 for b = 2, 3, 4): 2.0e-7, 5.2e-7 at
 * d = 128 (b = 2, 3); 4.0e-7, 1.0e-6, 2.5e-6 at d = 256; 8.0e-7, 2.1e-6,
 * 5.1e-6 at d = 512 (b = 2, 3, 4), plus ~1e-7 for the final fp32 products.
 * At d = 128, b = 4 the entries are fp32 (the pair table is stored for half
 * the field values, see the score kernel), summed in fp32: at most ~20 fp32
 * roundings, ~1.2e-6 of the same scale.  Every case is inside 1e-5.
 *   q       : device, [B][Hq][d] of q_dtype, 16-byte aligned
 *   packed  : device uint32, [B][Hkv][t_cap][W] as written by axr_quantize_keys
 *   norms   : device float, [B][Hkv][t_cap]
 *   scores  : device float, [B][Hq][T] (output), 4-byte aligned
 *   t_cap   : tokens allocated per (batch, KV head) row, t_cap >= T (pass T
 *             for a dense cache)
 * Requires Hq % Hkv == 0, Hq / Hkv <= 64 and T * d * b / 8 < 2^31 (the
 * records of one row are addressed with 32-bit offsets).  T = 0 or B = 0 is a
 * no-op.  Errors: AXR_EINVAL, AXR_EUNSUPPORTED, AXR_EALIGN, AXR_EHIP.
 */
int axr_score(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
              const uint32_t* sign_bits, int B, int Hq, int Hkv, int64_t T, int64_t t_cap,
              int d, int b, float* scores, void* stream);

/*
 * Decode-step write (AXELRAM, Abstract: each key is quantized once, when it is
 * written).  Quantizes one new key per (sequence, KV head) exactly as
 * axr_quantize_keys does and stores its record and norm in a cache laid out
 * [B][Hkv][t_cap] (records of W words, as above):
 *   key (bi, h) -> packed row (bi*Hkv + h)*t_cap + pos[bi], norms likewise.
 *   keys   : device, [B][Hkv][d] of `dtype`, 16-byte aligned
 *   pos    : device int32 [B], the slot of each sequence's new token; a
 *            sequence whose pos lies outside [0, t_cap) is skipped (nothing
 *            is written for it)
 *   packed : device uint32 [B][Hkv][t_cap][W], 16-byte aligned (in/out: only
 *            the appended slots are written)
 *   norms  : device float [B][Hkv][t_cap], 4-byte aligned (in/out)
 * B = 0 or Hkv = 0 is a no-op.  Requires t_cap >= 1 and B*Hkv < 2^31.
 * Errors: AXR_EINVAL, AXR_EUNSUPPORTED, AXR_EALIGN, AXR_EHIP.
 */
int axr_append_keys(const void* keys, int dtype, int B, int Hkv, int d, int b,
                    const uint32_t* sign_bits, const int32_t* pos, int64_t t_cap,
                    uint32_t* packed, float* norms, void* stream);

/*
 * Read path over sequences of different lengths (AXELRAM, Abstract: table
 * lookup on read).  As axr_score, but batch row bi scores only tokens
 * t < min(max(lens[bi], 0), T); scores[bi][h][t] for later t are not written.
 *   lens : device int32 [B], 4-byte aligned
 *   T    : row length of `scores` ([B][Hq][T]) and the largest length scored
 * Same requirements and errors as axr_score (lens must be non-null when B > 0
 * and T > 0).
 */
int axr_score_ragged(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                     const uint32_t* sign_bits, int B, int Hq, int Hkv, const int32_t* lens,
                     int64_t T, int64_t t_cap, int d, int b, float* scores, void* stream);

/*
 * One decode step in one launch: the effect of axr_append_keys(k_new, pos)
 * followed by axr_score_ragged(lens = pos + 1).  The block of the score
 * kernel whose tile holds slot pos[bi] quantizes the new key itself (same
 * rule as the write path; its arithmetic runs in a different order, so a
 * coordinate within ~1e-7 of a threshold may take the neighbouring cell and
 * the stored norm may differ in the last bits), stores its record and norm in
 * the cache and scores it from the fresh record.
 *   k_new : device [B][Hkv][d] of k_dtype, 4-byte aligned
 *   pos   : device int32 [B]; a slot outside [0, t_cap) appends nothing and
 *           row bi is scored for t < min(max(pos[bi] + 1, 0), T); a slot in
 *           [T, t_cap) is appended (by the row's last tile) but not scored,
 *           and with T = 0 the call is the append alone
 *   packed, norms : the cache, as for axr_append_keys (in/out)
 *   scores: device float [B][Hq][T]; entries past a row's length are not written
 * Same requirements and errors as axr_score.
 */
int axr_decode_step(const void* q, int q_dtype, const void* k_new, int k_dtype,
                    const uint32_t* sign_bits, const int32_t* pos, int B, int Hq, int Hkv,
                    int64_t T, int64_t t_cap, int d, int b, uint32_t* packed, float* norms,
                    float* scores, void* stream);

/*
 * Write and read path in one launch (AXELRAM, Abstract: each key is
 * transformed and quantized once on write; a query is scored by table lookup
 * on the stored indices).  The effect of axr_quantize_keys over the n =
 * B*Hkv*T keys of a dense cache followed by axr_score(t_cap = T): records,
 * norms and scores are bit for bit those two calls' results.  Each block of
 * the score kernel quantizes the keys of its tile with the write path's
 * arithmetic, stores their records and norms, and scores them from
 * registers, so the records are never read back.
 *   keys   : device [B][Hkv][T][d] of k_dtype, 16-byte aligned
 *   q      : device [B][Hq][d] of q_dtype, 16-byte aligned
 *   packed : device uint32 [B][Hkv][T][W] (output), 16-byte aligned
 *   norms  : device float [B][Hkv][T] (output), 4-byte aligned
 *   scores : device float [B][Hq][T] (output), 4-byte aligned
 * Built for d = 128, b = 2 or 3 with Hq / Hkv <= 4 (one table per (batch, KV
 * head) row), and for Hq / Hkv = 8 at b = 3 (two tables in one block); each
 * key is quantized by exactly one block.  Other shapes return
 * AXR_EUNSUPPORTED (use the two calls).
 * Same further requirements as axr_score, plus T * d * sizeof(key) < 2^31.
 * B = 0 or T = 0 is a no-op.  Errors: AXR_EINVAL, AXR_EUNSUPPORTED,
 * AXR_EALIGN, AXR_EHIP.
 */
int axr_quantize_score(const void* keys, int k_dtype, const void* q, int q_dtype,
                       const uint32_t* sign_bits, int B, int Hq, int Hkv, int64_t T, int d,
                       int b, uint32_t* packed, float* norms, float* scores, void* stream);

/*
 * Attention probabilities over the table-lookup scores, with the context split
 * across blocks.  The pages define the scores (AXELRAM, Abstract: score =
 * norm times the sum of table entries); the softmax over a row is the usual
 * normalisation that turns such scores into attention weights.  For batch
 * row bi, query head h and t < len(bi) = min(max(lens[bi], 0), T) (len = T
 * when lens is NULL):
 *   probs[bi][h][t] = exp(scale*s_t - M) / L,  M = max_t scale*s_t,
 *   L = sum_t exp(scale*s_t - M),  lse[bi][h] = M + log L,
 * where s is what axr_score(_ragged) returns; probs[bi][h][t] for t >= len
 * is not written, and an empty row gets lse = -inf.  Each tile of a row
 * leaves (max, sum of exps) in `workspace`; a second kernel merges them and
 * normalises the row in place.
 *   scale     : finite multiplier of the scores (1/sqrt(d) for scaled
 *               dot-product attention)
 *   probs     : device float [B][Hq][T] (output), 4-byte aligned
 *   lse       : device float [B][Hq] or NULL
 *   workspace : device memory of at least the size axr_score_softmax_workspace
 *               reports for the same (B, Hq, Hkv, T, d, b), 8-byte aligned;
 *               owned by the caller, contents on entry are ignored
 * Otherwise as axr_score_ragged.  Errors: AXR_EINVAL (also for a workspace
 * that is too small or a non-finite scale), AXR_EUNSUPPORTED, AXR_EALIGN,
 * AXR_EHIP.
 */
int axr_score_softmax_workspace(int B, int Hq, int Hkv, int64_t T, int d, int b,
                                int64_t* bytes);
int axr_score_softmax(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                      const uint32_t* sign_bits, int B, int Hq, int Hkv, const int32_t* lens,
                      int64_t T, int64_t t_cap, int d, int b, float scale, float* probs,
                      float* lse, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * axr_score_softmax without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The split-T partials go to a device array that the
 * library holds, 1 MiB per device, allocated with the library's code object
 * and kept until the process ends; this call allocates nothing.  Every call
 * on a device uses that device's array: calls that overlap on one device
 * (other streams, other threads) race on it and must be serialised by the
 * caller.  The array needs no clearing (every partial the second kernel
 * reads is written by the first).  Sizes whose partials
 * (B * Hq * tiles * 8 bytes, as axr_score_softmax_workspace reports) exceed
 * 1 MiB are rejected with AXR_EUNSUPPORTED before any device work.  Otherwise
 * arguments, results and errors are those of axr_score_softmax.
 */
int axr_score_softmax_noalloc(const void* q, int q_dtype, const uint32_t* packed,
                              const float* norms, const uint32_t* sign_bits, int B, int Hq,
                              int Hkv, const int32_t* lens, int64_t T, int64_t t_cap, int d,
                              int b, float scale, float* probs, float* lse, void* stream);

/*
 * One-time sign-pattern selection (AXELRAM, Abstract: gradient-free, a few
 * hundred candidate sign patterns, a few calibration samples, chosen once).
 * The pages rank candidates by perplexity, which needs model weights; this
 * call measures instead how far the table scores are from the exact scores.
 * For candidate c (sign words candidates[c*d/32 .. c*d/32 + d/32), HOST) and
 * calibration sample i, the calibration keys are quantized with that pattern
 * and scored against the sample's queries, and
 *   errors[(c*S + i)*2 + 0] = sum (s_lut - s_exact)^2
 *   errors[(c*S + i)*2 + 1] = sum s_exact^2
 * over every (batch, query head, token) of the sample, accumulated in fp64
 * (s_exact = q . k in fp32).  axr_sign_selection_choose turns these sums into
 * the choice.
 *   keys      : device [S][B][Hkv][T][d] of `dtype`, 16-byte aligned
 *   q         : device [S][B][Hq][d] of `q_dtype`, 16-byte aligned
 *   errors    : device double [C][S][2], 8-byte aligned
 *   workspace : device memory of the size axr_sign_selection_workspace
 *               reports, 256-byte aligned, owned by the caller
 * C, S, B or T = 0 is a no-op; S <= 64.  Same size limits as axr_score.  Errors:
 * AXR_EINVAL, AXR_EUNSUPPORTED, AXR_EALIGN, AXR_EHIP.
 */
int axr_sign_selection_workspace(int S, int B, int Hq, int Hkv, int64_t T, int d, int b,
                                 int64_t* bytes);
int axr_sign_selection_errors(const void* keys, int dtype, const void* q, int q_dtype, int S,
                              int B, int Hq, int Hkv, int64_t T, int d, int b,
                              const uint32_t* candidates, int C, double* errors,
                              void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Choice rule of the sign-pattern selection (AXELRAM, Abstract: the pattern
 * is chosen once, gradient-free, from the candidates' results on the
 * calibration samples).  Host only, no HIP call.  For candidate c the
 * objective is its worst sample's relative score error,
 *   objective[c] = max_i sqrt(err_ci / ref_ci),
 *   err_ci = errors[(c*S + i)*2 + 0],  ref_ci = errors[(c*S + i)*2 + 1],
 * where a sample with ref_ci = 0 (no exact score mass, e.g. a zero query)
 * counts 0 if err_ci = 0 and +inf otherwise; *index receives the candidate
 * with the smallest objective, the first one on ties.
 *   errors    : HOST double [C][S][2], as axr_sign_selection_errors writes them
 *               (copied to the host by the caller)
 *   index     : HOST int (output)
 *   objective : HOST double [C] (output), or NULL
 * Errors: AXR_EINVAL for C < 1, S < 1, a null errors or index pointer, or a
 * negative or NaN sum (nothing is written then).
 */
int axr_sign_selection_choose(const double* errors, int C, int S, int* index,
                              double* objective);

/*
 * Comparison write path with block-quaternion rotations in place of the sign
 * pattern + Walsh-Hadamard transform ("IsoQuant: Hardware-Aligned SO(4)
 * Isoclinic Rotations for LLM KV Cache Compression", arXiv 2603.28430,
 * Abstract): coordinates 4m..4m+3 of the unit key form the quaternion
 * v = (w, x, y, z) and become q_L[m] v conj(q_R[m]) (full = 1) or q_L[m] v
 * (full = 0); the result is quantized with the same Lloyd-Max codebook and
 * packed in the same layout, norms as in axr_quantize_keys.
 *   quats : device float [d/4][2][4], (q_L, q_R) of each block as (w, x, y, z),
 *           unit length, 16-byte aligned (q_R unused when full = 0)
 * Otherwise as axr_quantize_keys / axr_transform (y = T(x), divided by ||x||
 * when normalize != 0).  These scores need queries rotated the same way
 * (axr_score applies the Walsh-Hadamard transform and does not apply here).
 */
int axr_quantize_keys_isoquant(const void* keys, int dtype, int64_t n, int d, int b,
                               const float* quats, int full, uint32_t* packed, float* norms,
                               void* stream);
int axr_transform_isoquant(const void* x, int dtype, int64_t n, int d, const float* quats,
                           int full, int normalize, float* y, void* stream);

/*
 * Diagnostic export of the write-path transform (the same device code the
 * quantizer runs): y[i] = H_d (s * x[i]) / sqrt(d), divided by ||x[i]|| when
 * normalize != 0 (y = 0 for a zero row).
 *   x : device, n x d elements of `dtype`, 16-byte aligned
 *   y : device float [n][d], 16-byte aligned
 * Errors: AXR_EINVAL, AXR_EUNSUPPORTED, AXR_EALIGN, AXR_EHIP.
 */
int axr_transform(const void* x, int dtype, int64_t n, int d, const uint32_t* sign_bits,
                  int normalize, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AXR_H */
