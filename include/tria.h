/*
 * tria.h -- C ABI of the TriAttention KV-cache prune step on AMD MI355X (gfx950).
 *
 * The prune step, per stream (one sequence s, one layer l, one KV head g) of N cached keys:
 *   1. score every cached key for each of the G query heads that share the KV head with the
 *      trigonometric-series score plus the (1-R)-weighted norm score, future offsets averaged;
 *   2. z-score each query head's scores over the stream and take the max over the GQA group;
 *   3. keep the top B keys (ties to the lower index), in ascending index order;
 *   4. compact K, V and the key positions in place.
 * Definitions follow the pages on "TriAttention: Efficient Long Reasoning with Trigonometric KV
 * Compression" (arXiv 2604.04921):
 *   - scores: zhichai.net, "旋转舞台上的追光者..." section "TriAttention：把理论变成算法" items 1-2;
 *     chenxutan.com/d/2624, "TriAttention深度解析..." sections 3.1-3.3 (trig series, offsets D);
 *   - (1-R) weight, sum of the two parts, GQA z-score + max, 128-token cadence:
 *     10100.com/article/127765992 section "TriAttention方法"; watermelonwater.tech,
 *     "TriAttention：面向长文本推理的高效KV缓存压缩..." section "TriAttention 方案设计" item 4;
 *   - top-B kept in original order: chenxutan.com/d/2624 section 4.2 (prune_kv_cache).
 *
 * Conventions shared by every call:
 *   - head_dim d = 128.  A d-vector is read in the half-split RoPE layout: band f (f < 64) is
 *     the complex number v[f] + i*v[f+64].  w_f = fl32(theta^(-2f/d)) (fp64 power, rounded once).
 *   - Cached keys are post-RoPE: band f of key j holds k_f * exp(i*w_f*p_j).
 *   - A stream's id is (s*L + l)*Hkv + g; query head h belongs to KV head h / G, G = Hq/Hkv.
 *   - Device buffers are plain device pointers allocated and owned by the caller.  Layouts:
 *       K, V    [S][L][Hkv][N][128]   dtype bf16 or fp32, rows contiguous
 *       pos     [S][L][Hkv][N]        int32
 *       t       [S]                   int32, position of the newest cached token
 *       F       [S][L][Hkv][N]        fp32 final scores
 *       kept    [S][L][Hkv][min(B,N)] int32, ascending
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call is
 *     asynchronous on that stream; host-detectable argument errors return before any launch.
 *   - No call allocates device memory except tria_load_calib (the calibration table).  Scratch
 *     space is a caller-owned workspace sized by the *_workspace_bytes functions.
 *   - Errors are returned as tria_status; nothing is thrown across the ABI.
 */
#ifndef TRIA_H
#define TRIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRIA_OK = 0,
    TRIA_E_INVALID = -1,      /* bad argument: null pointer, bad size, misaligned buffer */
    TRIA_E_UNSUPPORTED = -2,  /* valid but not implemented: head_dim != 128, G > 8, ... */
    TRIA_E_NOMEM = -3,        /* device allocation failed (tria_load_calib only) */
    TRIA_E_DEVICE = -4,       /* a HIP runtime call or kernel launch failed */
    TRIA_E_NONFINITE = -5,    /* a non-finite key value or score was met (see tria_score_check) */
    TRIA_E_WORKSPACE = -6     /* workspace pointer missing or smaller than required */
} tria_status;

typedef enum { TRIA_BF16 = 0, TRIA_F32 = 1 } tria_dtype;

/* tria_score flags */
#define TRIA_PER_KEY_PHASE 1u /* recover each key's pre-RoPE band phase from its position
                                 (exact integer range reduction of w_f*p) and evaluate the score
                                 in the literal per-key form; same result, more arithmetic. */
#define TRIA_KEYS_PRE_ROPE 2u /* keys are stored before RoPE (k_f, not k_f*exp(i w_f p)); the
                                 score then needs each key's distance phase w_f*(t-p_j). */
#define TRIA_TRIG_WEIGHT_R 4u /* weight band f of the trigonometric series by R_f: the R / (1 - R)
                                 mix of zhichai.net section "TriAttention：把理论变成算法" item 3,
                                 per band (the norm term keeps its (1 - R_f) weight).  Not
                                 combined with the two flags above (TRIA_E_UNSUPPORTED). */
#define TRIA_OFFSET_MAX 8u    /* the trigonometric score is the largest of the per-offset series
                                 instead of their mean (chenxutan.com/d/2624 section 3.3), plus the
                                 norm score; |D| matrix-core contractions per key.  bf16 caches and
                                 at most 32 offsets; combines with TRIA_TRIG_WEIGHT_R, not with the
                                 per-key flags (TRIA_E_UNSUPPORTED). */
#define TRIA_SCORE_TILED 16u  /* score bf16 streams too long for one block's LDS on the tiled path
                                 (raw scores through the workspace, separate statistics and z-max
                                 kernels) instead of the stream clusters (a cooperative grid of one
                                 block per CU whose blocks keep a stream's raw scores in LDS and
                                 exchange per-head partial sums).  Same scores within rounding; the
                                 workspace must then hold the raw scores.  Without this flag the
                                 clusters are used when the device supports cooperative launch and a
                                 stream fits 32 blocks, else the tiled path. */

typedef struct tria_calib tria_calib; /* opaque, library-owned, immutable after load */

/*
 * Build the calibration table from offline statistics (chenxutan.com/d/2624 section 3.4;
 * zhichai.net section "破局之道" for R; watermelonwater.tech "TriAttention 方案设计" item 1).
 *   q_centre    host [L][Hq][d]   pre-RoPE query centres qbar (half-split layout)
 *   q_band_norm host [L][Hq][d/2] E|q_f| >= 0
 *   r_band      host [L][Hq][d/2] R_f in [0, 1]
 *   rope_theta  RoPE base (> 1)
 *   offsets     host [n_offsets]  future offsets D (each in [0, 2^24)); NULL with
 *               n_offsets = 0 selects D = {1, 2, 4, ..., 2^16}
 * The table holds, per (layer, query head), qbar_f * mean_d exp(i w_f d) and the norm weights
 * (1 - R_f) E|q_f|, plus w_f / 2pi per band as a 64-bit fixed-point fraction of a turn.
 * Host arrays are read during the call only.  The table is uploaded with a synchronous copy
 * ordered after `stream`.  *out receives a handle freed with tria_free_calib.
 * Errors: INVALID (null/negative/non-finite/out-of-range input), UNSUPPORTED (head_dim != 128,
 * Hq not a multiple of Hkv, G > 8), NOMEM, DEVICE.
 */
tria_status tria_load_calib(tria_calib **out, int n_layers, int n_q_heads, int n_kv_heads,
                            int head_dim, const float *q_centre, const float *q_band_norm,
                            const float *r_band, double rope_theta, const int32_t *offsets,
                            int n_offsets, void *stream);
void tria_free_calib(tria_calib *calib);

/*
 * The per-band constants tria_load_calib builds its table from, computed on the host alone (no
 * device work), f < head_dim/2:
 *   w[f]  = fl32(rope_theta^(-2f/head_dim)) (the fp64 power rounded once to fp32);
 *   C[f], S[f] = the mean over the offsets D of cos(w_f d) and sin(w_f d) (fp64; w_f d is exact in
 *         fp64), the offset average of the trigonometric series (chenxutan.com/d/2624 section 3.3;
 *         zhichai.net section "TriAttention：把理论变成算法" item 1);
 *   nu[f] = w_f / 2pi as an unsigned 64-bit fraction of a turn, round(w_f / 2pi * 2^64): the phase
 *         of an integer position n is then n * nu mod 2^64, exact in integer arithmetic.
 * offsets / n_offsets as in tria_load_calib.  Outputs are host arrays of head_dim/2 elements.
 * Errors: INVALID (null output, bad theta or offsets), UNSUPPORTED (head_dim != 128).
 */
tria_status tria_band_tables(double rope_theta, int head_dim, const int32_t *offsets, int n_offsets, double *w,
                             double *C, double *S, uint64_t *nu);

/* Shape queries of a loaded table (return -1 for a NULL handle). */
int tria_calib_dim(const tria_calib *calib, int which /* 0 L, 1 Hq, 2 Hkv, 3 d, 4 G */);

/* Workspace bytes tria_score needs for n_seq sequences of n_keys keys of the given cache dtype with
 * the given flags (0 on bad arguments).  The size depends on the path the flags and the shapes
 * select on the calibration table's device: the rotated queries and matrix-core operands always;
 * the cluster exchange words on the stream-cluster path; raw scores [S][L][Hq][N] fp32 and tile
 * partials only on the paths that stage raw scores in HBM (fp32 or TRIA_SCORE_TILED streams too
 * long for one block, TRIA_PER_KEY_PHASE, TRIA_KEYS_PRE_ROPE, TRIA_OFFSET_MAX). */
size_t tria_score_workspace_bytes(const tria_calib *calib, tria_dtype dtype, int n_seq, int n_keys,
                                  unsigned flags);

/*
 * Score every key of every stream and write the final score F (steps 1-2 above).
 *   k          device [S][L][Hkv][N][128] keys (dtype), 16-byte aligned
 *   pos        device [S][L][Hkv][N] key positions (read only with TRIA_PER_KEY_PHASE or
 *              TRIA_KEYS_PRE_ROPE; may be NULL otherwise)
 *   t          device [S] current positions
 *   F          device [S][L][Hkv][N] output final scores
 *   raw        device [S][L][Hq][N] optional output of the raw scores S_trig + S_norm (NULL: not written)
 *   head_stats device [S][L][Hq][2] optional output of each head's (mean, population std)
 *   ws         device workspace of at least tria_score_workspace_bytes(..., flags), 256-byte
 *              aligned; its contents need not be initialised.
 * Positions and t must satisfy |t - p| < 2^24 and |t + d| < 2^31.
 * A head whose raw scores span at most 2^-16 of their largest magnitude (equal up to rounding)
 * is constant: std 0, and it contributes z = 0.
 * Non-finite raw scores set a flag in the workspace; read it with tria_score_check.
 */
tria_status tria_score(const tria_calib *calib, tria_dtype dtype, const void *k, const int32_t *pos,
                       const int32_t *t, int n_seq, int n_keys, float *F, float *raw,
                       float *head_stats, unsigned flags, void *ws, size_t ws_bytes, void *stream);

/* Synchronise `stream` and report TRIA_E_NONFINITE if the last tria_score on this workspace
 * met a non-finite score, else TRIA_OK (TRIA_E_DEVICE on a runtime error, when a stream
 * cluster's exchange of partial sums did not complete, or, after tria_prune, when a tile of the
 * tile-parallel compaction did not see its predecessors hold their rows in time). */
tria_status tria_score_check(const void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes tria_select_topB needs (0 on bad arguments). */
size_t tria_select_workspace_bytes(int n_streams, int n_keys, int budget);

/*
 * Top-B selection per stream (step 3): kept[s][0..min(B,N)) = the indices of the min(B,N)
 * largest F, ties to the lower index, -0 equal to +0, written in ascending order.
 * B >= N gives kept = 0..N-1.  F must be finite (guaranteed when tria_score_check is OK).
 *   F    device [n_streams][N] fp32;  kept device [n_streams][min(B,N)] int32.
 */
tria_status tria_select_topB(const float *F, int n_streams, int n_keys, int budget, int32_t *kept,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * In-place, order-preserving compaction (step 4): for i < min(B,N), row i of K, V and pos takes
 * row kept[i].  kept must be strictly ascending with kept[i] in [i, N) (as tria_select_topB
 * writes it).  Rows >= min(B,N) are left as they were.  k, v 16-byte aligned; pos may be NULL.
 */
tria_status tria_compact(tria_dtype dtype, void *k, void *v, int32_t *pos, const int32_t *kept,
                         int n_streams, int n_keys, int budget, int head_dim, void *stream);

/* Whole prune step: tria_score, tria_select_topB and tria_compact in sequence on `stream`,
 * with kept written to the caller's buffer.  ws must hold tria_prune_workspace_bytes(..., flags).
 * With fewer streams than two per compute unit, or streams of at most 8192 keys, the compaction
 * runs one block per tile of 256 rows (same results as tria_compact's one block per stream);
 * tria_prune_workspace_bytes then adds 4 bytes per tile for its synchronisation words (a workspace
 * with room only for tria_score gets a fused per-stream selection and compaction, as do many
 * longer streams).
 * The step is asynchronous, so a scoring failure found on the device (a non-finite score, or a
 * stream cluster's exchange that did not complete) cannot be returned by this call: the selection
 * then writes kept = 0..min(B,N)-1 and K, V and pos are left untouched.  Confirm the step with
 * tria_score_check(ws) before relying on the compacted cache. */
size_t tria_prune_workspace_bytes(const tria_calib *calib, tria_dtype dtype, int n_seq, int n_keys,
                                  int budget, unsigned flags);
tria_status tria_prune(const tria_calib *calib, tria_dtype dtype, void *k, void *v, int32_t *pos,
                       const int32_t *t, int n_seq, int n_keys, int budget, float *F,
                       int32_t *kept, unsigned flags, void *ws, size_t ws_bytes, void *stream);

const char *tria_status_string(tria_status status);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): tria_prune with its workspace in a static device array
 * of TRIA_STATIC_WORKSPACE_BYTES that the library holds on every device it runs on until the
 * process ends; no call to hipMalloc or any other allocating routine is made (keep kernel timing
 * off: its events are runtime allocations).  Same arguments and results as tria_prune, without ws.
 * The caller still owns K, V, pos, t, F and kept.  When the workspace of all n_seq sequences does
 * not fit the array, the step runs in chunks of whole sequences, one after the other on `stream`
 * (same results).  Every call on a device shares that device's array: calls that overlap on one
 * device (other streams or threads) race; calls ordered on one stream do not.
 *   ws_used  (may be NULL) receives the array's device address: pass it to tria_score_check(ws_used,
 *            256, stream) to confirm the step (as after tria_prune; on a failed score every row of
 *            the affected sequences stays in place).  Valid until the next call on this device.
 * Errors: those of tria_prune; TRIA_E_WORKSPACE when one sequence's workspace exceeds the array
 * (e.g. the paths that stage raw scores in HBM at large N); TRIA_E_DEVICE when the array's address
 * cannot be obtained.
 */
#define TRIA_STATIC_WORKSPACE_BYTES (64u << 20)
tria_status tria_prune_static(const tria_calib *calib, tria_dtype dtype, void *k, void *v, int32_t *pos,
                              const int32_t *t, int n_seq, int n_keys, int budget, float *F, int32_t *kept,
                              unsigned flags, void **ws_used, void *stream);

/*
 * Decode loop (the cadence of the 10100.com article, section "TriAttention方法", and of
 * watermelonwater.tech "TriAttention 方案设计" item 4: prune once every 128 generated tokens; the
 * attention layer of chenxutan.com/d/2624 section 4 appends each token's K/V and prunes back to
 * the budget).  The cache of every stream is a fixed-capacity buffer of `cap` rows (stream
 * stride cap rows) of which the first `len` are live.
 *
 * tria_append: copy n_new rows per stream into rows [len, len + n_new) of K, V and pos.
 *   k, v       device [S][L][Hkv][cap][head_dim] (bf16 or fp32), 16-byte aligned
 *   pos        device [S][L][Hkv][cap] int32 (may be NULL)
 *   k_new, v_new device [S][L][Hkv][n_new][head_dim], pos_new device [S][L][Hkv][n_new] (NULL iff
 *              pos is NULL)
 *   Errors: INVALID (null pointers, len < 0, n_new < 1, len + n_new > cap, misaligned),
 *   UNSUPPORTED (head_dim != 128), DEVICE.
 *
 * tria_decode_step: tria_append, then, when the append fills the cache (len + n_new == cap) and
 * cap > budget, tria_prune over the full cache (N = cap, t = position of each sequence's newest
 * token) so that `budget` rows stay.  *new_len receives the live length afterwards (budget after
 * a prune, else len + n_new).  F [S][L][Hkv][cap] and kept [streams][budget] are scratch outputs
 * of the prune (valid when it ran); ws holds tria_prune_workspace_bytes(calib, dtype, n_seq, cap,
 * budget, flags).  As with tria_prune, a scoring failure found on the device leaves K, V and pos
 * as they were (all cap rows live) although *new_len reports budget: confirm the step with
 * tria_score_check(ws), and on failure keep the live length at cap.
 * Errors: those of tria_append and tria_prune.
 */
tria_status tria_append(tria_dtype dtype, void *k, void *v, int32_t *pos, int n_streams, int cap, int len,
                        const void *k_new, const void *v_new, const int32_t *pos_new, int n_new, int head_dim,
                        void *stream);
tria_status tria_decode_step(const tria_calib *calib, tria_dtype dtype, void *k, void *v, int32_t *pos,
                             const int32_t *t, int n_seq, int cap, int len, int budget, const void *k_new,
                             const void *v_new, const int32_t *pos_new, int n_new, float *F, int32_t *kept,
                             unsigned flags, void *ws, size_t ws_bytes, int *new_len, void *stream);

/*
 * Calibration statistics of captured pre-RoPE queries: the offline step that feeds
 * tria_load_calib (chenxutan.com/d/2624 section 3.4; zhichai.net section "破局之道" for R;
 * watermelonwater.tech "TriAttention 方案设计" item 1).  Per (layer, query head) and band f
 * (q[f] + i q[f + head_dim/2]): qbar_f = mean_n q_{n,f}, E|q_f| = mean_n |q_{n,f}| and
 * R_f = |qbar_f| / E|q_f| (0 when E|q_f| = 0).  Sums in fp64, in a fixed order (deterministic).
 *   q            device [L][Hq][n_cal][head_dim] bf16 or fp32, half-split layout, 16-byte aligned
 *   q_centre     device [L][Hq][head_dim] fp32 out
 *   q_band_norm  device [L][Hq][head_dim/2] fp32 out
 *   r_band       device [L][Hq][head_dim/2] fp32 out
 * The outputs, copied to the host, are tria_load_calib's inputs.  Non-finite inputs give
 * non-finite statistics (which tria_load_calib rejects).  Asynchronous on `stream`.
 * Errors: INVALID (null pointer, n_cal < 1, bad sizes, misaligned), UNSUPPORTED (head_dim != 128),
 * DEVICE (launch failure).
 */
tria_status tria_calib_stats(tria_dtype dtype, const void *q, int n_layers, int n_q_heads, int n_cal, int head_dim,
                             float *q_centre, float *q_band_norm, float *r_band, void *stream);

/*
 * Kernel timing (instrumentation, off by default).  While enabled, every timed kernel launched by
 * tria_score, tria_select_topB, tria_compact and tria_prune is bracketed by a pair of HIP events
 * recorded on the stream it runs on.  tria_timing_read waits for the recorded events, returns the
 * summed elapsed milliseconds and the number of timed launches per timer, and starts a new
 * accumulation.  Recording creates HIP events (a runtime allocation) the first time a pair is
 * needed: keep timing off where nothing may allocate.  Errors: INVALID (NULL outputs), DEVICE
 * (an event could not be read; the other sums are still returned).
 */
typedef enum {
    TRIA_TIMER_SCORE_KEYS = 0, /* the kernel that reads every cached key and scores it */
    TRIA_TIMER_NORMALISE = 1,  /* per-head statistics, z-score and GQA max (long streams) */
    TRIA_TIMER_SELECT = 2,     /* top-B selection */
    TRIA_TIMER_COMPACT = 3,    /* in-place compaction */
    TRIA_TIMER_CALIB = 4,      /* calibration statistics (tria_calib_stats) */
    TRIA_TIMER_SELECT_COMPACT = 5, /* selection and compaction in one kernel (tria_prune, streams of
                                      up to 32768 keys) */
    TRIA_TIMER_COUNT = 6
} tria_timer;

tria_status tria_timing_enable(int on);
tria_status tria_timing_read(double *ms /* [TRIA_TIMER_COUNT] */, int *launches /* [TRIA_TIMER_COUNT] */);

/*
 * Streaming device copy (instrumentation): copies n_bytes from src to dst, both device buffers
 * owned by the caller, 16-byte aligned, not overlapping, n_bytes a positive multiple of 16, with
 * non-temporal 16-byte loads and stores.  It computes nothing of the method: it is the read + write
 * reference whose rate the benchmark reports beside the prune step's (the in-place compaction reads
 * and writes every moved row, so a plain copy bounds it).  Asynchronous on stream.  Errors:
 * INVALID (NULL pointer, zero, ragged or misaligned size, overlapping buffers), DEVICE (launch).
 */
tria_status tria_copy(const void *src, void *dst, size_t n_bytes, void *stream);


#ifdef __cplusplus
}
#endif
#endif /* TRIA_H */
