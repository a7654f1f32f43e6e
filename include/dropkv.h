/*
 * dropkv.h — DropKV eviction scoring on AMD Instinct MI355X (gfx950).
 *
 * One call scores one sequence (one batch element) of one layer: for every
 * physical KV head it takes the queries of the last `window` positions and the
 * full causal K/V, and returns per-token eviction scores and the indices of
 * the tokens to evict.
 *
 * What is computed (DropKV, arXiv 2610.22130, as described by the write-up
 * "DropKV：精确单项输出扰动评分组件", section 核心公式 (core formula) and the
 * prose after its displayed equation; pipeline figure of section 背景与主要改动):
 *   for query head h and window row i (sequence position P = n - window + i,
 *   keys 0..P visible — causal tail alignment, section 代码映射与边界):
 *     p = softmax(K q / sqrt(d)),   a = sum_j p_j v_j,
 *     Delta_j = p_j / (1 - p_j) * (a - v_j)      (exact single-token removal),
 *     s_j(h) = sum over window rows of ||Delta_j||^2;
 *   S_g(j) = mean of s_j(h) over the query heads h of KV head g (GQA:
 *            h belongs to g = h / (Hq / Hkv));
 *   P_g = MaxPool1D(S_g) (odd kernel, stride 1, same padding, over [0, n));
 *   P_g(j) = +inf for the last `window` positions (recent-window protection);
 *   evict_g = the n_evict smallest P_g under the order (score, index),
 *             returned in ascending index order.
 *   A row whose largest probability rounds to 1 in binary32 (rest mass
 *   R = sum_{j != argmax} exp(x_j - x_max) <= 2^-24) makes exact single-token
 *   removal singular and is rejected (DROPKV_ERR_SINGULAR); no epsilon is used.
 *
 * Layouts (row-major, contiguous, device memory, one sequence):
 *   q            [Hq][window][d]   bf16 (as uint16 bit patterns) or fp32
 *   k, v         [Hkv][n][d]       same dtype as q
 *   out_scores   [Hkv][n]          fp32: pooled scores, +inf on the window
 *   out_evict_idx[Hkv][n_evict]    int64, ascending per head
 * All pointers are device pointers owned by the caller; the library keeps
 * none of them after the call returns. Batches are scored by one call per
 * sequence (pointer offsets).
 *
 * Errors: every entry point validates its arguments on the host first; an
 * invalid call launches nothing, leaves the outputs untouched and returns
 * DROPKV_ERR_INVALID. DROPKV_ERR_SINGULAR / DROPKV_ERR_NONFINITE are found
 * on the device; after them the outputs are unspecified and must not be used.
 * DROPKV_ERR_DEVICE covers HIP runtime failures (no device, launch or memory
 * errors). There is no CPU fallback. dropkv_last_error() describes the most
 * recent failure of the calling thread.
 *
 * Threading: the plain entry points use one library-owned, grow-only
 * workspace per device behind a mutex; calls from several threads are
 * serialised. dropkv_score_ex takes caller-owned workspace instead and never
 * synchronises.
 */
#ifndef DROPKV_H
#define DROPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DROPKV_OK = 0,
  DROPKV_ERR_INVALID = -1,   /* bad argument: nothing launched */
  DROPKV_ERR_SINGULAR = -2,  /* a window row has a probability that rounds to 1 */
  DROPKV_ERR_NONFINITE = -3, /* NaN/inf in the inputs or the scores */
  DROPKV_ERR_DEVICE = -4,    /* HIP runtime error */
  DROPKV_ERR_NEGATIVE = -5   /* dropkv_select only: a given raw score is negative */
} dropkv_status;

/* Element type of q, k, v. */
enum { DROPKV_BF16 = 0, DROPKV_F32 = 1 };

/* Bits of the device status word written by dropkv_score_ex (and, for
 * DROPKV_STATUS_BAD_INDEX, by dropkv_compact; DROPKV_STATUS_PENDING, by
 * dropkv_decode_select after dropkv_decode_step_deferred). */
enum {
  DROPKV_STATUS_SINGULAR = 1,
  DROPKV_STATUS_NONFINITE = 2,
  DROPKV_STATUS_BAD_INDEX = 4,
  DROPKV_STATUS_PENDING = 8,
  DROPKV_STATUS_NEGATIVE = 16, /* dropkv_select: a given raw score S[g][j] < 0 */
  DROPKV_STATUS_BOUNDS = 32    /* checking build (libdropkv_debug.so) only: a device-side
                                  bounds check failed; the call returns DROPKV_ERR_DEVICE */
};

/* Flags for dropkv_score_ex. */
enum {
  DROPKV_FLAG_GENERIC = 1, /* force the plain-VALU path even where the MFMA path applies */
  DROPKV_FLAG_STAGE_LOG = 2 /* dropkv_score_ex only: record each stage's begin and end time
                               (the dispatch timestamps of its first and last kernel on the
                               MFMA path and the select stage) into the library's stage log
                               (see dropkv_stage_log) */
};

/*
 * Score one sequence, bf16 inputs (uint16 bit patterns). Argument limits:
 * 1 <= window < n; Hq, Hkv >= 1 and Hq % Hkv == 0; 1 <= d <= 256;
 * pool_kernel odd and >= 1; 0 <= n_evict <= n - window (out_evict_idx may be
 * NULL when n_evict == 0). `stream` is a hipStream_t (NULL = default stream).
 * Enqueues on `stream`, then synchronises that stream to read the status word.
 */
int dropkv_score(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                 int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                 float* out_scores, int64_t* out_evict_idx, void* stream);

/* Same as dropkv_score with fp32 q, k, v. */
int dropkv_score_f32(const float* q, const float* k, const float* v, int64_t n, int32_t window,
                     int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                     float* out_scores, int64_t* out_evict_idx, void* stream);

/* Bytes of device workspace dropkv_score_ex needs for this shape (0 on invalid shape). */
size_t dropkv_workspace_bytes(int32_t dtype, int64_t n, int32_t window, int32_t Hq, int32_t Hkv,
                              int32_t d);

/*
 * Fully asynchronous form. `workspace` (>= dropkv_workspace_bytes, 256-byte
 * aligned, device memory owned by the caller) holds all scratch; `d_status`
 * is a caller-owned device int32 that the call clears and then ORs
 * DROPKV_STATUS_* bits into. Returns DROPKV_OK once enqueued (or
 * DROPKV_ERR_INVALID / DROPKV_ERR_DEVICE); device-side errors are visible only
 * in *d_status after the stream completes. Calls sharing a workspace must be
 * ordered on one stream.
 */
int dropkv_score_ex(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                    int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                    int64_t n_evict, float* out_scores, int64_t* out_evict_idx, void* workspace,
                    size_t workspace_bytes, int32_t* d_status, uint32_t flags, void* stream);

/*
 * dropkv_score_ex that also writes the kept token indices: out_keep_idx
 * [Hkv][n - n_evict] int64 (device memory, caller-owned; may be NULL only
 * when n_evict == n), per head the indices that out_evict_idx does not name
 * (the protected window included), ascending. The select stage emits them
 * alongside the evicted ones, for dropkv_compact_kept (write-up section
 * 代码映射与边界: the caller drops the evicted tokens from its cache; a kept
 * list is what a gather of the kept rows reads). Same limits, ownership,
 * status word and asynchrony as dropkv_score_ex.
 */
int dropkv_score_keep_ex(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                         int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_evict_idx, int64_t* out_keep_idx,
                         void* workspace, size_t workspace_bytes, int32_t* d_status, uint32_t flags,
                         void* stream);

/* Size of the static scratch array behind dropkv_score_noalloc, per GPU. */
#define DROPKV_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * scoring as dropkv_score_ex (same kernels, same outputs, bit for bit), with
 * all scratch in a library-owned static device array of
 * DROPKV_NOALLOC_SCRATCH_BYTES (64 MiB; every GPU the library runs on holds
 * one until the process ends) instead of a workspace argument. The caller
 * passes inputs, outputs and d_status (a device int32 that the call clears
 * and ORs DROPKV_STATUS_* bits into) as for dropkv_score_ex.
 * A shape whose dropkv_workspace_bytes exceeds the array is rejected with
 * DROPKV_ERR_INVALID before anything is launched (the 128K-token Llama-3.1-8B
 * layer, 32 query / 8 KV heads, window 64, needs about 60 MiB);
 * DROPKV_FLAG_STAGE_LOG is rejected too. The call makes no hipMalloc,
 * hipFree or other allocating call; its first call on a device looks up the
 * array's device address once. Every call on one GPU uses that GPU's one
 * array, which keeps the previous call's contents (everything that must start
 * at zero is cleared by the call's own first kernel): calls that overlap on
 * one GPU (several streams or threads) race and must be serialised by the
 * caller. Asynchronous: device-side errors are visible in *d_status after the
 * stream completes.
 */
int dropkv_score_noalloc(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                         int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_evict_idx, int32_t* d_status,
                         uint32_t flags, void* stream);

/*
 * Stage export: the GQA-mean scores S [Hkv][n] (fp32) before pooling and
 * protection. Synchronous like dropkv_score (returns SINGULAR / NONFINITE).
 */
int dropkv_raw_scores(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                      int32_t window, int32_t Hq, int32_t Hkv, int32_t d, float* out_S,
                      uint32_t flags, void* stream);

/*
 * Stage export: per window row (row index h*window + i) the softmax
 * statistics after all of n is seen: out_m = largest logit x_max (natural
 * units, x = q.k / sqrt(d)), out_rest = R = sum_{j != argmax} exp(x_j - x_max),
 * out_argmax = lowest index attaining x_max (valid where R < 1; -1 where the
 * path does not track it), and out_a [Hq*window][d] = the attention output a.
 * Any output pointer may be NULL. Synchronous; returns SINGULAR if a row is.
 */
int dropkv_row_stats(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                     int32_t window, int32_t Hq, int32_t Hkv, int32_t d, float* out_m,
                     float* out_rest, int32_t* out_argmax, float* out_a, uint32_t flags,
                     void* stream);

/*
 * The same export under the name of the boundary's stage list: pass-1
 * statistics of bf16 inputs, i.e. dropkv_row_stats(DROPKV_BF16, ..., flags = 0).
 * out_rest is R (the rest mass) as defined there. Synchronous.
 */
int dropkv_pass1_stats(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                       int32_t Hq, int32_t Hkv, int32_t d, float* out_m, float* out_rest,
                       int32_t* out_argmax, float* out_a, void* stream);

/*
 * The pooling, protection and selection stage alone, on caller-given raw
 * scores S [Hkv][n] (fp32): writes out_scores and out_evict_idx exactly as
 * dropkv_score does. DropKV scores are sums of squared norms, so S must be
 * non-negative (-0.0 counts as 0): a negative entry makes the call return
 * DROPKV_ERR_NEGATIVE (found on the device; the outputs are then
 * unspecified). Synchronous; NONFINITE if S holds NaN/inf.
 */
int dropkv_select(const float* S, int64_t n, int32_t window, int32_t Hkv, int32_t pool_kernel,
                  int64_t n_evict, float* out_scores, int64_t* out_evict_idx, void* stream);

/*
 * Measurement form of dropkv_score: runs the whole path once on `stream`
 * with each stage's begin and end time recorded (as DROPKV_FLAG_STAGE_LOG
 * does), synchronises, and writes the
 * duration of each stage in milliseconds to out_ms[0..*out_count-1] (at most
 * 12 stages) and their comma-separated names to out_names (names_bytes
 * bytes, NUL-terminated; may be NULL). Outputs and return codes are those of
 * dropkv_score / dropkv_score_f32 for the same dtype; `flags` as in
 * dropkv_score_ex.
 */
int dropkv_stage_times(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                       int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                       int64_t n_evict, float* out_scores, int64_t* out_evict_idx, uint32_t flags,
                       float* out_ms, char* out_names, int32_t names_bytes, int32_t* out_count,
                       void* stream);

/*
 * Reads the stage log of the current device: calls of dropkv_score_ex made
 * with DROPKV_FLAG_STAGE_LOG since the last read (at most 256 are kept; later
 * ones are not logged). Waits for their events, writes the mean duration of
 * each stage over those calls in milliseconds to out_ms[0..*out_count-1] (at
 * most 12), their comma-separated names to out_names (names_bytes bytes,
 * NUL-terminated; may be NULL) and the number of calls to *out_calls, then
 * empties the log. DROPKV_ERR_INVALID if the logged calls ran different
 * stage sequences; *out_calls = 0 if nothing was logged. Not thread-safe
 * against concurrent logged calls on the same device.
 */
int dropkv_stage_log(float* out_ms, char* out_names, int32_t names_bytes, int32_t* out_count,
                     int32_t* out_calls);

/*
 * Scoring from given window-row statistics, without pass 1: when a prefill
 * attention kernel has already seen the window rows, its per-row statistics
 * replace the first of the two streams over K and V (the step before the
 * path; the atlas summary of the paper, Experimental setup, lists
 * FlashAttention-2 among the work it builds on). Inputs as dropkv_score
 * (bf16 with d = 128 only, the MFMA path), plus per window row r = h*window + i
 * of query head h (device pointers, fp32 unless stated):
 *   m      [Hq*window]     largest logit x_max, x = q.k / sqrt(d) (natural units)
 *   rest   [Hq*window]     R = sum_{j != argmax} exp(x_j - x_max)
 *   argmax [Hq*window]     int32, lowest index attaining x_max (read where R < 1)
 *   a      [Hq*window][d]  attention output sum_j p_j v_j
 * exactly what dropkv_row_stats exports. Outputs and errors as dropkv_score
 * (NONFINITE also for non-finite statistics or an argmax outside [0, n) on a
 * row with R < 1). Synchronous.
 */
int dropkv_score_from_stats(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                            int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                            const float* m, const float* rest, const int32_t* argmax, const float* a,
                            float* out_scores, int64_t* out_evict_idx, void* stream);

/*
 * Asynchronous form of dropkv_score_from_stats, with caller-owned workspace
 * (>= dropkv_workspace_bytes(DROPKV_BF16, ...), 256-byte aligned) and device
 * status word, as dropkv_score_ex (which it mirrors; the status word is
 * cleared by the call).
 */
int dropkv_score_from_stats_ex(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                               int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                               const float* m, const float* rest, const int32_t* argmax, const float* a,
                               float* out_scores, int64_t* out_evict_idx, void* workspace,
                               size_t workspace_bytes, int32_t* d_status, void* stream);

/*
 * Prefill attention that hands over the scoring statistics (the step before
 * scoring: a prefill pass has already attended the window rows, so scoring
 * from its statistics reads K and V once instead of twice). For every query
 * head h and position pos (keys 0..pos of KV head h / (Hq / Hkv) visible),
 * p = softmax(K q / sqrt(d)) and o = sum_j p_j v_j (DropKV write-up, section
 * 核心公式; the atlas summary of the paper, Experimental setup, names
 * FlashAttention-2 as the basis of the paper's scorer). bf16 with d = 128 only;
 * Hq / Hkv <= 32.
 *   q_all      [Hq][n][d]        bf16, the queries of every position
 *   k, v       [Hkv][n][d]       bf16
 *   out_o      [Hq][n][d]        bf16, o of every position
 * and for the last `window` positions, window row r = h * window + i at
 * position n - window + i (the layout dropkv_score_from_stats reads):
 *   out_m      [Hq*window]       fp32, largest logit x_max (x = q.k / sqrt(d))
 *   out_rest   [Hq*window]       fp32, R = sum_{j != argmax} exp(x_j - x_max), formed
 *                                as (sum_j exp(x_j - x_max)) - 1 (exact where R < 1 is
 *                                not needed: scoring recomputes the argmax term then)
 *   out_argmax [Hq*window]       int32, lowest index attaining x_max
 *   out_a      [Hq*window][d]    fp32, o of the window rows
 * All pointers are caller-owned device memory; every output is required.
 * Asynchronous on `stream`: *d_status is cleared, then DROPKV_STATUS_NONFINITE
 * is ORed in for non-finite statistics. DROPKV_ERR_INVALID before any launch
 * for bad shapes or pointers.
 */
int dropkv_prefill_attention(const void* q_all, const void* k, const void* v, int64_t n, int32_t window,
                             int32_t Hq, int32_t Hkv, int32_t d, void* out_o, float* out_m, float* out_rest,
                             int32_t* out_argmax, float* out_a, int32_t* d_status, void* stream);

/*
 * Cache compaction, the step after scoring (write-up section 代码映射与边界:
 * the scorer returns per-head eviction indices and the caller drops those
 * tokens from its cache). Copies the rows of k and v [Hkv][n][d] (dtype
 * DROPKV_BF16 or DROPKV_F32) whose token index is not in evict_idx
 * [Hkv][n_evict] (int64, strictly increasing per head, inside [0, n), as
 * dropkv_score returns it) to out_k, out_v [Hkv][n - n_evict][d], in
 * ascending token order: kept token j of head g becomes row
 * j - #{evicted indices of g below j}. Bitwise copies.
 * Limits: 1 <= n < 2^31, Hkv >= 1, 1 <= d <= 4096, 0 <= n_evict <= n; every
 * pointer is a device pointer (evict_idx may be NULL when n_evict == 0,
 * out_k / out_v when n_evict == n); outputs must not overlap the inputs.
 * Asynchronous on `stream`: the call ORs DROPKV_STATUS_BAD_INDEX into the
 * caller-owned device int32 `d_status` (which the caller clears beforehand;
 * the call does not, so that it is one kernel launch) if some head's list is
 * not strictly increasing inside [0, n); the outputs are then unspecified,
 * but no write falls outside out_k / out_v. Returns DROPKV_OK once enqueued,
 * DROPKV_ERR_INVALID (nothing launched) or DROPKV_ERR_DEVICE.
 */
int dropkv_compact(int32_t dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                   const int64_t* evict_idx, int64_t n_evict, void* out_k, void* out_v,
                   int32_t* d_status, void* stream);

/*
 * Cache compaction from a kept list (as dropkv_score_keep_ex writes it):
 * output row r of head g in out_k, out_v [Hkv][n_keep][d] is row
 * keep_idx[g][r] of k, v [Hkv][n][d]; keep_idx [Hkv][n_keep] int64 must be
 * strictly increasing inside [0, n) per head. Same result as dropkv_compact
 * with the complementary eviction list, without searching that list.
 * Limits: 1 <= n < 2^31, Hkv >= 1, 1 <= d <= 4096, 0 <= n_keep <= n; device
 * pointers (keep_idx, out_k, out_v may be NULL when n_keep == 0); outputs must
 * not overlap the inputs. Asynchronous on `stream`; ORs
 * DROPKV_STATUS_BAD_INDEX into `d_status` (cleared by the caller) for a list
 * that breaks the order or range (outputs then unspecified, no write outside
 * out_k / out_v). Returns DROPKV_OK once enqueued, DROPKV_ERR_INVALID
 * (nothing launched) or DROPKV_ERR_DEVICE.
 */
int dropkv_compact_kept(int32_t dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                        const int64_t* keep_idx, int64_t n_keep, void* out_k, void* out_v,
                        int32_t* d_status, void* stream);

/*
 * Decode-time rescoring with a sliding observation window.
 *
 * The pages leave a decode-time scorer to future work and call per-step decode
 * bandwidth-bound (atlas summary, Limitations). These calls keep the raw score
 * S of the core formula (write-up section 核心公式: the sum over the window
 * queries of ||Delta_j||^2, averaged over the query heads of each KV head;
 * before pooling) up to date while tokens are appended one at a time, the
 * window always being the last `window` query positions: a step adds the
 * terms of the new position's query rows and subtracts those of the rows that
 * leave the window (a row's terms depend only on the keys it sees, which
 * appending does not change). S is kept in fp64 and the subtracted terms are
 * bit for bit the added ones, so the maintained S matches scoring the grown
 * cache from scratch to the path's own accuracy. After an eviction the
 * cache's softmaxes change: compact, then start again with dropkv_decode_init.
 *
 * Inputs are bf16 with d = 128. k and v are the caller's cache, [Hkv][n_max][d]
 * (head stride n_max token rows), of which the first n rows of each head are
 * valid; q is [Hq][window][d] (the last `window` positions' query rows, head
 * major), q_new [Hq][d] (the appended position's query rows). The caller owns
 * `state`: device memory of dropkv_decode_state_bytes(...) bytes (hipMalloc'd,
 * not managed memory: the single-pass step adds to it with fp64 atomics),
 * 256-byte aligned, used only through these calls (layout: fp64 S [Hkv][n_max] first,
 * then the window's rows). All calls are asynchronous on `stream` and return
 * DROPKV_OK once enqueued, DROPKV_ERR_INVALID (nothing launched: shape, count
 * or pointer checks) or DROPKV_ERR_DEVICE. Device-side findings go to the
 * caller's device int32 `d_status` as DROPKV_STATUS_* bits: a window row whose
 * rest mass is <= 2^-24 (SINGULAR) or non-finite values (NONFINITE) make S
 * unspecified until the next init. Limits: window >= 1, Hq a multiple of Hkv
 * with at most 16 query heads per KV head, n_max < 2^31. Calls on one state
 * must not overlap.
 */
size_t dropkv_decode_state_bytes(int64_t n_max, int32_t window, int32_t Hq, int32_t Hkv, int32_t d);

/* Score the first n tokens (window < n <= n_max) and fill the state; clears
 * *d_status first. The window rows' statistics come from the same pass 1 and
 * merge as dropkv_score. */
int dropkv_decode_init(const void* q, const void* k, const void* v, int64_t n, int64_t n_max, int32_t window,
                       int32_t Hq, int32_t Hkv, int32_t d, void* state, size_t state_bytes, int32_t* d_status,
                       void* stream);

/* One appended token: the caller has written its key and value at row n - 1
 * of every head, and n counts it (window + 2 <= n <= n_max, and the state
 * holds n - 1 tokens: one call per token, in order). ORs status bits. */
int dropkv_decode_step(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                       int32_t window, int32_t Hq, int32_t Hkv, int32_t d, void* state, size_t state_bytes,
                       int32_t* d_status, void* stream);

/* One appended token in a single pass over the cache (dropkv_decode_step
 * reads K and V twice: once for the new rows' statistics, then for their
 * terms). Arguments, limits and errors as dropkv_decode_step. The pass computes
 * the new position's row statistics, subtracts the terms of the rows leaving
 * the window and adds those of the rows a previous deferred step left pending;
 * the new rows' terms (which need their finished statistics) stay pending.
 * Their argmax terms are added at once. So after this call S lacks the
 * newest position's non-argmax terms until the next step of either form (a
 * two-pass step adds them), dropkv_decode_flush or dropkv_decode_rebuild;
 * dropkv_decode_select ORs DROPKV_STATUS_PENDING into d_status when called in
 * that state (its result is then that of the incomplete S), and
 * dropkv_decode_scores returns the incomplete S. With more than 8 query heads
 * per KV head this call runs the two-pass step (nothing is left pending). */
int dropkv_decode_step_deferred(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                                int32_t window, int32_t Hq, int32_t Hkv, int32_t d, void* state, size_t state_bytes,
                                int32_t* d_status, void* stream);

/* Add the terms a deferred step left pending (none: nothing changes; the
 * call still launches two small kernels). k, v, n as for the step that left
 * them. */
int dropkv_decode_flush(const void* k, const void* v, int64_t n, int64_t n_max, int32_t window, int32_t Hq,
                        int32_t Hkv, int32_t d, void* state, size_t state_bytes, void* stream);

/* Recompute S from the window rows kept in the state (no new statistics):
 * equal to the incrementally kept S up to fp64 rounding. Nothing stays
 * pending afterwards. ORs status bits. */
int dropkv_decode_rebuild(const void* k, const void* v, int64_t n, int64_t n_max, int32_t window, int32_t Hq,
                          int32_t Hkv, int32_t d, void* state, size_t state_bytes, int32_t* d_status,
                          void* stream);

/* The kept raw score S rounded to fp32 into out_S [Hkv][n]. */
int dropkv_decode_scores(const void* state, size_t state_bytes, int64_t n, int64_t n_max, int32_t window,
                         int32_t Hq, int32_t Hkv, int32_t d, float* out_S, void* stream);

/* Re-eviction on the kept score: max-pool (odd pool_kernel, stride 1, same
 * padding), +inf on the last `window` positions, the n_evict smallest per head
 * under (score, index) ascending, exactly as dropkv_score does after its own
 * raw scores (0 <= n_evict <= n - window). out_scores [Hkv][n] fp32,
 * out_evict_idx [Hkv][n_evict] int64. ORs status bits. */
int dropkv_decode_select(void* state, size_t state_bytes, int64_t n, int64_t n_max, int32_t window, int32_t Hq,
                         int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict, float* out_scores,
                         int64_t* out_evict_idx, int32_t* d_status, void* stream);

/* 1 if (dtype, d) takes the MFMA path by default, 0 if the plain-VALU path. */
int dropkv_uses_mfma(int32_t dtype, int32_t d);

/* Human-readable description of the calling thread's most recent error ("" if none). */
const char* dropkv_last_error(void);

/* The same text under the boundary's second name for it. */
const char* dropkv_last_error_string(void);

/* Library version string. */
const char* dropkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DROPKV_H */
