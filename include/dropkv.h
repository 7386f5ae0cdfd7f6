/*
 * dropkv.h -- C ABI of libdropkv: DropKV per-token output-perturbation scoring,
 * eviction selection and cache compaction on AMD Instinct MI355X (gfx950).
 *
 * The method (DropKV: Decoupling Residual-Output Perturbation for Near-Optimal
 * KV-Cache Eviction, arXiv 2610.22130):
 *   - Section 3.1 / Appendix C.2: deleting token j from the softmax of one query
 *     changes the attention output a = sum_j p_j v_j by
 *         Delta_j = p_j / (1 - p_j) * (a - v_j).
 *   - Section 3.3, and the "Core equation" of the third-party implementation
 *     notes: over the observation window of w tail queries the score is
 *         s_j = sum_t || Delta_j^(t) ||^2 .
 *   - The notes' description of "Algorithm 1": query heads sharing one physical
 *     KV head are averaged, MaxPool1D smooths the scores, the recent window is
 *     set to +inf, the smallest scores are evicted, and a probability that
 *     rounds to 1 is rejected instead of being epsilon-patched.
 *   - Section 2.2: eviction shrinks the resident cache (compaction).
 *   - "paper tables", Table 14 and "paper digest", App. B: the attention-only
 *     (SnapKV-style) score the pages compare against (dropkv_score_attention).
 *
 * Conventions shared by every call:
 *   - bf16 tensors are passed as uint16_t bit patterns in device memory.
 *   - q_win  [Hq][w][d]  : the w tail queries of every query head; window query t
 *                          sits at position n-w+t and sees keys 0..n-w+t.
 *   - k, v   [Hkv][n][d] : the cache of every KV head, rows contiguous.
 *     Layers and batch entries fold into the head dimension ([L][B][H] is
 *     Hkv = L*B*H heads), as long as q_win folds the same way.
 *   - query head h belongs to KV head g = h / G, G = Hq / Hkv.
 *   - every pointer is caller-owned device memory, 16-byte aligned; outputs are
 *     preallocated by the caller; the library never frees or retains them.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call is
 *     asynchronous on that stream except dropkv_sync.  Scratch the library
 *     (re)initialises is cleared by kernels on the call's own stream, so streams
 *     created non-blocking (which do not wait for the null stream) are fine.
 *   - Calls on one context share its scratch: calls that may overlap in time
 *     (streams with no ordering between them) need separate contexts.
 *   - Host-side argument checks happen before any launch and return EINVAL
 *     synchronously.  Conditions found on the device (ESINGULAR, ENONFINITE,
 *     ERANGE) are latched in the context and returned by dropkv_sync; while a
 *     condition is latched, dropkv_select does not produce a keep list.
 *   - On any error the contents of the outputs are unspecified.
 *   - A context is bound to one device and must not be used from two host
 *     threads at once.
 */
#ifndef DROPKV_H
#define DROPKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DROPKV_OK = 0,
    DROPKV_EINVAL = 1,     /* bad argument, found on the host before any launch */
    DROPKV_ESINGULAR = 2,  /* some window query puts probability that rounds to 1 on one key */
    DROPKV_ENONFINITE = 3, /* a non-finite input element */
    DROPKV_ERANGE = 4,     /* an input element of magnitude >= 2^48, a keep index outside
                              [0, n), or an in-place keep list that is not strictly
                              ascending */
    DROPKV_EDEVICE = 5,    /* a HIP runtime error */
    DROPKV_ENOMEM = 6,     /* scratch allocation failed */
    DROPKV_ESCRATCH = 7    /* dropkv_score_noalloc: the call needs more scratch than its
                              static buffer holds */
};

typedef struct dropkv_ctx dropkv_ctx;

/* Create a context on `device` (a HIP device ordinal).  The context owns the
 * scratch used by dropkv_score (split partial states and per-query state,
 * O(Hq * w * d * splits) bytes, grown on demand) and the device error latch. */
int dropkv_create(dropkv_ctx **out, int device);

/* Release the context and its scratch.  Synchronises the device first. */
int dropkv_destroy(dropkv_ctx *ctx);

/*
 * Score every cached token of every KV head.
 *   scores [Hkv][n] fp32 (out): for each KV head g and position j,
 *       raw_g[j]   = (1/G) * sum_{h in group g} sum_{t < w} ||Delta_j^(h,t)||^2
 *                    (Delta = 0 where query t does not see key j),
 *       scores[g][j] = max over i in [j - r, j + r] and [0, n) of raw_g[i],
 *                    r = (pool - 1)/2, then +inf for j >= n - w.
 *   No attention weights, distances or per-token intermediates are materialised:
 *   scratch is O(Hq * w * d * splits).
 * EINVAL if: a pointer is NULL or not 16-byte aligned; Hq % Hkv != 0; w < 1 or
 *   w > n; n < 1 or n >= 2^31; pool < 1, pool even or pool > 129; d % 8 != 0 or
 *   d > 256; G * w > 128 (the window rows of one KV head, in groups of 32; the
 *   first pass reads K and V once per group); for d > 128, G * w > 96.
 * Input contract: every q, k and v element finite and of magnitude below
 *   2^48 (then no logit, distance or score, and no fp32 intermediate of them,
 *   comes near FLT_MAX).
 * Latched, in this order of precedence: ENONFINITE if an input element is not
 *   finite; ERANGE if one has magnitude >= 2^48; ESINGULAR if for some window
 *   query the mass off its arg-max key, relative to the arg-max, is <= 2^-53
 *   (so p_max rounds to 1 in binary64).
 */
int dropkv_score(dropkv_ctx *ctx, const uint16_t *q_win, const uint16_t *k_cache,
                 const uint16_t *v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d,
                 int32_t pool, float *scores, void *stream);

/*
 * dropkv_score for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and the same results, bit for bit, as dropkv_score, but the
 * split partial states and per-query state live in a static device array of
 * dropkv_noalloc_scratch_bytes() bytes (16 MiB: the headline Llama-shaped
 * layer, Hkv = 8, d = 128, w = 8, G = 4, needs 9 MB) instead of the context's
 * scratch.  The call allocates nothing (no hipMalloc, no events; the context
 * must exist, and dropkv_create is where the array's device address is read).
 * Every call on one device shares that device's array and it keeps the last
 * call's contents; nothing in it needs clearing between calls.  Calls that may
 * overlap in time on one device -- any two streams without ordering, even with
 * different contexts -- race on the array and must not be issued.
 * ESCRATCH (synchronously, nothing launched) if dropkv_scratch_bytes reports a
 * score scratch above dropkv_noalloc_scratch_bytes() for these sizes.  All
 * other arguments, checks and latched conditions as for dropkv_score.
 */
int dropkv_score_noalloc(dropkv_ctx *ctx, const uint16_t *q_win, const uint16_t *k_cache,
                         const uint16_t *v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                         int32_t d, int32_t pool, float *scores, void *stream);

/* Size in bytes of dropkv_score_noalloc's static scratch array. */
int64_t dropkv_noalloc_scratch_bytes(void);

/*
 * dropkv_score, also handing back what the first pass computes anyway for the
 * window queries (the pages' result object returns the query output with the
 * scores; the notes, "Code mapping and limits"):
 *   out_a   [Hq][w][d] fp32 (may be NULL): a = sum_j p_j v_j of window query
 *           (h, t), p = softmax over the keys j <= n-w+t of q.k_j / sqrt(d);
 *   out_lse [Hq][w] fp32 (may be NULL): log sum_j exp(q.k_j / sqrt(d)) over the
 *           same keys (natural log).
 * Both are caller-owned device memory, 16-byte aligned.  Everything else is as
 * for dropkv_score; on a latched error their contents are unspecified.
 */
int dropkv_score_ex(dropkv_ctx *ctx, const uint16_t *q_win, const uint16_t *k_cache,
                    const uint16_t *v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                    int32_t d, int32_t pool, float *scores, float *out_a, float *out_lse,
                    void *stream);

/*
 * Attention-only scores: the comparison rule the pages evaluate DropKV against
 * ("paper tables", Table 14, SnapKV row: MaxPool1d over the window-summed
 * attention weights; "paper digest", App. B: the same observation window and
 * pooling kernel, without DropKV's value-residual factor).  For each KV head g
 * and position j:
 *       raw_g[j]    = (1/G) * sum_{h in group g} sum_{t < w} p_j^(h,t)
 *                     (p = softmax(K q / sqrt(d)) over the keys query t sees),
 *       scores[g][j] = max over [j - r, j + r] and [0, n) of raw_g[i], then +inf
 *                     for j >= n - w  -- the same pooling and protection as
 *                     dropkv_score, so dropkv_select applies unchanged.
 * Only K is read (no value cache).  Arguments and layouts as dropkv_score.
 * EINVAL as for dropkv_score.  Latched: ENONFINITE if a q or k element is not
 * finite, else ERANGE if one has magnitude >= 2^48.  (A probability near 1 is
 * not an error here.)
 */
int dropkv_score_attention(dropkv_ctx *ctx, const uint16_t *q_win, const uint16_t *k_cache,
                           int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool,
                           float *scores, void *stream);

/*
 * Keep `budget` tokens per KV head: evict the k = n - budget smallest scores by
 * the total order (score, index) ascending -- among equal scores the older token
 * goes first -- and write the survivors' indices in ascending order.
 *   scores [Hkv][n] fp32 (in), keep [Hkv][budget] int32 (out).
 * Scores are compared as floats with -0 == +0; NaN orders above +inf.
 * EINVAL if: a pointer is NULL or misaligned; Hkv < 1; n < 1 or n >= 2^31;
 *   budget < 0 or budget > n.  (dropkv_score's protected window survives any
 *   budget >= w.)
 * If the context has a latched device error, nothing is written.
 * A head of at most 16384 tokens is one workgroup.  Larger heads: when
 * Hkv * ceil(n / 16384) workgroups of 1024 threads fit on the device at once,
 * one launch whose workgroups (a team per head) exchange histograms and
 * candidates; a workgroup whose teammates have not all arrived at an exchange
 * after dropkv_set_select_wait polls (e.g. on a device shared with other work)
 * finishes its share alone from the scores in memory, which is slower but
 * gives the same keep entries -- the call never fails for lack of
 * co-residency.  Otherwise four launches.  All paths give the same result.
 */
int dropkv_select(dropkv_ctx *ctx, const float *scores, int32_t Hkv, int64_t n, int64_t budget,
                  int32_t *keep, void *stream);

/*
 * dropkv_score then dropkv_select on its scores, as one call: the same scores
 * (same bits) and the same keep list, with the selection's first radix round
 * built inside the scoring's second pass.  The pages pool the perturbation
 * scores and then evict the lowest ("paper digest", Section 3.3 and the
 * implementation notes' "Algorithm 1"); here the pass that writes the pooled,
 * protected scores also counts them into the 4096 bins of their top 12 key
 * bits, so a selection that runs as one launch of a team per head (see
 * dropkv_select) starts at the bin search instead of a histogram round and a
 * team barrier.  Other sizes (a head of at most 16384 tokens, a team that does
 * not fit, budget 0 or n) run exactly dropkv_score and dropkv_select.
 * Arguments, layouts, errors and the latch as for the two calls; budget == 0
 * writes only the scores.  The histogram lives in the context's selection
 * scratch, so calls that overlap on one context race, as for dropkv_select.
 */
int dropkv_score_select(dropkv_ctx *ctx, const uint16_t *q_win, const uint16_t *k_cache,
                        const uint16_t *v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                        int32_t d, int32_t pool, int64_t budget, float *scores, int32_t *keep,
                        void *stream);

/*
 * Layer-wide selection for cross-head budgets ("paper digest" §5.3 pairs DropKV
 * scores with an adaptive per-head budget; the pages do not give the
 * allocation rule, and this call takes the plainest one: a single selection over
 * the whole layer).  Evict the Hkv*n - budget smallest of all the layer's scores
 * by (score, head, index) ascending.
 *   scores [Hkv][n] fp32 (in), budget = total tokens kept over all heads;
 *   keep   [budget] int32 (out): survivors as flat indices g*n + j, ascending
 *          (so head-major, each head's indices ascending);
 *   counts [Hkv] int32 (out): survivors per head (they sum to budget).
 * The +inf window of every head survives whenever budget >= Hkv*w.  The packed
 * cache follows from dropkv_compact with Hkv = 1 and n = Hkv*n (the keep
 * entries address rows of the [Hkv][n][d] cache directly).
 * EINVAL if: a pointer is NULL or misaligned (keep may be NULL when budget is
 * 0); Hkv < 1; n < 1; Hkv*n >= 2^31; budget < 0 or budget > Hkv*n.
 * Latched errors and device waits as for dropkv_select.
 */
int dropkv_select_layer(dropkv_ctx *ctx, const float *scores, int32_t Hkv, int64_t n,
                        int64_t budget, int32_t *keep, int32_t *counts, void *stream);

/*
 * Gather the kept rows into a packed cache (exact bit copies):
 *   k_out[g][r][:] = k[g][keep[g][r]][:],  v_out likewise;  [Hkv][budget][d] bf16.
 * Inputs and outputs must not overlap.
 * EINVAL as for dropkv_score's shape checks, plus budget < 0 or budget > n.
 * Latched: ERANGE if some keep index lies outside [0, n) (that row is zero-filled).
 */
int dropkv_compact(dropkv_ctx *ctx, const uint16_t *k, const uint16_t *v, int32_t Hkv, int64_t n,
                   int32_t d, const int32_t *keep, int64_t budget, uint16_t *k_out,
                   uint16_t *v_out, void *stream);

/*
 * Compact a resident cache in place (exact bit copies): for every KV head g and
 * r < budget, row r of k_cache and v_cache [Hkv][cap][d] bf16 becomes old row
 * keep[g][r].  keep [Hkv][budget] int32 must be strictly ascending inside
 * [0, n_valid) -- dropkv_select's output is -- so no row is overwritten before
 * it has been read.  Rows budget .. n_valid-1 are unspecified afterwards; rows
 * n_valid .. cap-1 and other memory are untouched.  The caller owns both
 * buffers; the call allocates nothing.
 * EINVAL if: a pointer is NULL or misaligned; Hkv < 1; cap < 1 or cap >= 2^31;
 *   n_valid < 1 or n_valid > cap; d not a multiple of 8 in [8, 256]; budget < 0
 *   or budget > n_valid.
 * Latched: ERANGE if some head's keep list is not strictly ascending inside
 *   [0, n_valid) (that head's rows stay where they are; other heads move).  While
 *   an error of scoring or selection is latched, nothing moves.
 */
int dropkv_compact_inplace(dropkv_ctx *ctx, uint16_t *k_cache, uint16_t *v_cache, int32_t Hkv,
                           int64_t cap, int64_t n_valid, int32_t d, const int32_t *keep,
                           int64_t budget, void *stream);

/*
 * Decode-time rescoring of a resident cache.  "paper digest" §6 (Discussion
 * and Limitation) leaves a decode-time kernel as future work and §5.4 runs
 * decoding on the evicted cache; the plainest reading, taken here: after m
 * decode steps the cache [Hkv][cap][d] holds n_valid <= cap rows per KV head
 * (the tokens kept so far, in their order, then the m appended tokens), and
 * q_win [Hq][w][d] holds the queries of its last w positions.  One call
 *   1. scores those rows exactly as dropkv_score scores a prefill cache of
 *      n = n_valid tokens (the window is rows n_valid - w .. n_valid - 1,
 *      protected with +inf): scores [Hkv][n_valid] fp32 (out);
 *   2. keeps `budget` rows per head by dropkv_select's rule: keep
 *      [Hkv][budget] int32 (out), ascending old row indices;
 *   3. compacts the cache in place as dropkv_compact_inplace does.
 * Afterwards each head holds `budget` valid rows (set n_valid = budget and
 * append further decode tokens after them).  budget == 0 scores only.
 * EINVAL as for dropkv_score with n = n_valid (k/v rows are cap apart per
 * head), plus cap < 1 or cap >= 2^31, n_valid > cap, budget < 0 or budget >
 * n_valid.  Latched errors as for dropkv_score and dropkv_select; while one is
 * latched the cache is not moved.  Scratch as for dropkv_score.
 */
int dropkv_rescore(dropkv_ctx *ctx, const uint16_t *q_win, uint16_t *k_cache, uint16_t *v_cache,
                   int64_t cap, int64_t n_valid, int32_t w, int32_t Hq, int32_t Hkv, int32_t d,
                   int32_t pool, int64_t budget, float *scores, int32_t *keep, void *stream);

/* Wait for `stream`, then return and clear the latched device condition
 * (ENONFINITE before ESINGULAR before ERANGE), or DROPKV_OK; EDEVICE if the
 * HIP runtime reports an error. */
int dropkv_sync(dropkv_ctx *ctx, void *stream);

/* Polls a workgroup of the single-launch selection makes at a team exchange
 * before it finishes its share alone (see dropkv_select).  Default 16384
 * (about 10-20 ms); 0 stops waiting at the first poll that finds a teammate
 * missing; a negative value makes every workgroup go alone at once (no
 * exchange at all).  The result is the same for every value.  EINVAL if ctx is
 * NULL. */
int dropkv_set_select_wait(dropkv_ctx *ctx, int64_t polls);

/* Static string naming a status code. */
const char *dropkv_strerror(int code);

/*
 * Per-kernel timing for measurement.  While enabled, every kernel the library
 * launches is bracketed by HIP events on the caller's stream; dropkv_profile_read
 * returns, for the kernel family `name` ("pass1", "merge", "pass2",
 * "select", "compact", "attn_pass1", "attn_pass2", "stream_read"), the summed milliseconds and launch count since the last
 * reset (it synchronises on the recorded events).  Disabled by default.
 */
int dropkv_profile_enable(dropkv_ctx *ctx, int on);
int dropkv_profile_reset(dropkv_ctx *ctx);
int dropkv_profile_read(dropkv_ctx *ctx, const char *name, double *total_ms, int64_t *launches);

/*
 * Measurement reference: read `bytes` of device memory at `p` once, as one
 * coalesced streaming scan (eight workgroups per CU, each over a contiguous
 * slice), and write nothing the caller can observe.  Timed with the profile
 * name "stream_read", it gives the read bandwidth the device actually reaches,
 * the yardstick for the two score passes, which each stream K and V once.
 * `p` is caller-owned device memory, 16-byte aligned; `bytes` a positive
 * multiple of 16, else EINVAL.  Asynchronous on `stream`.
 */
int dropkv_stream_read(dropkv_ctx *ctx, const void *p, int64_t bytes, void *stream);

/* Device scratch (bytes) the context holds for these sizes: *score_bytes for
 * dropkv_score (split partial states and per-query state; independent of n
 * beyond the split count, which the device's size fixes), *select_bytes for
 * dropkv_select over [Hkv][n] scores.  Nothing of size O(n * d) -- no attention
 * weights or distances -- is ever allocated.  EINVAL as for dropkv_score's
 * shape checks, or a NULL output pointer. */
int dropkv_scratch_bytes(int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d,
                         int64_t *score_bytes, int64_t *select_bytes);

/* Launch geometry dropkv_score would use for these sizes (for tests/diagnostics):
 * number of sequence splits of the first pass. */
int dropkv_plan_splits(int64_t n, int32_t Hkv, int32_t *splits);

#ifdef __cplusplus
}
#endif
#endif /* DROPKV_H */
