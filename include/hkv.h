/*
 * hkv.h — C ABI of the HeadKV decode-time path on AMD Instinct MI355X (gfx950).
 *
 * The method (pages: "Head-Aware Key-Value Compression for Efficient
 * Autoregressive Image Generation", gist.science technical summaries, section
 * "Methodology"):
 *   step 1  the cache is prefilled without compression;
 *   step 2  once it reaches a predefined length every attention head is
 *           classified once: the current query's attention is accumulated
 *           backward from the current position until it reaches tau (0.9);
 *           fewer tokens than the local window -> Local, otherwise Global;
 *   step 3  Local heads keep a sliding window of the newest tokens; Global heads
 *           keep a budget enforced by Stratified Token Eviction (STE): the
 *           history is split by distance into disjoint near and far subsets,
 *           each scored from past queries, and the lowest-scoring tokens of each
 *           subset are evicted (M/2 + M/2).
 *   Budgets are asymmetric (section "Key contributions", item 2): compact for
 *   Local heads, larger for Global heads, at a total of rho of the full cache.
 *
 * Readings this library implements where the pages are silent (all are
 * checked against an independent CPU oracle):
 *   - attention: single-query softmax, logits q.k/sqrt(d), one KV head per head;
 *     at decode step t token t is appended first, then attended;
 *   - classification query: position P-1 over positions 0..P-1; count n = the
 *     smallest k with (mass of the k newest) >= tau; Local iff n < w;
 *   - budget per (layer, sequence): A = floor(N*rho_num/rho_den), Local heads w
 *     slots, Global heads B_g = floor((H*A - n_L*w) / n_G), capacity B_g + M;
 *   - score of a slot = sum of the softmax probabilities it received from the
 *     last W queries (W = w_obs = M), evaluated at the eviction step as the
 *     causal W x count probability tile; the W newest tokens are not candidates;
 *     near: W <= t-pos < D, far: t-pos >= D; quotas floor(E/2) near and the
 *     rest far, a short subset gives all it has; order (score, position);
 *   - layout: Local slot = pos mod w; Global: an eviction frees the evicted
 *     slots (position -1) without moving any row, and the next tokens fill the
 *     freed slots in ascending order before the table grows; at classification
 *     an over-long Global prefix is reduced by STE with the W last prefill
 *     queries, survivors compacted in ascending position order.
 *
 * Conventions (every entry point):
 *   - Streams: s = (l*batch + b)*heads + h.  Calls on a stream range take
 *     [s_begin, s_begin + s_count); per-stream operands are addressed with the
 *     ABSOLUTE stream index: row of stream s at ptr + s*ld (ld in elements).
 *   - Pointers are device pointers unless stated; the CALLER owns every buffer.
 *     Data operands (pools, stage, q, k_new, v_new, out) must be 16-byte
 *     aligned and their row strides multiples of 16 bytes.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     is complete when that stream is.  Calls on one state must be ordered on
 *     one stream by the caller; distinct states are independent.
 *   - Every call returns hkv_status and never aborts.  Host-detectable errors
 *     return before anything is enqueued.  Invariant violations found on the
 *     device set a sticky bit in *err, reported by hkv_check.
 *   - Element type: bf16 (bit pattern in uint16) or fp32, for q, k, v and out.
 *     Scores are fp32; arithmetic is fp32.
 */
#ifndef HKV_H
#define HKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HKV_OK = 0,
  HKV_E_INVAL = -1,        /* bad config or argument (null, misaligned, range) */
  HKV_E_STATE = -2,        /* call out of order (decode before classification) */
  HKV_E_CAPACITY = -3,     /* device found a stream over its capacity          */
  HKV_E_HIP = -4,          /* HIP runtime error (launch, copy, sync)            */
  HKV_E_UNSUPPORTED = -5   /* valid but not implemented (e.g. head_dim 96)     */
} hkv_status;

typedef enum { HKV_DT_BF16 = 0, HKV_DT_F32 = 1 } hkv_dtype;
typedef enum { HKV_LOCAL = 0, HKV_GLOBAL = 1, HKV_FULL = 2 } hkv_label;

/* Ablation variants (hkv_config.variant), for equal-memory comparisons with
 * the two choices the pages credit (section "Key contributions", items 2 and 3):
 *   HKV_VARIANT_UNSTRATIFIED    eviction without the near/far split: the M
 *                               lowest (score, position) candidates over all
 *                               candidates (same protected zone, same scores);
 *   HKV_VARIANT_UNIFORM_BUDGET  every head gets the same budget A = floor(N*rho)
 *                               (the fixed uniform per-head budget the pages
 *                               ascribe to LineAR, section "Problem
 *                               definition"): Local heads a ring of A slots,
 *                               Global heads budget A.
 * Classification, scores and layout rules are otherwise unchanged. */
#define HKV_VARIANT_UNSTRATIFIED   1
#define HKV_VARIANT_UNIFORM_BUDGET 2

/* Device error bits in *err. */
#define HKV_ERRBIT_CAPACITY 1   /* append into a full Global/FULL stream          */
#define HKV_ERRBIT_LAYOUT   2   /* count/label/budget inconsistent                */
#define HKV_ERRBIT_SELECT   4   /* fewer eviction candidates than evictions       */

typedef struct {
  int32_t layers, batch, heads, head_dim;   /* head_dim in {64, 128}            */
  int32_t dtype;                            /* hkv_dtype                        */
  int32_t final_len;                        /* N: prefix + generated tokens     */
  int32_t prefill_len;                      /* P: cached length at classification */
  int32_t local_window;                     /* w                                */
  float   tau;                              /* accumulation threshold, (0, 1]   */
  int32_t rho_num, rho_den;                 /* rho as an exact fraction         */
  int32_t split_dist;                       /* D: near/far split distance       */
  int32_t w_obs;                            /* W: scoring window (queries)      */
  int32_t evict_m;                          /* M: evictions per event (== W, even) */
  int32_t full_cache;                       /* 1: uncompressed baseline layout  */
  int32_t variant;                          /* 0, or HKV_VARIANT_* bits (ablations) */
} hkv_config;

/* Cache state: device buffers owned by the caller (sizes from the helpers).
 * Index buffers must be aligned to their element size (label: 4 bytes). */
typedef struct {
  void    *k_pool, *v_pool;   /* one buffer [pool_slots, 2, head_dim] of the
                               * element type: each slot's K row, then its V
                               * row.  k_pool points at the buffer (slot 0's K
                               * row), v_pool = k_pool + head_dim elements (slot
                               * 0's V row); both rows of slot j are at
                               * 2 * head_dim * j elements past them.  Any other
                               * v_pool is rejected (HKV_E_INVAL).              */
  int32_t *pos;               /* [pool_slots] position held by each slot       */
  float   *score;             /* [pool_slots] STE scores at the last eviction  */
  int64_t *base;              /* [S] first pool slot of each stream            */
  int32_t *cap;               /* [S] slots reserved                            */
  int32_t *count;             /* [S] slots in use, including freed ones        */
  int32_t *budget;            /* [S] w (Local), B_g (Global), N (full)         */
  int32_t *n_tokens;          /* [S] classification count                      */
  uint8_t *label;             /* [S] hkv_label (4-byte aligned)                */
  int32_t *free_slots;        /* [S, max(M, 1)] slots freed by the last eviction
                                 (the decode step reads a row whatever the label) */
  int32_t *n_free;            /* [S] of those, how many are still free         */
  float   *qstat;             /* [S, w_obs, 4] per Global stream, the softmax
                               * statistics of its last w_obs decode queries:
                               * (max, 1/sum, step bits, 0), exp2 domain; written
                               * by the attention, reset by classification,
                               * 16-byte aligned                               */
  int32_t *err;               /* [1] sticky device error bits                  */
  void    *workspace;         /* hkv_workspace_bytes() bytes, 256-B aligned    */
  size_t   workspace_bytes;
  int32_t  phase;             /* host side: 0 new, 1 classified                */
} hkv_state;

/* Pool slots a state needs: S*(floor(rho*N) + M), or S*N for full_cache.
 * Label-independent, so the caller allocates before classification.  0 if the
 * config is invalid. */
size_t hkv_pool_slots(const hkv_config *cfg);

/* Workspace bytes for the state (classification scores plus the spill area for
 * Global streams too long for on-chip scratch).  0 if the config is invalid. */
size_t hkv_workspace_bytes(const hkv_config *cfg);

/* Pure host check of a configuration; no HIP call. */
hkv_status hkv_validate(const hkv_config *cfg);

/* Steps 1-2: classification and initial layout, once per generation.
 *   k_stage, v_stage: prefilled cache, stream s row p at ptr + s*ld_stage + p*head_dim
 *   q_obs: the W last prefill queries (positions P-W .. P-1), stream s row r at
 *          q_obs + s*ld_qobs + r*head_dim
 * Writes label, n_tokens, budget, cap, base, count, pos, score and the pools for
 * all S streams; sets phase = 1.  With full_cache every stream is FULL (slot =
 * position) and q_obs may be NULL. */
hkv_status hkv_classify(const hkv_config *cfg, hkv_state *st,
                        const void *k_stage, const void *v_stage, int64_t ld_stage,
                        const void *q_obs, int64_t ld_qobs, void *stream);

/* hkv_classify for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same classification and initial layout, bit for bit, with the classification
 * scores kept in a buffer the library holds per device for the life of the
 * process (32 MiB, taken when the library is first used on the device) instead
 * of the state's workspace, which may be NULL here.  Nothing is allocated and
 * no allocating routine is called.  The buffer needs S*P*4 bytes (S streams,
 * P = prefill_len): larger configurations return HKV_E_UNSUPPORTED before
 * anything is enqueued.  Every call on one device shares that buffer and keeps
 * what the last call left in it, so calls that overlap on one device (on
 * different streams, or from several threads without ordering) race; calls
 * ordered on one stream do not.  Other arguments, outputs and errors are those
 * of hkv_classify. */
hkv_status hkv_classify_noalloc(const hkv_config *cfg, hkv_state *st,
                                const void *k_stage, const void *v_stage, int64_t ld_stage,
                                const void *q_obs, int64_t ld_qobs, void *stream);

/* Steps 1-2 fused into the prefill attention (bf16): the causal attention of
 * every prefill position over the prefilled cache, written to `out` (stream s
 * row p at out + s*ld_out + p*head_dim), with the classification of
 * hkv_classify computed from the same logits, and the initial layout.  The
 * observation queries are the last W rows of q_stage, so a classification that
 * only needs the prefill pass (methodology, steps 1 and 2) adds no pass over K.
 *   q_stage: stream s query of position p at q_stage + s*ld_q + p*head_dim
 *   k_stage, v_stage: stream s row p at ptr + s*ld_stage + p*head_dim
 * Same state outputs as hkv_classify; HKV_E_UNSUPPORTED for fp32.  With
 * full_cache only the attention and the layout are done. */
hkv_status hkv_prefill(const hkv_config *cfg, hkv_state *st, const void *q_stage,
                       int64_t ld_q, const void *k_stage, const void *v_stage,
                       int64_t ld_stage, void *out, int64_t ld_out, void *stream);

/* Append token t (P <= t < N) to every stream of the range.
 * Pages: section "Methodology", step 3 — a Local head's sliding window takes the
 * newest token and drops the oldest; a Global head's cache takes every new
 * token until its budget forces an eviction (the append itself is implicit on
 * the pages).
 * Local: slot t mod w (ring; the uniform-budget variant: t mod A); Global: the
 * lowest freed slot if any, else slot `count`, with score 0; FULL: slot
 * `count`.  k_new/v_new: device rows of stream s at ptr + s*ld_kv (elements),
 * 16-byte aligned, read only.  Errors: HKV_E_STATE before classification,
 * HKV_E_INVAL for a bad t, range or pointer; appending to a full Global or FULL
 * stream sets HKV_ERRBIT_CAPACITY on the device (hkv_check). */
hkv_status hkv_append(const hkv_config *cfg, hkv_state *st, int32_t t,
                      const void *k_new, const void *v_new, int64_t ld_kv,
                      int32_t s_begin, int32_t s_count, void *stream);

/* Decode attention at step t over the slots present (the cache already holds
 * token t).
 * Pages: section "Methodology", step 3 — a Local head attends only to its
 * sliding window of the newest tokens, a Global head to the tokens its
 * Stratified Token Eviction has kept; the problem definition names the KV
 * cache read of this step as what limits decoding.
 * o = sum_j softmax_j(q.k_j / sqrt(d)) v_j over the stream's live slots, fp32
 * arithmetic, rounded to the element type.  q: device row of stream s at
 * q + s*ld_q; out: device row at out + s*ld_o (written, 4-byte aligned).  The
 * state is read only.  Errors: HKV_E_STATE before classification, HKV_E_INVAL
 * for a bad t, range or pointer. */
hkv_status hkv_decode_attn(const hkv_config *cfg, hkv_state *st, int32_t t,
                           const void *q, int64_t ld_q, void *out, int64_t ld_o,
                           int32_t s_begin, int32_t s_count, void *stream);

/* STE at step t for every Global stream of the range holding budget + M
 * tokens: score the slots, evict M (floor(M/2) near, the rest far) and free
 * their slots (free_slots, n_free = M; no row moves).
 * Pages: section "Methodology", step 3, Global heads — Stratified Token
 * Eviction splits the candidate past tokens by distance into disjoint near and
 * far subsets, scores each subset on its own from past query features and
 * evicts the lowest-scoring tokens of each (M/2 + M/2); section "Key
 * contributions", item 3, for why the split keeps distant tokens.
 *   q_win: the W most recent queries (positions t-W+1 .. t, oldest first) of
 *          stream s at q_win + s*ld_qw + r*head_dim.  A slot's score is the sum
 *          over these queries of the softmax probability it receives, each query
 *          attending to the slots whose position does not exceed its own — the
 *          probabilities the slot received during the last W decode steps.
 *          NULL: the scores are taken from st->score as stored by the caller.
 *   evicted_pos_log (optional, device, [S, M] int32): evicted positions in
 *          ascending slot order, -1 for streams that did not evict.
 * With a log, an eviction also writes the score of every slot it ranked to
 * st->score, the evicted ones included (a freed slot's score is reset to 0 when
 * a token refills it).  Errors: HKV_E_STATE before classification, HKV_E_INVAL
 * for a bad t, range or pointer; too few candidates sets HKV_ERRBIT_SELECT on
 * the device (hkv_check). */
hkv_status hkv_ste_evict(const hkv_config *cfg, hkv_state *st, int32_t t,
                         const void *q_win, int64_t ld_qw, int32_t *evicted_pos_log,
                         int32_t s_begin, int32_t s_count, void *stream);

/* One decode step in a single launch: exactly hkv_append, then hkv_decode_attn
 * with the newest query of the window (row W-1), then hkv_ste_evict with the
 * window, with identical results (bit for bit).
 * Pages: section "Methodology", step 3 — the whole per-token work of the
 * compressed decode: the Local sliding window or the Global cache takes the new
 * token, the head attends over what it keeps, and a Global head at its budget
 * runs Stratified Token Eviction.  Arguments, layouts and errors are those of
 * the three calls; k_new/v_new rows at ptr + s*ld_kv, the W-query window at
 * q_win + s*ld_qw (oldest first), out at out + s*ld_o.
 * Performance only (results do not depend on it): a launch over every stream
 * reads a fixed share of the pool, about 140 MiB, with default caching and the
 * rest with non-temporal loads, so that the share stays in the GPU's
 * memory-side cache from one step to the next; the environment variable
 * HKV_RESIDENT_MB, read once per process, sets that size (0: none).  A launch
 * over part of the streams streams everything. */
hkv_status hkv_decode_step(const hkv_config *cfg, hkv_state *st, int32_t t,
                           const void *k_new, const void *v_new, int64_t ld_kv,
                           const void *q_win, int64_t ld_qw, void *out, int64_t ld_o,
                           int32_t *evicted_pos_log, int32_t s_begin, int32_t s_count,
                           void *stream);

/* hkv_decode_step for launches with few streams, such as one layer of a model
 * (a few hundred to a thousand streams give a few workgroups per compute unit,
 * and each launch then lasts as long as its slowest stream).  Pages: section
 * "Methodology", step 3, as for hkv_decode_step, and the end-to-end speedups of
 * section "Results", which a model measures layer by layer.  Each stream's
 * table rows are spread over n_split workgroups (1 .. 8) that each leave a
 * partial softmax state in the state's workspace; a second kernel on `stream`
 * merges them into the output, writes the stream metadata back and runs the
 * eviction of due Global streams (bf16: each split scores its own slots on
 * the way, so that the second kernel only finishes the keys and selects;
 * the workspace holds those scores).  Arguments, layouts, outputs and errors are
 * those of hkv_decode_step, and so are the results except for the order of
 * floating-point sums (outputs agree to rounding; a decision changes only where
 * two scores lie that close).  Calls on one state must not overlap: the
 * partial states live in its workspace.  n_split outside [1, 8]: HKV_E_INVAL. */
hkv_status hkv_decode_step_split(const hkv_config *cfg, hkv_state *st, int32_t t,
                                 const void *k_new, const void *v_new, int64_t ld_kv,
                                 const void *q_win, int64_t ld_qw, void *out, int64_t ld_o,
                                 int32_t *evicted_pos_log, int32_t s_begin, int32_t s_count,
                                 int32_t n_split, void *stream);

/* Synchronises `stream`, reads *err and maps it: CAPACITY bit -> HKV_E_CAPACITY,
 * other bits -> HKV_E_STATE, 0 -> HKV_OK.  Does not clear the word. */
hkv_status hkv_check(const hkv_config *cfg, const hkv_state *st, void *stream);

/* Static text for a status code. */
const char *hkv_status_string(int32_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char *hkv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HKV_H */
