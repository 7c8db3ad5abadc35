/*
 * dustin.h — C ABI of the MI355X (gfx950) sparse-verification library.
 *
 * The calls follow the steps of the verification workflow in the English
 * Dustin summary ("Methodology" 3, steps 2-5):
 *   dustin_srh_score          step 2: the importance map, computed from the semantic
 *                             retrieval heads only ("Methodology" 1 and 2)
 *   dustin_select             step 3: the fixed-size verification set I_verify
 *                             ("Methodology" 1, last two sentences)
 *   dustin_sparse_verify_attn step 4: the target verifies the draft block against the
 *                             selected tokens only
 *   dense_verify_attn         the full-cache verification it replaces ("Problem
 *                             Statement": the target loads the full KV cache)
 *   dustin_kv_write_block,    step 5: the verified block in the cache, and the cache
 *   dustin_kv_commit          length advanced over the drafts the target kept
 *   dustin_attn_recovery      the share of full-cache attention mass the kept set
 *                             carries ("Methodology" 2: attention recovery rate)
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked (host).  bf16 data are raw 16-bit
 *     patterns; every bf16 row (head_dim elements) is contiguous and 16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  No call
 *     allocates device memory, synchronises, or copies between host and device.
 *   - Arguments are validated on the host before anything is enqueued; on error the
 *     call returns a negative status and enqueues nothing (outputs untouched).
 *   - Device-resident values (ctx_len, budget, idx, count, page tables, ...) cannot be
 *     checked without a sync; kernels clamp each of them into range instead, so no
 *     value can make a kernel read or write out of bounds.  Results for out-of-range
 *     values are defined by that clamping, not by the method.
 *   - The library keeps no state between calls.  Calls that share a workspace must be
 *     ordered on one stream.
 *   - Two environment variables tune the attention calls (for experiments and tests;
 *     values other than those listed are ignored):
 *       DUSTIN_ATTN_TARGET_WGS  a positive integer: workgroups per round of the attention
 *                               grid (default: the device's compute units).  It changes the split plan, so
 *                               the workspace size and the order of the partial sums;
 *                               set it before the size queries (a workspace smaller than
 *                               the plan needs is rejected with DUSTIN_ERR_WORKSPACE).
 *       DUSTIN_ATTN_FUSED_MERGE "1": the budget splits of one (sequence, KV head) are
 *                               combined by the workgroup that finishes last, in the
 *                               attention kernel itself; "0" (the default): by a second
 *                               kernel.  Both give bit-identical results.
 */
#ifndef DUSTIN_H
#define DUSTIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DUSTIN_OK = 0,
    DUSTIN_ERR_INVALID_ARG = -1, /* null pointer, bad size, stride or alignment        */
    DUSTIN_ERR_WORKSPACE = -2,   /* workspace missing or smaller than the size query  */
    DUSTIN_ERR_UNSUPPORTED = -3, /* a shape outside what the kernels are built for    */
    DUSTIN_ERR_HIP = -4,         /* the HIP runtime reported an error at launch        */
    DUSTIN_ERR_SCRATCH = -5      /* the no-allocation call would need more than the
                                    library's static scratch array holds               */
} dustin_status;

/* Scoring modes of dustin_srh_score. */
enum {
    /* Sum over every (SRH query head, query) pair of the softmax probability of the
       token under that pair (English Dustin summary, "Methodology" 1: attention scores
       of the target-historical and draft-lookahead queries form the importance map). */
    DUSTIN_SCORE_PROB_SUM = 0,
    /* Sum over the SRH query heads and over the queries {0, n_q-1} of the scaled
       pre-softmax logit (German Vegas summary, 2A formula restricted to the first and
       the bonus query of 2B, "Collect-2-Query").  Query 0 counts once when n_q == 1.  */
    DUSTIN_SCORE_LOGIT_SUM2 = 1,
    /* Sum over the SRH query heads and over every query j < n_q of the scaled
       pre-softmax logit (German Vegas summary, 2A formula as stated: the aggregate over
       all queries and heads).  Equal to LOGIT_SUM2 when n_q <= 2.                     */
    DUSTIN_SCORE_LOGIT_SUM_ALL = 2
};

/* A bf16 K or V cache of one layer, contiguous or paged.
 *   contiguous: row(b, t, h) = base + b*stride_batch + t*stride_token + h*stride_head
 *               for 0 <= t < n_tokens
 *   paged     : row(b, t, h) = base + page_table[b*max_pages + t/page_size]*stride_page
 *                                   + (t % page_size)*stride_token + h*stride_head
 *               for 0 <= t < max_pages*page_size; page ids are clamped to [0, num_pages)
 * Strides are in elements, multiples of 8 (16-byte rows).  The gamma+1 tokens being
 * verified must already be stored at positions ctx_len[b] .. ctx_len[b]+gamma. */
typedef struct {
    const void *base;
    int64_t stride_batch;        /* unused when paged                                  */
    int64_t stride_token;
    int64_t stride_head;
    int32_t n_tokens;            /* contiguous: tokens addressable per sequence        */
    int32_t n_heads;             /* KV heads stored in the view                        */
    const int32_t *page_table;   /* NULL = contiguous; else [B][max_pages] (device)    */
    int64_t stride_page;
    int32_t page_size;           /* power of two                                       */
    int32_t max_pages;
    int32_t num_pages;
} dustin_kv_view;

/* One scored stream: the K cache of one model layer, one of its KV heads, and the
 * number of SRH query heads that read that KV head. */
typedef struct {
    dustin_kv_view k;
    int32_t kv_head;
    int32_t n_qheads;
} dustin_srh_group;

const char *dustin_status_string(dustin_status s);

/* ---------------------------------------------------------------------------------
 * Step 2 — SRH importance scoring.
 * For every sequence b and token i < ctx_len[b] (clamped to [0, n_max] and to each
 * view's capacity):
 *   PROB_SUM   score[b][i] = sum over groups g, query heads h of g, queries j < n_q of
 *                            softmax_i(scale * q[b][h][j] . K_g[b][i])
 *   LOGIT_SUM2 score[b][i] = sum over groups, heads, j in {0, n_q-1} of
 *                            scale * q[b][h][j] . K_g[b][i]
 *   LOGIT_SUM_ALL           the same sum over every j < n_q
 * score[b][i] = 0 for ctx_len[b] <= i < n_max.  One call scores one signal (the draft
 * lookahead queries, or the target-historical queries); the softmax runs over the
 * committed context [0, ctx_len[b]).
 *   groups : (host) [n_groups], 1 <= n_groups <= 16; all groups share head_dim
 *   q      : bf16 [B][sum of n_qheads][n_q][head_dim], heads in group order
 *   scale  : any finite value (0 and negative included); non-finite -> INVALID_ARG
 *   head_dim in {64, 128}; 1 <= n_q <= 16; pairs per group (n_qheads * queries used)
 *   at most 16 in PROB_SUM mode and 64 in the logit-sum modes
 *   score  : fp32 [B][n_max], fully written; 16-byte aligned (else INVALID_ARG)
 *   workspace: at least dustin_srh_score_workspace_size(...) bytes, any contents
 * ------------------------------------------------------------------------------- */
dustin_status dustin_srh_score_workspace_size(int B, int n_max, int total_qheads, int n_q,
                                              int mode, size_t *bytes /* host */);
dustin_status dustin_srh_score(int B, int n_max, const int32_t *ctx_len, int n_groups,
                               const dustin_srh_group *groups /* host */, int head_dim,
                               const void *q, int n_q, float scale, int mode, float *score,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Both signals in one call (the draft lookahead and the target historical queries score
 * the same contexts): the softmax-mode signals share one logit launch and every signal one
 * finalize launch, so the launch ramp and tail are paid once.  Each signal's results are
 * those of a dustin_srh_score call with its own arguments, up to the rounding order of the
 * per-workgroup statistics (the grid is shared, so a stream's tiles fall into different
 * workgroup shares); every argument rule of dustin_srh_score applies per signal.
 *   signals   : (host) [n_signals], 1 <= n_signals <= 2; at most 16 groups in all
 *   workspace : dustin_srh_score_signals_workspace_size(...) bytes, 16-byte aligned
 */
typedef struct {
    int32_t n_groups;
    const dustin_srh_group *groups; /* host [n_groups]                                   */
    int32_t head_dim;               /* 64 or 128, shared by the signal's groups           */
    const void *q;                  /* bf16 [B][sum of n_qheads][n_q][head_dim]           */
    int32_t n_q;
    float scale;
    int32_t mode;                   /* DUSTIN_SCORE_*                                     */
    float *score;                   /* fp32 [B][n_max], fully written                     */
} dustin_srh_signal;

dustin_status dustin_srh_score_signals_workspace_size(int B, int n_max, int n_signals,
                                                      const dustin_srh_signal *signals /* host */,
                                                      size_t *bytes /* host */);
dustin_status dustin_srh_score_signals(int B, int n_max, const int32_t *ctx_len, int n_signals,
                                       const dustin_srh_signal *signals /* host */, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Step 3 — hybrid budgeted selection of I_verify.
 * Per sequence b, with N = ctx_len[b] clamped to [0, n_max] and
 * k = min(budget[b], N, k_max):
 *   k == N : I = [0, N)
 *   else   : s = min(n_sink[b], k); w = min(n_window[b], k - s)
 *            P = [0, s) u [N - w, N)                     (always kept)
 *            m' = min(m[b], k - |P|)                     (0 when score_draft is NULL)
 *            D = the m' best tokens of [0,N) \ P by score_draft
 *            T = the k - |P| - m' best tokens of [0,N) \ (P u D) by score_target
 *            I = P u D u T
 *   "best": larger score first, then smaller position; -0 equals +0.  NaN scores are
 *   outside the contract.
 *   idx   : int32 [B][k_max] ascending positions, entries count[b].. set to -1
 *   count : int32 [B] = |I|
 *   budget, n_sink, n_window, m : int32 [B] (negative values act as 0)
 *   score_draft, score_target : fp32 [B][n_max], 16-byte aligned (else INVALID_ARG)
 *   n_max <= 65536.
 *   workspace: NULL, or dustin_select_workspace_size(...) bytes (B x (16 KiB + 8)),
 *   16-byte aligned, any contents on the first call (else DUSTIN_ERR_WORKSPACE).  With a
 *   workspace, a sequence whose two tiers are both non-empty (and |D| + |T| <= 4096) runs
 *   them on two workgroups at once: the best |T| of the best |D| + |T| candidates by
 *   score_target that are not in D are exactly T.  Each workgroup publishes its tier's
 *   position mask and counts itself in on the sequence's arrival counter (recognised by
 *   a 40-bit tag, left cleared by the call); the second to arrive combines the two.
 *   Without a workspace, one workgroup runs both tiers in turn; the result is the same
 *   set either way.
 * ------------------------------------------------------------------------------- */
dustin_status dustin_select_workspace_size(int B, int n_max, size_t *bytes /* host */);
dustin_status dustin_select(int B, int n_max, const int32_t *ctx_len, const float *score_draft,
                            const float *score_target, const int32_t *budget,
                            const int32_t *n_sink, const int32_t *n_window, const int32_t *m,
                            int k_max, int32_t *idx, int32_t *count, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Step 4 — verification attention over the selected tokens.
 * For sequence b, verify query t (0 <= t < n_verify) and query head h (KV head
 * g = h / (Hq/Hkv)), the attended set is I_b u {ctx_len[b] + j : 0 <= j <= t} with
 * I_b = idx[b][0 .. count[b]) (count clamped to [0, k_max], positions clamped to
 * [0, ctx_len[b])):
 *   out[b][t][h] = sum_x softmax_x(scale * q[b][t][h] . K[b][x][g]) V[b][x][g]
 *   lse[b][h][t] = ln sum_x exp(scale * q[b][t][h] . K[b][x][g])
 *   q, out : bf16 [B][n_verify][Hq][head_dim];  lse : fp32 [B][Hq][n_verify]
 *   scale  : any finite value (0 and negative included); non-finite -> INVALID_ARG
 *   head_dim in {64, 128}; 1 <= n_verify <= 16; Hq % Hkv == 0;
 *   k_max + n_verify (dense: n_max + n_verify) <= 131072
 *   workspace: dustin_sparse_verify_attn_workspace_size(...) bytes, 16-byte aligned, any
 *   contents on the first call (it holds the partial results of the budget splits and
 *   one arrival counter per (sequence, KV head, query group); a counter is recognised
 *   by a 40-bit tag and left cleared by the call that used it).
 *   Paged views (and contiguous views next to a paged one): every page and batch stride
 *   must be a multiple of stride_token and the rows addressed below 2^32 rows, else
 *   DUSTIN_ERR_UNSUPPORTED.
 * dense_verify_attn is the same with I_b = [0, ctx_len[b]); n_max bounds ctx_len.
 * ------------------------------------------------------------------------------- */
dustin_status dustin_sparse_verify_attn_workspace_size(int B, int Hq, int Hkv, int head_dim,
                                                       int n_verify, int k_max,
                                                       size_t *bytes /* host */);
dustin_status dustin_sparse_verify_attn(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                        const void *q, const dustin_kv_view *k /* host */,
                                        const dustin_kv_view *v /* host */,
                                        const int32_t *ctx_len, const int32_t *idx,
                                        const int32_t *count, int k_max, float scale,
                                        void *out, float *lse, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* dustin_sparse_verify_attn_logits — dustin_sparse_verify_attn that also writes the
 * Collect-2 signal of the selected tokens as a by-product of verification (German Vegas
 * summary, 2B "Collect-2-Query" and 3 "Kernel-Instrumentierung": the verification kernel
 * itself hands out the pre-softmax logits of the first and the bonus verify query):
 *   logit_sum2[b][g][j] = sum over the query heads h of KV head g and t in {0, n_verify-1}
 *                         (t = 0 once when n_verify == 1) of scale * q[b][t][h] . K[b][i][g]
 *   for list entries j < count[b] (clamped as in the attention), i = idx[b][j] (clamped);
 *   entries j >= count[b] are not written.
 *   logit_sum2 : fp32 [B][Hkv][k_max], 4-byte aligned (else INVALID_ARG).
 * The other arguments, results and errors are those of dustin_sparse_verify_attn, with
 * the same workspace; a shape whose query rows per KV head (Hq/Hkv * n_verify) exceed 80
 * returns DUSTIN_ERR_UNSUPPORTED (each (sequence, KV head) must fit one workgroup).
 */
dustin_status dustin_sparse_verify_attn_logits(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                               const void *q, const dustin_kv_view *k /* host */,
                                               const dustin_kv_view *v /* host */,
                                               const int32_t *ctx_len, const int32_t *idx,
                                               const int32_t *count, int k_max, float scale,
                                               void *out, float *lse, float *logit_sum2,
                                               void *workspace, size_t workspace_bytes, void *stream);

/* dustin_attn_plan — the launch plan the attention calls use for these sizes, for tools
 * that name the kernels they time.  n_positions: k_max (sparse) or n_max (dense).
 * layout: 0 = a sparse list, or paged views whose K and V rows sit at the same offsets;
 * 1 = paged views with K and V rows at different offsets; 2 = dense over unpaged views.
 *   plan (host int32 [5]): [0] 16-row query tiles per workgroup (the kernels' QT),
 *   [1] query groups per (sequence, KV head), [2] splits of the position list,
 *   [3] workgroups of the attention kernel, [4] how the splits are combined: 0 not at all
 *   (one split), 1 by a second kernel, 2 inside the attention kernel
 *   (DUSTIN_ATTN_FUSED_MERGE=1).  Errors as in the workspace-size queries.
 */
dustin_status dustin_attn_plan(int B, int Hq, int Hkv, int head_dim, int n_verify, int n_positions, int layout,
                               int32_t *plan /* host */);

/* dustin_sparse_verify_attn_noalloc — for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * dustin_sparse_verify_attn with the same arguments, results and errors, minus the
 * workspace.  The split partials and arrival counters live in a static device array of
 * DUSTIN_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from the first
 * call on that device until the process ends.  The call allocates nothing.
 *   - A shape whose dustin_sparse_verify_attn_workspace_size exceeds
 *     DUSTIN_NOALLOC_SCRATCH_BYTES returns DUSTIN_ERR_SCRATCH and enqueues nothing.
 *   - The call uses the scratch of the CURRENT device; a non-NULL stream of another
 *     device returns DUSTIN_ERR_INVALID_ARG.
 *   - Every call on one device shares that array and leaves the last call's contents in
 *     it (partials are always written before they are read; the counters are left
 *     cleared).  Calls that may overlap on one device (different streams, host threads)
 *     race on it: order them on one stream.
 */
#define DUSTIN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
dustin_status dustin_sparse_verify_attn_noalloc(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                                const void *q, const dustin_kv_view *k /* host */,
                                                const dustin_kv_view *v /* host */,
                                                const int32_t *ctx_len, const int32_t *idx,
                                                const int32_t *count, int k_max, float scale,
                                                void *out, float *lse, void *stream);

/* dustin_gather_floor — a measurement call for tools that rate the verification
 * attention against its memory ceiling (the English Dustin summary's "Problem Statement":
 * memory access sets the latency): it reads exactly the K and V row slices of the list
 * entries that dustin_sparse_verify_attn reads for them, and computes nothing.  For every
 * sequence b, KV head g and list entry j < k_max it reads the head_dim bf16 elements of
 * K[b][i][g] and V[b][i][g], i = idx[b][j] clamped to [0, min(k->n_tokens, v->n_tokens)),
 * with 16-byte non-temporal loads and every row of a workgroup's 512 entries in flight at
 * once (when k_max is not a multiple of 512, the last workgroup's lanes past k_max re-read
 * entry k_max - 1's rows, which the cache serves, and leave them out of the checksum).
 * Its time per launch is the gather floor for those bytes as they lie in memory.
 *   idx      : int32 [B][k_max] (device); every entry is read, whatever the list count
 *   k, v     : contiguous (unpaged) views; paged -> DUSTIN_ERR_UNSUPPORTED
 *   head_dim : 64 or 128
 *   checksum : uint32 [B][Hkv] (device, 4-byte aligned).  mode 1: XOR of every 32-bit
 *              word read for (b, g) is XOR-ed into checksum[b][g] (zero it first to get
 *              the XOR itself).  mode 0 (timing): left unchanged, except that a
 *              workgroup lane whose own XOR equals 0x9e3779b9 stores it there (the store
 *              keeps the loads; with real data it practically never happens).
 * B == 0 or k_max == 0 enqueues nothing. */
dustin_status dustin_gather_floor(int B, int Hkv, int head_dim, const dustin_kv_view *k /* host */,
                                  const dustin_kv_view *v /* host */, const int32_t *idx, int k_max,
                                  uint32_t *checksum, int mode, void *stream);

dustin_status dense_verify_attn_workspace_size(int B, int Hq, int Hkv, int head_dim,
                                               int n_verify, int n_max,
                                               size_t *bytes /* host */);
dustin_status dense_verify_attn(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                const void *q, const dustin_kv_view *k /* host */,
                                const dustin_kv_view *v /* host */, const int32_t *ctx_len,
                                int n_max, float scale, void *out, float *lse,
                                void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Step 5 — the verified block in the cache (English Dustin summary, Verification
 * Workflow step 5: the cache after the target's decision on the drafts).
 *
 * dustin_kv_write_block stores the block being verified behind the committed context,
 * where dustin_sparse_verify_attn and dense_verify_attn read the new tokens:
 *   K[b][ctx_len[b] + j][g] = k_new[b][j][g] and V likewise, for j < n_new, g < Hkv
 *   k_new, v_new : bf16 [B][n_new][Hkv][head_dim], contiguous, 16-byte aligned
 *   k, v         : (host) views of the two caches.  The call WRITES through them (their
 *                  base pointers are const in the struct because every other call only
 *                  reads); the K and V caches must not overlap.
 *   ctx_len[b] is clamped to [0, min(capacity of k, capacity of v) - n_new] and is not
 *   changed.  head_dim in {64, 128}; 1 <= n_new <= 16.
 *
 * dustin_kv_commit runs once verification has decided: the block's first row (the token
 * produced by the previous step) and its first n_accept[b] draft rows are kept, the rows
 * behind the new length are discarded (the next block overwrites them):
 *   ctx_len[b] <- clamp(ctx_len[b], 0, 2^30) + 1 + clamp(n_accept[b], 0, n_new - 1)
 *   n_accept, ctx_len : int32 [B] (device; ctx_len in/out); 1 <= n_new <= 16
 * ------------------------------------------------------------------------------- */
dustin_status dustin_kv_write_block(int B, int Hkv, int head_dim, int n_new, const void *k_new,
                                    const void *v_new, const int32_t *ctx_len,
                                    const dustin_kv_view *k /* host */,
                                    const dustin_kv_view *v /* host */, void *stream);
dustin_status dustin_kv_commit(int B, int n_new, const int32_t *n_accept, int32_t *ctx_len,
                               void *stream);

/* ---------------------------------------------------------------------------------
 * Attention recovery.  The English Dustin summary ("Methodology" 2) picks its SRHs to
 * maximise an attention recovery rate that it does not define; read here as the share of
 * the full-cache attention probability that falls on the kept set.  Given the lse of a
 * dustin_sparse_verify_attn call and of a dense_verify_attn call on the same queries and
 * caches (both natural logs of their softmax normalisers), that share is
 *   rec[i] = exp(lse_sparse[i] - lse_dense[i]),   0 <= i < n
 * for every (b, h, t) of the [B][Hq][n_verify] layout.  All arrays fp32, device.
 * ------------------------------------------------------------------------------- */
dustin_status dustin_attn_recovery(int n, const float *lse_sparse, const float *lse_dense,
                                   float *rec, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DUSTIN_H */
