/*
 * Oracle for the Dustin sparse-verification path — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C computing in double precision from the same bf16
 * bits the GPU path reads.  It shares no code, header, table or helper with the HIP
 * library; only tests, the smoke check and the bench's CPU-baseline leg may load it.
 * The product path never calls it.
 *
 * Sources (page = one of the four summaries the method is described in):
 *   English Dustin summary, "Methodology" 1 "Hybrid Attention Aggregation"
 *     - the two signals (target-historical attention, draft-lookahead attention),
 *     - the fixed-size set I_verify: sinks + local window always kept, then the top-m
 *       tokens by the draft signal, then the best remaining tokens by the target signal.
 *   English Dustin summary, "Methodology" 2 (SRHs): scoring is restricted to the
 *     semantic retrieval heads.
 *   English Dustin summary, "Methodology" 3 "Verification Workflow", steps 2-4.
 *   German Vegas summary, section 2A (aggregated-logit objective, the one formula on
 *     the pages) and 2B (Collect-2-Query: only the first draft token and the bonus token).
 *
 * Every array is a host array.  bf16 values are passed as their raw 16-bit patterns.
 * Return value: 0 on success, negative on a bad argument (nothing written then).
 */
#ifndef DUSTIN_ORACLE_H
#define DUSTIN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_PROB_SUM = 0, ORACLE_LOGIT_SUM2 = 1, ORACLE_LOGIT_SUM_ALL = 2 };

/* Importance scores of one scored key stream, ADDED into acc[B][n_max].
 *   K   : [B][n_rows][d]      the stream's key rows (one head of one layer)
 *   Q   : [B][n_heads][n_q][d] the SRH queries that read this stream
 *   token i of sequence b is scored for 0 <= i < ctx_len[b] (<= n_rows, <= n_max)
 *   PROB_SUM   : for every (head, query) pair, softmax over i of scale*q.k_i, summed
 *   LOGIT_SUM2 : scale*q.k_i summed over heads and the queries {0, n_q-1} (query 0
 *                once when n_q == 1), no softmax
 *   LOGIT_SUM_ALL : scale*q.k_i summed over heads and every query j < n_q, no softmax */
int oracle_score_stream(int B, int n_rows, int n_max, const int32_t *ctx_len, int d,
                        const uint16_t *K, int n_heads, int n_q, const uint16_t *Q,
                        double scale, int mode, double *acc);

/* Hybrid budgeted selection of I_verify for every sequence.
 *   score_draft / score_target : [B][n_max]; score_draft NULL = no draft tier (m' = 0)
 *   budget, n_sink, n_window, m : [B]
 *   idx   : [B][k_max] out, ascending positions, tail filled with -1
 *   count : [B] out, = min(budget[b], ctx_len[b], k_max)                             */
int oracle_select(int B, int n_max, const int32_t *ctx_len,
                  const double *score_draft, const double *score_target,
                  const int32_t *budget, const int32_t *n_sink, const int32_t *n_window,
                  const int32_t *m, int k_max, int32_t *idx, int32_t *count);

/* Verification attention over I_b plus the causal block of new tokens.
 *   Q    : [B][n_verify][Hq][d]
 *   K, V : [B][n_cap][Hkv][d]; the n_verify new tokens of sequence b are rows
 *          ctx_len[b] .. ctx_len[b]+n_verify-1
 *   idx  : [B][k_max] selected positions (first count[b] used); NULL = dense [0, ctx_len[b])
 *   O    : [B][n_verify][Hq][d] out;  lse : [B][Hq][n_verify] out (natural log)
 *   query head h reads kv head h / (Hq / Hkv)                                          */
int oracle_verify_attn(int B, int Hq, int Hkv, int d, int n_verify,
                       const uint16_t *Q, const uint16_t *K, const uint16_t *V, int n_cap,
                       const int32_t *ctx_len, const int32_t *idx, const int32_t *count,
                       int k_max, double scale, double *O, double *lse);

/* Attention recovery: the share of full-cache attention probability that falls on the
 * kept set.  For (b, h, t) the dense softmax runs over [0, ctx_len[b]) and the new tokens
 * 0..t; rec[b][h][t] is its sum over I_b (idx[b][0..count[b])) and the new tokens 0..t.
 *   Q : [B][n_verify][Hq][d];  K : [B][n_cap][Hkv][d];  rec : [B][Hq][n_verify] out     */
int oracle_attn_recovery(int B, int Hq, int Hkv, int d, int n_verify,
                         const uint16_t *Q, const uint16_t *K, int n_cap,
                         const int32_t *ctx_len, const int32_t *idx, const int32_t *count,
                         int k_max, double scale, double *rec);

/* The block of n_new tokens being verified, written into the caches behind the
 * committed context: row ctx_len[b] + j of K and V (all heads) <- row j of Knew / Vnew.
 * Nothing else changes and ctx_len is not advanced.
 *   Knew, Vnew : [B][n_new][Hkv][d];  K, V : [B][n_cap][Hkv][d] (in/out)                */
int oracle_kv_write_block(int B, int Hkv, int d, int n_new, const uint16_t *Knew,
                          const uint16_t *Vnew, const int32_t *ctx_len, uint16_t *K,
                          uint16_t *V, int n_cap);

/* Commit after verification: the block's first row and its first n_accept[b] draft rows
 * are kept, the rest are discarded.  ctx_len[b] += 1 + n_accept[b] (in/out),
 * 0 <= n_accept[b] <= n_new - 1.                                                        */
int oracle_kv_commit(int B, int n_new, const int32_t *n_accept, int32_t *ctx_len);

#ifdef __cplusplus
}
#endif
#endif
