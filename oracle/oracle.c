/*
 * Oracle for the Dustin sparse-verification path — TEST INFRASTRUCTURE ONLY.
 * Plain single-threaded C in double precision.  See oracle.h for the sources and the
 * contract of each function.  Nothing here is blocked, fused or reordered beyond what
 * the definitions say; built with -O2 -ffp-contract=off so no multiply-add is fused.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top half of an IEEE binary32; widen it exactly. */
static double bf(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double dot_bf16(const uint16_t *a, const uint16_t *b, int d)
{
    double s = 0.0;
    for (int i = 0; i < d; ++i)
        s += bf(a[i]) * bf(b[i]);
    return s;
}

/* ------------------------------------------------------------------------------------
 * Scoring.  English Dustin summary, Methodology 1 (target-historical and draft-lookahead
 * attention scores aggregated into one importance map) and Methodology 2 (only the SRHs
 * are scored).  The attention score of a context token under one (head, query) pair is
 * its softmax probability over the scored context; the map sums those probabilities.
 * LOGIT_SUM_ALL is the objective of the German Vegas summary 2A as it stands: raw logits
 * summed over every query and every head.  LOGIT_SUM2 restricts it to the two queries of
 * 2B (first draft token, bonus token).
 * ---------------------------------------------------------------------------------- */
int oracle_score_stream(int B, int n_rows, int n_max, const int32_t *ctx_len, int d,
                        const uint16_t *K, int n_heads, int n_q, const uint16_t *Q,
                        double scale, int mode, double *acc)
{
    if (B < 0 || n_rows < 0 || n_max < 0 || d <= 0 || n_heads < 0 || n_q <= 0 || !ctx_len ||
        !acc || (mode != ORACLE_PROB_SUM && mode != ORACLE_LOGIT_SUM2 && mode != ORACLE_LOGIT_SUM_ALL))
        return -1;
    double *logit = (double *)malloc(sizeof(double) * (size_t)(n_max > 0 ? n_max : 1));
    if (!logit)
        return -2;
    for (int b = 0; b < B; ++b) {
        int n = ctx_len[b];
        if (n < 0 || n > n_rows || n > n_max) {
            free(logit);
            return -1;
        }
        const uint16_t *Kb = K + (size_t)b * n_rows * d;
        for (int h = 0; h < n_heads; ++h) {
            for (int j = 0; j < n_q; ++j) {
                if (mode == ORACLE_LOGIT_SUM2 && j != 0 && j != n_q - 1)
                    continue;
                const uint16_t *q = Q + (((size_t)b * n_heads + h) * n_q + j) * d;
                for (int i = 0; i < n; ++i)
                    logit[i] = scale * dot_bf16(q, Kb + (size_t)i * d, d);
                double *out = acc + (size_t)b * n_max;
                if (mode != ORACLE_PROB_SUM) {
                    for (int i = 0; i < n; ++i)
                        out[i] += logit[i];
                    continue;
                }
                if (n == 0)
                    continue;
                double mx = logit[0];
                for (int i = 1; i < n; ++i)
                    if (logit[i] > mx)
                        mx = logit[i];
                double z = 0.0;
                for (int i = 0; i < n; ++i)
                    z += exp(logit[i] - mx);
                for (int i = 0; i < n; ++i)
                    out[i] += exp(logit[i] - mx) / z;
            }
        }
    }
    free(logit);
    return 0;
}

/* ------------------------------------------------------------------------------------
 * Selection.  English Dustin summary, Methodology 1, last two sentences: a fixed-size
 * set; a small prefix of attention sinks and a local window of recent tokens are always
 * kept; the rest of the budget is filled first with the top-m tokens by the draft signal,
 * then with the most relevant REMAINING tokens by the target signal.
 * "Best" = larger score, ties to the smaller position (the pages give no tie rule).
 * ---------------------------------------------------------------------------------- */
typedef struct {
    double s;
    int32_t i;
} cand;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand *a = (const cand *)pa, *b = (const cand *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

int oracle_select(int B, int n_max, const int32_t *ctx_len,
                  const double *score_draft, const double *score_target,
                  const int32_t *budget, const int32_t *n_sink, const int32_t *n_window,
                  const int32_t *m, int k_max, int32_t *idx, int32_t *count)
{
    if (B < 0 || n_max < 0 || k_max < 0 || !ctx_len || !score_target || !budget || !n_sink ||
        !n_window || !m || !idx || !count)
        return -1;
    cand *c = (cand *)malloc(sizeof(cand) * (size_t)(n_max > 0 ? n_max : 1));
    unsigned char *in = (unsigned char *)malloc((size_t)(n_max > 0 ? n_max : 1));
    if (!c || !in) {
        free(c);
        free(in);
        return -2;
    }
    for (int b = 0; b < B; ++b) {
        int N = clampi(ctx_len[b], 0, n_max);
        int k = clampi(budget[b], 0, N < k_max ? N : k_max);
        memset(in, 0, (size_t)(n_max > 0 ? n_max : 1));
        if (k == N) {
            for (int i = 0; i < N; ++i)
                in[i] = 1;
        } else {
            /* protected prefix and window; if they exceed the budget, sinks win first,
               then the most recent window tokens (k < N here, so the two never overlap) */
            int s = clampi(n_sink[b], 0, k);
            int w = clampi(n_window[b], 0, k - s);
            for (int i = 0; i < s; ++i)
                in[i] = 1;
            for (int i = N - w; i < N; ++i)
                in[i] = 1;
            int p = s + w;
            int md = score_draft ? clampi(m[b], 0, k - p) : 0; /* no draft signal: no draft tier */
            int r = k - p - md;
            /* tier 1: top-md by the draft score among the unprotected tokens */
            if (md > 0) {
                const double *sd = score_draft + (size_t)b * n_max;
                int nc = 0;
                for (int i = 0; i < N; ++i)
                    if (!in[i]) {
                        c[nc].s = sd[i];
                        c[nc].i = i;
                        ++nc;
                    }
                qsort(c, (size_t)nc, sizeof(cand), cand_cmp);
                for (int j = 0; j < md; ++j)
                    in[c[j].i] = 1;
            }
            /* tier 2: top-r by the target score among what is still unselected */
            if (r > 0) {
                const double *st = score_target + (size_t)b * n_max;
                int nc = 0;
                for (int i = 0; i < N; ++i)
                    if (!in[i]) {
                        c[nc].s = st[i];
                        c[nc].i = i;
                        ++nc;
                    }
                qsort(c, (size_t)nc, sizeof(cand), cand_cmp);
                for (int j = 0; j < r; ++j)
                    in[c[j].i] = 1;
            }
        }
        int o = 0;
        int32_t *row = idx + (size_t)b * k_max;
        for (int i = 0; i < N; ++i)
            if (in[i])
                row[o++] = i;
        count[b] = o;
        for (int j = o; j < k_max; ++j)
            row[j] = -1;
    }
    free(c);
    free(in);
    return 0;
}

/* ------------------------------------------------------------------------------------
 * Verification attention.  English Dustin summary, Verification Workflow steps 3-4: the
 * target verifies the draft tokens against a cache formed from the selected tokens only.
 * Verify query t also sees the new tokens 0..t (its own causal block).  Plain softmax
 * attention: O = sum_x e^{s_x - M} v_x / sum_x e^{s_x - M}, LSE = M + ln sum_x e^{s_x - M}.
 * ---------------------------------------------------------------------------------- */
int oracle_verify_attn(int B, int Hq, int Hkv, int d, int n_verify,
                       const uint16_t *Q, const uint16_t *K, const uint16_t *V, int n_cap,
                       const int32_t *ctx_len, const int32_t *idx, const int32_t *count,
                       int k_max, double scale, double *O, double *lse)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || n_verify <= 0 || !Q || !K ||
        !V || !ctx_len || !O || !lse || (idx && !count))
        return -1;
    int G = Hq / Hkv;
    int cap = (n_cap > k_max ? n_cap : k_max) + n_verify;
    int *set = (int *)malloc(sizeof(int) * (size_t)cap);
    double *s = (double *)malloc(sizeof(double) * (size_t)cap);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    if (!set || !s || !acc) {
        free(set);
        free(s);
        free(acc);
        return -2;
    }
    int rc = 0;
    for (int b = 0; b < B && !rc; ++b) {
        int N = ctx_len[b];
        if (N < 0 || N + n_verify > n_cap) {
            rc = -1;
            break;
        }
        int n_sel;
        if (idx) {
            n_sel = count[b];
            if (n_sel < 0 || n_sel > k_max) {
                rc = -1;
                break;
            }
            for (int j = 0; j < n_sel; ++j) {
                int x = idx[(size_t)b * k_max + j];
                if (x < 0 || x >= N) {
                    rc = -1;
                    break;
                }
                set[j] = x;
            }
            if (rc)
                break;
        } else {
            n_sel = N;
            for (int j = 0; j < N; ++j)
                set[j] = j;
        }
        for (int t = 0; t < n_verify; ++t) {
            int n_set = n_sel + t + 1; /* the causal block: new tokens 0..t */
            for (int j = 0; j <= t; ++j)
                set[n_sel + j] = N + j;
            for (int h = 0; h < Hq; ++h) {
                int g = h / G;
                const uint16_t *q = Q + (((size_t)b * n_verify + t) * Hq + h) * d;
                double mx = -INFINITY;
                for (int j = 0; j < n_set; ++j) {
                    const uint16_t *kr = K + (((size_t)b * n_cap + set[j]) * Hkv + g) * d;
                    s[j] = scale * dot_bf16(q, kr, d);
                    if (s[j] > mx)
                        mx = s[j];
                }
                double z = 0.0;
                for (int e = 0; e < d; ++e)
                    acc[e] = 0.0;
                for (int j = 0; j < n_set; ++j) {
                    double p = exp(s[j] - mx);
                    z += p;
                    const uint16_t *vr = V + (((size_t)b * n_cap + set[j]) * Hkv + g) * d;
                    for (int e = 0; e < d; ++e)
                        acc[e] += p * bf(vr[e]);
                }
                double *o = O + (((size_t)b * n_verify + t) * Hq + h) * d;
                for (int e = 0; e < d; ++e)
                    o[e] = acc[e] / z;
                lse[((size_t)b * Hq + h) * n_verify + t] = mx + log(z);
            }
        }
    }
    free(set);
    free(s);
    free(acc);
    return rc;
}

/* ------------------------------------------------------------------------------------
 * Attention recovery.  The English Dustin summary ("Methodology" 2) picks its SRHs by an
 * Attention Recovery Rate that it names but does not define; the plain reading taken
 * here is the share of the full-cache attention probability that the kept set carries.
 * For every (b, h, t): the dense probabilities over [0, N) and the new tokens 0..t, then
 * their sum over I_b and the new tokens (which both attentions see).
 * ---------------------------------------------------------------------------------- */
int oracle_attn_recovery(int B, int Hq, int Hkv, int d, int n_verify,
                         const uint16_t *Q, const uint16_t *K, int n_cap,
                         const int32_t *ctx_len, const int32_t *idx, const int32_t *count,
                         int k_max, double scale, double *rec)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || n_verify <= 0 || !Q || !K ||
        !ctx_len || !idx || !count || !rec || k_max < 0 || n_cap < n_verify)
        return -1;
    int G = Hq / Hkv;
    double *s = (double *)malloc(sizeof(double) * (size_t)n_cap);
    unsigned char *kept = (unsigned char *)malloc((size_t)n_cap);
    if (!s || !kept) {
        free(s);
        free(kept);
        return -2;
    }
    int rc = 0;
    for (int b = 0; b < B && !rc; ++b) {
        int N = ctx_len[b];
        int n_sel = count[b];
        if (N < 0 || N + n_verify > n_cap || n_sel < 0 || n_sel > k_max) {
            rc = -1;
            break;
        }
        memset(kept, 0, (size_t)n_cap);
        for (int j = 0; j < n_sel; ++j) {
            int x = idx[(size_t)b * k_max + j];
            if (x < 0 || x >= N) {
                rc = -1;
                break;
            }
            kept[x] = 1;
        }
        if (rc)
            break;
        for (int t = 0; t < n_verify; ++t) {
            int n_all = N + t + 1; /* the context, then the new tokens 0..t */
            for (int h = 0; h < Hq; ++h) {
                int g = h / G;
                const uint16_t *q = Q + (((size_t)b * n_verify + t) * Hq + h) * d;
                double mx = -INFINITY;
                for (int x = 0; x < n_all; ++x) {
                    s[x] = scale * dot_bf16(q, K + (((size_t)b * n_cap + x) * Hkv + g) * d, d);
                    if (s[x] > mx)
                        mx = s[x];
                }
                double z = 0.0, kz = 0.0;
                for (int x = 0; x < n_all; ++x) {
                    double p = exp(s[x] - mx);
                    z += p;
                    if (x >= N || kept[x])
                        kz += p;
                }
                rec[((size_t)b * Hq + h) * n_verify + t] = kz / z;
            }
        }
    }
    free(s);
    free(kept);
    return rc;
}

/* ------------------------------------------------------------------------------------
 * KV block write and commit.  English Dustin summary, Verification Workflow step 5:
 * accepted tokens are appended to the cache and rejected ones discarded.  The block
 * being verified is stored behind the committed context (where step 4 reads the new
 * tokens); the commit then advances the context over the rows that are kept.  The block's
 * first row is the token produced by the previous step and is always kept; each accepted
 * draft token keeps one more row.  Rows behind the new context length are discarded
 * (the next block overwrites them).
 * ---------------------------------------------------------------------------------- */
int oracle_kv_write_block(int B, int Hkv, int d, int n_new, const uint16_t *Knew,
                          const uint16_t *Vnew, const int32_t *ctx_len, uint16_t *K,
                          uint16_t *V, int n_cap)
{
    if (B < 0 || Hkv <= 0 || d <= 0 || n_new < 0 || !Knew || !Vnew || !ctx_len || !K || !V)
        return -1;
    for (int b = 0; b < B; ++b)
        if (ctx_len[b] < 0 || ctx_len[b] + n_new > n_cap)
            return -1;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < n_new; ++j)
            for (int g = 0; g < Hkv; ++g)
                for (int e = 0; e < d; ++e) {
                    size_t src = (((size_t)b * n_new + j) * Hkv + g) * d + e;
                    size_t dst = (((size_t)b * n_cap + ctx_len[b] + j) * Hkv + g) * d + e;
                    K[dst] = Knew[src];
                    V[dst] = Vnew[src];
                }
    return 0;
}

int oracle_kv_commit(int B, int n_new, const int32_t *n_accept, int32_t *ctx_len)
{
    if (B < 0 || n_new <= 0 || !n_accept || !ctx_len)
        return -1;
    for (int b = 0; b < B; ++b)
        if (n_accept[b] < 0 || n_accept[b] > n_new - 1 || ctx_len[b] < 0)
            return -1;
    for (int b = 0; b < B; ++b)
        ctx_len[b] += 1 + n_accept[b];
    return 0;
}
