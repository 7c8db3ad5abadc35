/*
 * A C program that drives the library through include/dustin.h alone: device memory from
 * the HIP runtime, plain pointers and sizes, no Python.  Results are fixed by hand:
 *
 *   selection  (policy of the English Dustin summary, "Methodology" 1, last two sentences)
 *     sequence 0: 16 tokens, budget 6, 2 sinks, window 2, m = 1.  Kept: sinks {0, 1} and
 *     window {14, 15}; the draft tier takes the best draft score outside them (position
 *     7); the target tier takes the best remaining target score (positions 3 and 9 tie at
 *     0.8; the smaller position wins; 7 is already taken).  I = {0, 1, 3, 7, 14, 15}.
 *     sequence 1: 10 tokens, budget 10: the whole context.  Unused entries are -1.
 *
 *   attention (verification step 4; dense_verify_attn for the full cache)
 *     all keys zero, so every attended row has the same weight: O is the mean of the
 *     attended V rows and LSE = ln(number of attended rows).  V row x holds x + 1 in every
 *     element; 4 context tokens, 2 verify queries, I = {0, 2}.
 *       sparse: query 0 sees {0, 2, 4} -> 3,    ln 3;  query 1 sees {0, 2, 4, 5} -> 3.75, ln 4
 *       dense : query 0 sees {0..4}    -> 3,    ln 5;  query 1 sees {0..5}       -> 3.5,  ln 6
 *
 *   error path: a negative batch is rejected with DUSTIN_ERR_INVALID_ARG before anything
 *   is enqueued, and every status has a message.
 *
 * Prints one line per check; the exit status is 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dustin.h"

static int failures = 0;

#define HIP_OK(call)                                                                    \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess) {                                                         \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            return 2;                                                                   \
        }                                                                               \
    } while (0)

static void check(int ok, const char *what)
{
    printf("%s: %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok)
        ++failures;
}

static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);   /* exact for the small integers used here */
}

static float float_of(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int selection_case(void)
{
    enum { B = 2, N_MAX = 16, K_MAX = 12 };
    const int32_t ctx[B] = {16, 10}, budget[B] = {6, 10}, sink[B] = {2, 1}, window[B] = {2, 1},
                  m[B] = {1, 1};
    float draft[B][N_MAX], target[B][N_MAX];
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N_MAX; ++i) {
            draft[b][i] = 0.1f;
            target[b][i] = 0.2f;
        }
    draft[0][0] = draft[0][15] = 5.f;   /* protected anyway */
    draft[0][7] = 0.9f;
    draft[0][3] = 0.5f;
    target[0][7] = 1.f;
    target[0][9] = 0.8f;
    target[0][3] = 0.8f;

    int32_t *d_i32;
    float *d_f32;
    HIP_OK(hipMalloc((void **)&d_i32, sizeof(int32_t) * (5 * B + B * K_MAX + B)));
    HIP_OK(hipMalloc((void **)&d_f32, sizeof(float) * 2 * B * N_MAX));
    int32_t *d_ctx = d_i32, *d_budget = d_i32 + B, *d_sink = d_i32 + 2 * B, *d_window = d_i32 + 3 * B,
            *d_m = d_i32 + 4 * B, *d_idx = d_i32 + 5 * B, *d_count = d_idx + B * K_MAX;
    float *d_draft = d_f32, *d_target = d_f32 + B * N_MAX;
    HIP_OK(hipMemcpy(d_ctx, ctx, sizeof ctx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_budget, budget, sizeof budget, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sink, sink, sizeof sink, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_window, window, sizeof window, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_m, m, sizeof m, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_draft, draft, sizeof draft, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_target, target, sizeof target, hipMemcpyHostToDevice));

    size_t ws_bytes = 0;
    check(dustin_select_workspace_size(B, N_MAX, &ws_bytes) == DUSTIN_OK, "selection workspace query");
    void *ws = NULL;
    if (ws_bytes)
        HIP_OK(hipMalloc(&ws, ws_bytes));
    const dustin_status st = dustin_select(B, N_MAX, d_ctx, d_draft, d_target, d_budget, d_sink, d_window,
                                           d_m, K_MAX, d_idx, d_count, ws, ws_bytes, NULL);
    check(st == DUSTIN_OK, "dustin_select returns DUSTIN_OK");
    HIP_OK(hipDeviceSynchronize());
    int32_t idx[B][K_MAX], count[B];
    HIP_OK(hipMemcpy(idx, d_idx, sizeof idx, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(count, d_count, sizeof count, hipMemcpyDeviceToHost));

    const int32_t want0[K_MAX] = {0, 1, 3, 7, 14, 15, -1, -1, -1, -1, -1, -1};
    const int32_t want1[K_MAX] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, -1, -1};
    check(count[0] == 6 && memcmp(idx[0], want0, sizeof want0) == 0,
          "sequence 0: sinks, window, one draft pick, the tie to the smaller position");
    check(count[1] == 10 && memcmp(idx[1], want1, sizeof want1) == 0,
          "sequence 1: budget = context keeps every token");

    check(dustin_select(-1, N_MAX, d_ctx, d_draft, d_target, d_budget, d_sink, d_window, d_m, K_MAX, d_idx,
                        d_count, ws, ws_bytes, NULL) == DUSTIN_ERR_INVALID_ARG,
          "a negative batch is rejected");
    const char *msg = dustin_status_string(DUSTIN_ERR_INVALID_ARG);
    check(msg != NULL && msg[0] != '\0', "every status has a message");
    if (ws)
        HIP_OK(hipFree(ws));
    HIP_OK(hipFree(d_i32));
    HIP_OK(hipFree(d_f32));
    return 0;
}

static int attention_case(void)
{
    enum { B = 1, HQ = 2, HKV = 1, D = 64, NV = 2, CTX = 4, CAP = CTX + NV, K_MAX = 2 };
    static uint16_t k[B][CAP][HKV][D], v[B][CAP][HKV][D], q[B][NV][HQ][D], out[B][NV][HQ][D];
    memset(k, 0, sizeof k);
    for (int x = 0; x < CAP; ++x)
        for (int e = 0; e < D; ++e)
            v[0][x][0][e] = bf16_of((float)(x + 1));
    for (int t = 0; t < NV; ++t)
        for (int h = 0; h < HQ; ++h)
            for (int e = 0; e < D; ++e)
                q[0][t][h][e] = bf16_of((float)((e % 5) - 2));   /* any values: K is zero */
    const int32_t ctx[B] = {CTX}, idx[B][K_MAX] = {{0, 2}}, count[B] = {2};

    uint16_t *d_k, *d_v, *d_q, *d_out;
    int32_t *d_i32;
    float *d_lse;
    HIP_OK(hipMalloc((void **)&d_k, sizeof k));
    HIP_OK(hipMalloc((void **)&d_v, sizeof v));
    HIP_OK(hipMalloc((void **)&d_q, sizeof q));
    HIP_OK(hipMalloc((void **)&d_out, sizeof out));
    HIP_OK(hipMalloc((void **)&d_i32, sizeof(int32_t) * (B + B * K_MAX + B)));
    HIP_OK(hipMalloc((void **)&d_lse, sizeof(float) * B * HQ * NV));
    int32_t *d_ctx = d_i32, *d_idx = d_i32 + B, *d_count = d_i32 + B + B * K_MAX;
    HIP_OK(hipMemcpy(d_k, k, sizeof k, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, v, sizeof v, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_q, q, sizeof q, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_ctx, ctx, sizeof ctx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_count, count, sizeof count, hipMemcpyHostToDevice));

    dustin_kv_view kv, vv;
    memset(&kv, 0, sizeof kv);
    kv.stride_batch = (int64_t)CAP * HKV * D;
    kv.stride_token = (int64_t)HKV * D;
    kv.stride_head = D;
    kv.n_tokens = CAP;
    kv.n_heads = HKV;
    vv = kv;
    kv.base = d_k;
    vv.base = d_v;

    size_t ws_sparse = 0, ws_dense = 0;
    check(dustin_sparse_verify_attn_workspace_size(B, HQ, HKV, D, NV, K_MAX, &ws_sparse) == DUSTIN_OK &&
              dense_verify_attn_workspace_size(B, HQ, HKV, D, NV, CTX, &ws_dense) == DUSTIN_OK,
          "attention workspace queries");
    const size_t ws_bytes = ws_sparse > ws_dense ? ws_sparse : ws_dense;
    void *ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 16));

    const float scale = 0.125f;
    float lse[B][HQ][NV];
    for (int dense = 0; dense < 2; ++dense) {
        const dustin_status st =
            dense ? dense_verify_attn(B, HQ, HKV, D, NV, d_q, &kv, &vv, d_ctx, CTX, scale, d_out, d_lse, ws,
                                      ws_bytes, NULL)
                  : dustin_sparse_verify_attn(B, HQ, HKV, D, NV, d_q, &kv, &vv, d_ctx, d_idx, d_count, K_MAX,
                                              scale, d_out, d_lse, ws, ws_bytes, NULL);
        check(st == DUSTIN_OK, dense ? "dense_verify_attn returns DUSTIN_OK"
                                     : "dustin_sparse_verify_attn returns DUSTIN_OK");
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(lse, d_lse, sizeof lse, hipMemcpyDeviceToHost));
        const double want_o[2][NV] = {{3.0, 3.75}, {3.0, 3.5}};
        const double want_n[2][NV] = {{3.0, 4.0}, {5.0, 6.0}};
        double err_o = 0.0, err_l = 0.0;
        for (int t = 0; t < NV; ++t)
            for (int h = 0; h < HQ; ++h) {
                for (int e = 0; e < D; ++e)
                    err_o = fmax(err_o, fabs((double)float_of(out[0][t][h][e]) - want_o[dense][t]));
                err_l = fmax(err_l, fabs((double)lse[0][h][t] - log(want_n[dense][t])));
            }
        printf("      %s: max|O - mean V| = %.3g, max|LSE - ln n| = %.3g\n", dense ? "dense" : "sparse",
               err_o, err_l);
        check(err_o <= 2e-2 && err_l <= 1e-3,
              dense ? "dense attention: mean of V over the whole cache"
                    : "sparse attention: mean of V over the selected and causal new rows");
    }
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(d_k));
    HIP_OK(hipFree(d_v));
    HIP_OK(hipFree(d_q));
    HIP_OK(hipFree(d_out));
    HIP_OK(hipFree(d_i32));
    HIP_OK(hipFree(d_lse));
    return 0;
}

int main(void)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        printf("no GPU\n");
        return 3;
    }
    if (selection_case() || attention_case())
        return 2;
    if (failures) {
        printf("c abi example: %d check(s) failed\n", failures);
        return 1;
    }
    printf("c abi example ok\n");
    return 0;
}
