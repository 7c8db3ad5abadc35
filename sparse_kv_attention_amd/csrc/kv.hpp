// Launch interface of the KV block write/commit and attention-recovery kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dustin {

constexpr int kMaxNewRows = 16;   // rows of one verified block

struct KvWriteArgs {
    int B, Hkv, n_new;
    const uint16_t *k_new, *v_new;   // [B][n_new][Hkv][head_dim]
    KvView k, v;                     // written
    const int32_t *ctx_len;
    int ctx_clamp;                   // ctx_len is clamped to [0, ctx_clamp]
};

hipError_t launch_kv_write_block(const KvWriteArgs &a, int head_dim, hipStream_t st);
hipError_t launch_kv_commit(int B, int n_new, const int32_t *n_accept, int32_t *ctx_len, hipStream_t st);
hipError_t launch_attn_recovery(int n, const float *lse_sparse, const float *lse_dense, float *rec,
                                hipStream_t st);

}  // namespace dustin
