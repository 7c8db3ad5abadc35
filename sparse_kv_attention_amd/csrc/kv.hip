// The verified block in the cache, and attention recovery.
//
// English Dustin summary, Verification Workflow step 5 (what happens to the cache once
// the target has decided which drafts it keeps).  The block being verified is stored behind
// the committed context (where the verification attention reads the new tokens); the
// commit advances each sequence's length over the rows that are kept, and the rows
// behind the new length are simply overwritten by the next block.  Both are pure data
// movement: the write is one 16-byte chunk per thread, read from a contiguous staging
// block (coalesced) and stored through the cache view (a row's chunks are contiguous in
// every layout, so the stores of a row are one 128- or 256-byte run).
//
// Attention recovery ("Methodology" 2 of the same summary names an attention recovery
// rate as the objective of the offline SRH search): the share of the full-cache
// attention probability on the kept set.  The two attention calls' LSEs are the natural
// logs of their softmax normalisers over the kept set and over the whole context, so the
// share is exp(LSE_sparse - LSE_dense), with no per-token pass over the probabilities.
#include "kv.hpp"

namespace dustin {

namespace {

constexpr int kThreads = 256;

// Thread i moves chunk c of row (b, j, g) of K (first half of the grid) or V.
template <int D>
__global__ __launch_bounds__(kThreads) void kv_write_block_kernel(KvWriteArgs a)
{
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    const int64_t per = (int64_t)a.B * a.n_new * a.Hkv * CPR;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= 2 * per)
        return;
    const bool is_v = i >= per;
    int64_t r = is_v ? i - per : i;
    const int c = (int)(r % CPR);
    r /= CPR;
    const int g = (int)(r % a.Hkv);
    r /= a.Hkv;
    const int j = (int)(r % a.n_new);
    const int b = (int)(r / a.n_new);
    const uint16_t *src = (is_v ? a.v_new : a.k_new) + (((int64_t)b * a.n_new + j) * a.Hkv + g) * D + c * 8;
    const int N = clampi(a.ctx_len[b], 0, a.ctx_clamp);
    const KvView &view = is_v ? a.v : a.k;
    uint16_t *dst = const_cast<uint16_t *>(view.base) + kv_offset(view, b, N + j, g) + c * 8;
    *reinterpret_cast<u32x4 *>(dst) = load16(src);
}

// ctx_len[b] <- clamp(ctx_len[b], 0, 2^30) + 1 + clamp(n_accept[b], 0, n_new - 1)
__global__ __launch_bounds__(kThreads) void kv_commit_kernel(int B, int n_new, const int32_t *n_accept,
                                                             int32_t *ctx_len)
{
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= B)
        return;
    ctx_len[b] = clampi(ctx_len[b], 0, 1 << 30) + 1 + clampi(n_accept[b], 0, n_new - 1);
}

__global__ __launch_bounds__(kThreads) void attn_recovery_kernel(int n, const float *lse_sparse,
                                                                 const float *lse_dense, float *rec)
{
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n)
        return;
    rec[i] = expf(lse_sparse[i] - lse_dense[i]);
}

}  // namespace

hipError_t launch_kv_write_block(const KvWriteArgs &a, int head_dim, hipStream_t st)
{
    const int64_t threads = 2ll * a.B * a.n_new * a.Hkv * (head_dim / 8);
    if (threads == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    if (head_dim == 64)
        hipLaunchKernelGGL((kv_write_block_kernel<64>), grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((kv_write_block_kernel<128>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_kv_commit(int B, int n_new, const int32_t *n_accept, int32_t *ctx_len, hipStream_t st)
{
    hipLaunchKernelGGL(kv_commit_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0, st, B, n_new,
                       n_accept, ctx_len);
    return hipGetLastError();
}

hipError_t launch_attn_recovery(int n, const float *lse_sparse, const float *lse_dense, float *rec,
                                hipStream_t st)
{
    hipLaunchKernelGGL(attn_recovery_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st, n,
                       lse_sparse, lse_dense, rec);
    return hipGetLastError();
}

}  // namespace dustin
