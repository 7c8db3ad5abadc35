// SRH importance scoring (English Dustin summary, "Methodology" 1 and 2: attention scores
// of the target-historical and draft-lookahead queries, computed on the semantic
// retrieval heads only, summed into one importance value per context token; German
// Vegas summary 2A/2B for the logit-sum mode over the first and bonus queries).
//
// Softmax mode (PROB_SUM), two kernels:
//   srh_prob_logits  one workgroup per (256-token tile, group, sequence).  The tile's key
//                    rows are read with coalesced 16-byte loads into LDS; each thread then
//                    owns one token and forms its logits for the group's (query head,
//                    query) pairs with fp64 FMAs (bf16 x bf16 products are exact in fp64,
//                    so the only rounding left is fp64 accumulation).  Logits are stored
//                    as fp32 offsets from the tile's per-pair maximum, so tokens near the
//                    maximum — the ones that carry probability mass — keep full relative
//                    precision even when logits are large; the tile leaves (max, sum of
//                    exp2) per pair.
//   srh_finalize     one workgroup per (1024 tokens, sequence): per pair (one wave per
//                    pair, lanes over tiles) the global max and 1/Z from the tile
//                    partials, then per token the sum over pairs of
//                    exp2(offset + tile max - max) / Z.
// Logit-sum mode (LOGIT_SUM2): srh_logit_sum computes the raw scaled logits on MFMA (bf16
// in, fp32 accumulate; the sum's tolerance scales with the sum of |logits|), and the
// finalize kernel sums them per token.
// Every pass streams: the K stream is read once, the logit workspace written once and
// read once.
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kThreads = 256;
constexpr int kProbTilesPerWg = 4;         // tiles each softmax-mode workgroup streams

__device__ __forceinline__ double wave_max_f64(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmax(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

template <int D, int PC>
__global__ __launch_bounds__(kThreads) void srh_prob_logits_kernel(ScoreArgs a)
{
    constexpr int RB = D * 2;          // bytes per key row
    constexpr int RSTR = RB + 16;      // LDS row stride (conflict-free 16-byte row reads)
    constexpr int CPR = RB / 16;       // 16-byte chunks per row
    constexpr int LPT = kProbTile * CPR / kThreads;   // 16-byte loads per thread per tile
    __shared__ __align__(16) uint8_t sK[kProbTile * RSTR];
    __shared__ __align__(16) double sQ[PC][D];
    __shared__ double sMx[4][PC];
    __shared__ float sSm[4][PC];

    const ScoreGroup &G = a.grp[blockIdx.y];
    const int b = blockIdx.z;
    const int N = clampi(a.ctx_len[b], 0, a.ctx_clamp);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n_live = (N + kProbTile - 1) / kProbTile;     // tiles holding context tokens

    // tiles past the context: empty partials
    for (int tile = n_live + blockIdx.x; tile < a.n_tiles; tile += gridDim.x)
        for (int p = tid; p < G.n_pairs; p += kThreads) {
            const int64_t st = ((int64_t)b * a.total_pairs + G.pair0 + p) * a.n_tiles + tile;
            a.tile_max[st] = -INFINITY;
            a.tile_sum[st] = 0.f;
        }
    if ((int)blockIdx.x >= n_live)
        return;

    // the group's queries (fp64) stay in LDS for every tile of this workgroup
    for (int e = tid; e < PC * D; e += kThreads) {
        const int p = e / D;
        const int dd = e - p * D;
        double qv = 0.0;
        if (p < G.n_pairs) {
            const int hl = p / a.n_q;
            const int j = p - hl * a.n_q;
            const uint16_t h = a.q[((int64_t)(b * a.total_qheads + G.q_head0 + hl) * a.n_q + j) * D + dd];
            qv = (double)__uint_as_float((uint32_t)h << 16);
        }
        sQ[p][dd] = qv;
    }

    // tile rows: thread tid loads chunks tid + i*256 (row = chunk / CPR), all issued at once
    u32x4 kr[LPT];
    auto issue = [&](int tile) {
        const int t0 = tile * kProbTile;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = tid + i * kThreads;
            const int r = c / CPR;
            const int t = t0 + r;
            kr[i] = t < N ? load16(G.k.base + kv_offset(G.k, b, t, G.kv_head) + (c - r * CPR) * 8)
                          : u32x4{0, 0, 0, 0};
        }
    };
    int tile = blockIdx.x;
    issue(tile);
    for (; tile < n_live; tile += gridDim.x) {
        __syncthreads();                  // previous tile's rows consumed
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = tid + i * kThreads;
            const int r = c / CPR;
            *reinterpret_cast<u32x4 *>(&sK[r * RSTR + (c - r * CPR) * 16]) = kr[i];
        }
        if (tile + (int)gridDim.x < n_live)
            issue(tile + gridDim.x);      // next tile in flight during this tile's math
        __syncthreads();

        const int tok = tile * kProbTile + tid;
        const bool valid = tok < N;
        const uint8_t *row = &sK[tid * RSTR];
        double acc[PC];
#pragma unroll
        for (int p = 0; p < PC; ++p)
            acc[p] = 0.0;
#pragma unroll 2
        for (int dd = 0; dd < D; dd += 8) {
            const u32x4 kw = *reinterpret_cast<const u32x4 *>(row + dd * 2);
            double kv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kv[2 * j] = (double)bf16_lo(kw[j]);
                kv[2 * j + 1] = (double)bf16_hi(kw[j]);
            }
#pragma unroll
            for (int p = 0; p < PC; ++p)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[p] = fma(kv[j], sQ[p][dd + j], acc[p]);
        }

        // ---- per-pair tile maximum (fp64), offsets from it, sum of exp2 ----
        double l[PC];
#pragma unroll
        for (int p = 0; p < PC; ++p) {
            l[p] = valid ? acc[p] * a.mul : -INFINITY;
            const double m = wave_max_f64(l[p]);
            if (lane == 0)
                sMx[w][p] = m;
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PC; ++p) {
            const double m = fmax(fmax(sMx[0][p], sMx[1][p]), fmax(sMx[2][p], sMx[3][p]));
            const float off = valid ? (float)(l[p] - m) : -INFINITY;
            const float s = wave_sum_f32(valid ? fast_exp2(off) : 0.f);
            if (lane == 0)
                sSm[w][p] = s;
            if (valid && p < G.n_pairs)
                a.logits[((int64_t)b * a.total_pairs + G.pair0 + p) * a.n_pad + tok] = off;
        }
        __syncthreads();
        if (tid < G.n_pairs && tid < PC) {
            const int p = tid;
            const double m = fmax(fmax(sMx[0][p], sMx[1][p]), fmax(sMx[2][p], sMx[3][p]));
            const int64_t st = ((int64_t)b * a.total_pairs + G.pair0 + p) * a.n_tiles + tile;
            a.tile_max[st] = m;
            a.tile_sum[st] = (sSm[0][p] + sSm[1][p]) + (sSm[2][p] + sSm[3][p]);
        }
    }
}

// ---- logit-sum mode: raw scaled logits on MFMA -------------------------------------
constexpr int kSumTile = 512;              // tokens per workgroup
constexpr int kPerWave = kSumTile / 4;
constexpr int kSub = kPerWave / 16;
constexpr int kBatch = 4;

template <int D, int PT>
__global__ __launch_bounds__(kThreads) void srh_logit_sum_kernel(ScoreArgs a)
{
    constexpr int KS = D / 32;
    const int tile = blockIdx.x;
    const ScoreGroup &G = a.grp[blockIdx.y];
    const int b = blockIdx.z;
    const int N = clampi(a.ctx_len[b], 0, a.ctx_clamp);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane >> 4;
    const int li = lane & 15;
    const int t0 = tile * kSumTile;
    if (t0 >= N)
        return;
    const int nqe = min(2, a.n_q);
    const float mul = (float)a.mul;

    // SRH queries as the MFMA B operand: lane holds pair pt*16 + li, its quarter of d
    u32x4 qop[PT][KS];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const int p = pt * 16 + li;
        if (p < G.n_pairs) {
            const int hl = p / nqe;
            const int j = (p - hl * nqe) == 0 ? 0 : a.n_q - 1;
            const uint16_t *qp =
                a.q + ((int64_t)(b * a.total_qheads + G.q_head0 + hl) * a.n_q + j) * D + quad * (D / 4);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qop[pt][ks] = load16(qp + ks * 8);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qop[pt][ks] = u32x4{0, 0, 0, 0};
        }
    }
    const int wbase = t0 + w * kPerWave;
    for (int bt = 0; bt < kSub; bt += kBatch) {
        u32x4 kop[kBatch][KS];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int t = wbase + (bt + u) * 16 + li;      // A operand row = token
            if (t < N) {
                const uint16_t *kp = G.k.base + kv_offset(G.k, b, t, G.kv_head) + quad * (D / 4);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kop[u][ks] = load16(kp + ks * 8);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kop[u][ks] = u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int tb = wbase + (bt + u) * 16 + 4 * quad;   // lane's 4 tokens
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                f32x4 c{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    c = mfma_bf16(kop[u][ks], qop[pt][ks], c);
                c *= mul;
                const int p = pt * 16 + li;
                if (p < G.n_pairs && tb < N) {
                    float *dst = a.logits + ((int64_t)b * a.total_pairs + G.pair0 + p) * a.n_pad + tb;
                    if (tb + 3 < N) {
                        *reinterpret_cast<f32x4 *>(dst) = c;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (tb + r < N)
                                dst[r] = c[r];
                    }
                }
            }
        }
    }
}

constexpr int kFinTokens = 1024;
constexpr int kFinTiles = kFinTokens / kProbTile;

__global__ __launch_bounds__(kThreads) void srh_finalize_kernel(ScoreArgs a)
{
    __shared__ float sOff[kMaxGroups * kMaxPairsPerGroup][kFinTiles];
    __shared__ float sInvZ[kMaxGroups * kMaxPairsPerGroup];
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int N = clampi(a.ctx_len[b], 0, a.ctx_clamp);
    const bool prob = a.mode == DUSTIN_SCORE_PROB_SUM;
    const int tile0 = blockIdx.x * kFinTiles;
    if (prob) {
        // one wave per pair: lanes take the tiles; the max (fp64) and the normaliser (fp32
        // exp2 of the fp64 difference, summed in fp64) are reduced across the wave
        const int w = tid >> 6, lane = tid & 63;
        for (int p = w; p < a.total_pairs; p += kThreads / 64) {
            const double *mx = a.tile_max + ((int64_t)b * a.total_pairs + p) * a.n_tiles;
            const float *sm = a.tile_sum + ((int64_t)b * a.total_pairs + p) * a.n_tiles;
            double M = -INFINITY;
            for (int t = lane; t < a.n_tiles; t += 64)
                M = fmax(M, mx[t]);
            M = wave_max_f64(M);
            double Z = 0.0;
            for (int t = lane; t < a.n_tiles; t += 64)
                if (sm[t] > 0.f)
                    Z += (double)sm[t] * (double)fast_exp2((float)(mx[t] - M));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                Z += __shfl_xor(Z, o);
            if (lane == 0)
                sInvZ[p] = Z > 0.0 ? (float)(1.0 / Z) : 0.f;
            if (lane < kFinTiles) {
                const int t = tile0 + lane;
                sOff[p][lane] = t < a.n_tiles && mx[t] > -INFINITY ? (float)(mx[t] - M) : 0.f;
            }
        }
        __syncthreads();
    }
    const int tb = blockIdx.x * kFinTokens + tid * 4;
    if (tb >= a.n_max)
        return;
    const int tl = (tid * 4) / kProbTile;   // tile of these 4 tokens within the block
    f32x4 v{0.f, 0.f, 0.f, 0.f};
    if (tb < N) {
        const float *lg = a.logits + (int64_t)b * a.total_pairs * a.n_pad + tb;
        for (int p = 0; p < a.total_pairs; ++p) {
            const f32x4 l = *reinterpret_cast<const f32x4 *>(lg + (int64_t)p * a.n_pad);
            if (prob) {
                const float c = sOff[p][tl], iz = sInvZ[p];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] += fast_exp2(l[r] + c) * iz;
            } else {
                v += l;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tb + r >= N)
                v[r] = 0.f;
    }
    float *dst = a.score + (int64_t)b * a.n_max + tb;
    if ((a.n_max & 3) == 0) {
        *reinterpret_cast<f32x4 *>(dst) = v;
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tb + r < a.n_max)
                dst[r] = v[r];
    }
}

template <int D>
hipError_t launch_logit_sum(const ScoreArgs &a, int pt, dim3 grid, hipStream_t st)
{
    switch (pt) {
    case 1: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 3>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 4>), grid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

// the softmax-mode kernel, instantiated for the pair counts of one group
template <int D>
hipError_t launch_prob(const ScoreArgs &a, int max_pairs, dim3 grid, hipStream_t st)
{
    if (max_pairs <= 4)
        hipLaunchKernelGGL((srh_prob_logits_kernel<D, 4>), grid, dim3(kThreads), 0, st, a);
    else if (max_pairs <= 5)
        hipLaunchKernelGGL((srh_prob_logits_kernel<D, 5>), grid, dim3(kThreads), 0, st, a);
    else if (max_pairs <= 8)
        hipLaunchKernelGGL((srh_prob_logits_kernel<D, 8>), grid, dim3(kThreads), 0, st, a);
    else if (max_pairs <= 16)
        hipLaunchKernelGGL((srh_prob_logits_kernel<D, 16>), grid, dim3(kThreads), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const ScoreArgs &a, int head_dim, int max_pairs, hipStream_t st)
{
    hipError_t e = hipSuccess;
    if (a.mode == DUSTIN_SCORE_PROB_SUM) {
        const dim3 g1((unsigned)((a.n_tiles + kProbTilesPerWg - 1) / kProbTilesPerWg), (unsigned)a.n_groups,
                      (unsigned)a.B);
        if (head_dim == 64)
            e = launch_prob<64>(a, max_pairs, g1, st);
        else
            e = launch_prob<128>(a, max_pairs, g1, st);
        if (e != hipSuccess)
            return e;
    } else {
        const dim3 g1((unsigned)((a.n_max + kSumTile - 1) / kSumTile), (unsigned)a.n_groups, (unsigned)a.B);
        const int pt = (max_pairs + 15) / 16;
        e = head_dim == 64 ? launch_logit_sum<64>(a, pt, g1, st) : launch_logit_sum<128>(a, pt, g1, st);
        if (e != hipSuccess)
            return e;
    }
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const dim3 g2((unsigned)((a.n_max + kFinTokens - 1) / kFinTokens), (unsigned)a.B);
    hipLaunchKernelGGL(srh_finalize_kernel, g2, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dustin
