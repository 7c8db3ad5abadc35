// Verification attention over a gathered token list (sparse) or the whole context (dense).
//
// Computes, for every sequence b, verify query t and query head h (KV head g = h / G):
//   out = softmax(scale * q . K[x]) V[x] over x in I_b u {ctx_len[b] + j : j <= t}
// (English Dustin summary, Verification Workflow steps 3-4: the draft block is verified
// against the selected tokens only; the selected rows are gathered by position, never
// copied into a compacted cache, because the method keeps the full history resident —
// "Significance and Limitations" 2).
//
// Work decomposition (gfx950, 64-wide waves, 4 waves per workgroup):
//   workgroup = (b, g, query group, split of the token list); the split's tokens are
//   processed in chunks of 64 list positions.  Per chunk:
//     1. all 256 threads gather the chunk's 64 K rows and 64 V rows (16-byte loads,
//        4 threads per row) into a double-buffered LDS stage; the next chunk's loads
//        are issued before the current chunk is computed;
//     2. wave w computes S^T = K Q^T for chunk tokens 16w..16w+15 against all (up to
//        QT*16) queries of the KV head's group on MFMA (bf16 in, fp32 accumulate);
//     3. a workgroup-wide online softmax (chunk max exchanged through LDS) gives
//        P = exp(S - m) for every query; P^T is staged in LDS as bf16;
//     4. wave w accumulates O^T[dv][q] += V^T P^T for its quarter of the head dim over
//        all 64 chunk tokens on MFMA.
//   Splits of one (b, g, query group) are merged by the last workgroup to finish
//   (per-pair counter), with the usual log-sum-exp weights, in fixed split order.
//   Block ids are mapped so that all splits of one pair run on one XCD (blocks are
//   dispatched round-robin over the 8 XCDs), keeping the partials in that XCD's L2.
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kChunk = 64;
constexpr int kThreads = 256;

template <int D, int QT>
struct AttnShape {
    static constexpr int KS = D / 32;          // MFMA k-steps over the head dim
    static constexpr int ROWB = D * 2;         // bytes per K/V row
    static constexpr int PIECE = ROWB / 4;     // bytes of a row owned by one lane group
    static constexpr int LPR = PIECE / 16;     // 16-byte loads per thread per row
    static constexpr int KSTR = ROWB + 16;     // LDS row stride of K (conflict-free QK reads)
    static constexpr int VSTR = ROWB + 8;      // LDS row stride of V (conflict-free PV reads)
    static constexpr int QR = QT * 16;         // padded query rows
    static constexpr int PSTR = kChunk * 2 + 16;
    static constexpr int DVT_W = D / 64;       // 16-wide dv tiles per wave
};

template <int D, int QT>
__global__ __launch_bounds__(kThreads) void verify_attn_kernel(AttnArgs a)
{
    using S = AttnShape<D, QT>;
    __shared__ __align__(16) uint8_t sK[2][kChunk * S::KSTR];
    __shared__ __align__(16) uint8_t sV[2][kChunk * S::VSTR];
    __shared__ __align__(16) uint8_t sP[S::QR * S::PSTR];
    __shared__ float sMax[4][S::QR];
    __shared__ float sSum[4][S::QR];
    __shared__ int sLast;

    // ---- block -> (pair, split); all splits of a pair share blockIdx % 8 ----
    const int x = blockIdx.x;
    const int pair = ((x >> 3) / a.splits) * 8 + (x & 7);
    const int split = (x >> 3) % a.splits;
    if (pair >= a.pairs)
        return;
    const int qg = pair % a.qgroups;
    const int bg = pair / a.qgroups;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane >> 4;   // MFMA lane group
    const int li = lane & 15;

    // ---- sequence geometry; every device value is clamped ----
    const int N = clampi(a.ctx_len[b], 0, a.ctx_clamp);
    const int nsel = a.idx ? clampi(a.count[b], 0, min(a.k_max, N)) : N;
    const int L = nsel + a.nv;
    const int nchunks = (L + kChunk - 1) / kChunk;
    const int c0 = split * a.cps;
    const int c1 = min(c0 + a.cps, nchunks);

    // ---- Q as the B operand of S^T = K Q^T: lane holds q-row (qt*16 + li), its quarter
    //      of the head dim; k-step ks covers elements quad*D/4 + ks*8 .. +8 ----
    u32x4 qop[QT][S::KS];
    int qrow_t[QT];   // verify index t of the lane's query row (large for padding rows)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int row = qg * S::QR + qt * 16 + li;
        if (row < a.GV) {
            const int t = row / a.G;
            const int h = g * a.G + (row - t * a.G);
            const uint16_t *p = a.q + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + quad * (D / 4);
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks)
                qop[qt][ks] = load16(p + ks * 8);
            qrow_t[qt] = t;
        } else {
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks)
                qop[qt][ks] = u32x4{0, 0, 0, 0};
            qrow_t[qt] = 1 << 20;
        }
    }

    f32x4 acc[S::DVT_W][QT];
#pragma unroll
    for (int i = 0; i < S::DVT_W; ++i)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            acc[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun[QT], lrun[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        mrun[qt] = -INFINITY;
        lrun[qt] = 0.f;
    }

    // ---- gather: thread tid owns row slot tid/4, piece tid%4 of K and of V ----
    const int slot = tid >> 2;
    const int piece = tid & 3;
    u32x4 kreg[S::LPR], vreg[S::LPR];
    auto gather = [&](int c) {
        const int pos = c * kChunk + slot;
        int tok = -1;
        if (pos < nsel)
            tok = a.idx ? clampi(a.idx[(int64_t)b * a.k_max + pos], 0, N - 1) : pos;
        else if (pos < L)
            tok = N + (pos - nsel);
        if (tok >= 0) {
            const uint16_t *kp = a.k.base + kv_offset(a.k, b, tok, g) + piece * (S::PIECE / 2);
            const uint16_t *vp = a.v.base + kv_offset(a.v, b, tok, g) + piece * (S::PIECE / 2);
#pragma unroll
            for (int i = 0; i < S::LPR; ++i) {
                kreg[i] = load16(kp + i * 8);
                vreg[i] = load16(vp + i * 8);
            }
        } else {
#pragma unroll
            for (int i = 0; i < S::LPR; ++i) {
                kreg[i] = u32x4{0, 0, 0, 0};
                vreg[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < S::LPR; ++i) {
            *reinterpret_cast<u32x4 *>(&sK[buf][slot * S::KSTR + piece * S::PIECE + i * 16]) = kreg[i];
            // V rows are 8-byte aligned only (stride chosen for conflict-free PV reads)
            u32x2 *vd = reinterpret_cast<u32x2 *>(&sV[buf][slot * S::VSTR + piece * S::PIECE + i * 16]);
            vd[0] = u32x2{vreg[i][0], vreg[i][1]};
            vd[1] = u32x2{vreg[i][2], vreg[i][3]};
        }
    };

    if (c0 < c1) {
        gather(c0);
        stage(0);
    }
    for (int c = c0; c < c1; ++c) {
        const int buf = (c - c0) & 1;
        if (c + 1 < c1)
            gather(c + 1);            // in flight while chunk c is computed
        __syncthreads();              // chunk c staged

        // ---- S^T for tokens 16w .. 16w+15 of the chunk ----
        u32x4 kop[S::KS];
        const uint8_t *krow = &sK[buf][(16 * w + li) * S::KSTR + quad * S::PIECE];
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
            kop[ks] = *reinterpret_cast<const u32x4 *>(krow + ks * 16);
        f32x4 s[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            s[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks)
                s[qt] = mfma_bf16(kop[ks], qop[qt][ks], s[qt]);
        }
        // lane holds tokens 16w + 4*quad + r (r = 0..3) for query row qt*16 + li
        const int pos0 = c * kChunk + 16 * w + 4 * quad;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pos = pos0 + r;
                const bool ok = pos < L && (pos < nsel || pos - nsel <= qrow_t[qt]);
                const float v = ok ? s[qt][r] * a.scale_log2 : -INFINITY;
                s[qt][r] = v;
                mx = fmaxf(mx, v);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (quad == 0)
                sMax[w][qt * 16 + li] = mx;
        }
        __syncthreads();              // chunk maxima exchanged

#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int q = qt * 16 + li;
            const float cm = fmaxf(fmaxf(sMax[0][q], sMax[1][q]), fmaxf(sMax[2][q], sMax[3][q]));
            const float mnew = fmaxf(mrun[qt], cm);
            const float muse = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = fast_exp2(mrun[qt] - muse);
            mrun[qt] = mnew;
            float p[4];
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = fast_exp2(s[qt][r] - muse);
                ps += p[r];
            }
            lrun[qt] = lrun[qt] * alpha + ps;
#pragma unroll
            for (int i = 0; i < S::DVT_W; ++i)
                acc[i][qt] *= alpha;
            u32x2 pk{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
            *reinterpret_cast<u32x2 *>(&sP[q * S::PSTR + (16 * w + 4 * quad) * 2]) = pk;
        }
        __syncthreads();              // P^T staged

        // ---- O^T[dv][q] += V^T P^T over the chunk's 64 tokens, dv quarter of wave w ----
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {
            u32x4 pop[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                pop[qt] = *reinterpret_cast<const u32x4 *>(
                    &sP[(qt * 16 + li) * S::PSTR + (ts * 32 + 8 * quad) * 2]);
#pragma unroll
            for (int i = 0; i < S::DVT_W; ++i) {
                const int dv = (w * S::DVT_W + i) * 16 + li;
                const uint8_t *vcol = &sV[buf][(ts * 32 + 8 * quad) * S::VSTR + dv * 2];
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    e[j] = *reinterpret_cast<const uint16_t *>(vcol + j * S::VSTR);
                const u32x4 vop{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                e[6] | (e[7] << 16)};
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    acc[i][qt] = mfma_bf16(vop, pop[qt], acc[i][qt]);
            }
        }
        if (c + 1 < c1)
            stage(buf ^ 1);           // every wave is past chunk c-1, which used buf^1
    }

    // ---- row sums: over the 4 lane groups, then over the 4 waves ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float l = lrun[qt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (quad == 0)
            sSum[w][qt * 16 + li] = l;
    }
    __syncthreads();
    float ltot[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int q = qt * 16 + li;
        ltot[qt] = (sSum[0][q] + sSum[1][q]) + (sSum[2][q] + sSum[3][q]);
    }

    if (a.splits == 1) {
        // ---- final output straight from registers ----
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int row = qg * S::QR + qt * 16 + li;
            if (row >= a.GV)
                continue;
            const int t = row / a.G;
            const int h = g * a.G + (row - t * a.G);
            const float inv = 1.f / ltot[qt];
            uint16_t *o = a.out + ((int64_t)(b * a.nv + t) * a.Hq + h) * D;
#pragma unroll
            for (int i = 0; i < S::DVT_W; ++i) {
                const int dv = (w * S::DVT_W + i) * 16 + 4 * quad;
                u32x2 pk{pack_bf16x2(acc[i][qt][0] * inv, acc[i][qt][1] * inv),
                         pack_bf16x2(acc[i][qt][2] * inv, acc[i][qt][3] * inv)};
                *reinterpret_cast<u32x2 *>(o + dv) = pk;
            }
            if (w == 0 && quad == 0)
                a.lse[((int64_t)b * a.Hq + h) * a.nv + t] = (mrun[qt] + __log2f(ltot[qt])) * kLn2;
        }
        return;
    }

    // ---- split partial: acc [QR][D], then m [QR], l [QR] ----
    const int64_t pstride = (int64_t)S::QR * D + 2 * S::QR;
    float *part = a.part + ((int64_t)pair * a.splits + split) * pstride;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int q = qt * 16 + li;
#pragma unroll
        for (int i = 0; i < S::DVT_W; ++i) {
            const int dv = (w * S::DVT_W + i) * 16 + 4 * quad;
            *reinterpret_cast<f32x4 *>(part + (int64_t)q * D + dv) = acc[i][qt];
        }
        if (w == 0 && quad == 0) {
            part[S::QR * D + q] = mrun[qt];
            part[S::QR * D + S::QR + q] = ltot[qt];
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0)
        sLast = atomicAdd(&a.counters[pair], 1) == a.splits - 1;
    __syncthreads();
    if (!sLast)
        return;
    __threadfence();

    // ---- last workgroup of the pair: merge the splits in fixed order ----
    const float *base = a.part + (int64_t)pair * a.splits * pstride;
    for (int item = tid; item < S::QR * (D / 4); item += kThreads) {
        const int q = item / (D / 4);
        const int dv = (item % (D / 4)) * 4;
        const int row = qg * S::QR + q;
        if (row >= a.GV)
            continue;
        float M = -INFINITY;
        for (int sp = 0; sp < a.splits; ++sp)
            M = fmaxf(M, base[sp * pstride + S::QR * D + q]);
        f32x4 num{0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
        for (int sp = 0; sp < a.splits; ++sp) {
            const float *ps = base + sp * pstride;
            const float wgt = fast_exp2(ps[S::QR * D + q] - M);
            num += wgt * *reinterpret_cast<const f32x4 *>(ps + (int64_t)q * D + dv);
            den += wgt * ps[S::QR * D + S::QR + q];
        }
        const int t = row / a.G;
        const int h = g * a.G + (row - t * a.G);
        const float inv = 1.f / den;
        uint16_t *o = a.out + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + dv;
        u32x2 pk{pack_bf16x2(num[0] * inv, num[1] * inv), pack_bf16x2(num[2] * inv, num[3] * inv)};
        *reinterpret_cast<u32x2 *>(o) = pk;
        if (dv == 0)
            a.lse[((int64_t)b * a.Hq + h) * a.nv + t] = (M + __log2f(den)) * kLn2;
    }
    if (tid == 0)
        a.counters[pair] = 0;         // ready for the next call
}

template <int D>
hipError_t launch_d(const AttnArgs &a, int qt, dim3 grid, hipStream_t st)
{
    switch (qt) {
    case 1: hipLaunchKernelGGL((verify_attn_kernel<D, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((verify_attn_kernel<D, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((verify_attn_kernel<D, 3>), grid, dim3(kThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((verify_attn_kernel<D, 4>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((verify_attn_kernel<D, 5>), grid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace

AttnPlan plan_attn(int B, int Hkv, int G, int nv, int max_list, int target_wgs)
{
    AttnPlan p;
    const int gv = G * nv;
    const int qt_total = (gv + 15) / 16;
    p.qgroups = (qt_total + kMaxQT - 1) / kMaxQT;
    p.qt = (qt_total + p.qgroups - 1) / p.qgroups;
    p.pairs = B * Hkv * p.qgroups;
    const int max_chunks = max(1, (max_list + kChunk - 1) / kChunk);
    int s = (target_wgs + p.pairs - 1) / max(1, p.pairs);
    s = max(1, min(s, max_chunks));
    p.cps = (max_chunks + s - 1) / s;
    p.splits = (max_chunks + p.cps - 1) / p.cps;
    p.part_floats = p.splits > 1 ? (size_t)p.pairs * p.splits * ((size_t)p.qt * 16 * 128 + 2 * p.qt * 16) : 0;
    p.grid = (size_t)((p.pairs + 7) / 8) * 8 * p.splits;
    return p;
}

hipError_t launch_attn(const AttnArgs &a, int head_dim, int qt, hipStream_t st)
{
    const dim3 grid((unsigned)(((a.pairs + 7) / 8) * 8 * a.splits));
    return head_dim == 64 ? launch_d<64>(a, qt, grid, st) : launch_d<128>(a, qt, grid, st);
}

}  // namespace dustin
