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
//   workgroup = (b, g, query group, split of the token list).  The split's list
//   positions (at most 1024) are resolved once into an LDS table of tokens (and pages),
//   then each wave streams its own 16-token tiles (tiles w, w+4, ...) with no workgroup
//   barrier inside the loop:
//     - K rows are loaded straight into the MFMA A-operand layout (lane = row, four
//       16-byte loads per lane) and S^T = K Q^T is formed for all (up to QT*16) queries
//       of the KV head's group on v_mfma_f32_16x16x32_bf16 (fp32 accumulate);
//     - the wave's online softmax keeps P in registers: the S^T output layout of a lane
//       (4 tokens x 1 query) is exactly the B operand of v_mfma_f32_16x16x16_bf16;
//     - V rows are transposed through a wave-private LDS tile and O^T += V^T P^T is
//       accumulated over the whole head dim;
//     - the next tile's K and V loads are in flight while the current one is computed.
//   The four waves merge their (max, sum, O) in LDS at the end; splits of one pair are
//   merged by a second kernel with log-sum-exp weights in fixed split order (a kernel
//   boundary, not per-workgroup device-scope fences, which write back and invalidate
//   the XCD's L2).  Block ids are mapped so that all splits of one pair run on one XCD
//   (blocks are dispatched round-robin over the 8 XCDs).
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kThreads = 256;
constexpr float kLazy = 8.f;       // rescale O only when a tile's max exceeds the reference by 2^8

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma_bf16_k16(u32x2 a, u32x2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                      __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int D, int QT, int R>
struct AttnShape {
    static constexpr int KS = D / 32;          // 16x16x32 k-steps of QK = 16-byte loads per row quarter
    static constexpr int QD = D / 4;           // head-dim quarter held by one MFMA lane group
    static constexpr int DVT = D / 16;         // 16-wide head-dim tiles of PV
    static constexpr int QR = QT * 16;         // padded query rows
    static constexpr int SLOT = 2 * KS * 1024; // one ring slot: KS KB of K rows, then KS KB of V rows
    static constexpr int ACC = DVT * QT * 4;   // O accumulator floats per lane
    static constexpr int TAB = kSplitMax * 4 * 3;
    static constexpr int RING = 4 * R * SLOT;
    static constexpr int MRG = 64 * ACC * 4 + 2 * QR * 4;
    static constexpr int LDS = TAB + (RING > MRG ? RING : MRG);
};

template <int D, int QT, int R>
__global__ __launch_bounds__(kThreads) void verify_attn_split_kernel(AttnArgs a)
{
    using S = AttnShape<D, QT, R>;
    __shared__ __align__(16) uint8_t lds[S::LDS];
    int *sTok = reinterpret_cast<int *>(lds);
    int *sPgK = sTok + kSplitMax;
    int *sPgV = sPgK + kSplitMax;

    // ---- block -> (pair, split); all splits of a pair share blockIdx % 8 (one XCD) ----
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
    const int p0 = split * a.spl;
    const int p1 = min(p0 + a.spl, L);
    const int cnt = max(p1 - p0, 0);
    const int full_end = min(p1, nsel);   // positions below this need no mask

    // ---- the split's tokens (and pages) into LDS: index loads first, then pages ----
    {
        int raw[kSplitMax / kThreads];
#pragma unroll
        for (int k = 0; k < kSplitMax / kThreads; ++k) {
            const int i = tid + k * kThreads;
            const int pos = p0 + i;
            raw[k] = (i < cnt && a.idx && pos < nsel) ? a.idx[(int64_t)b * a.k_max + pos] : 0;
        }
#pragma unroll
        for (int k = 0; k < kSplitMax / kThreads; ++k) {
            const int i = tid + k * kThreads;
            if (i >= cnt)
                continue;
            const int pos = p0 + i;
            const int tok = pos < nsel ? (a.idx ? clampi(raw[k], 0, N - 1) : pos) : N + (pos - nsel);
            sTok[i] = tok;
            if (a.k.pt)
                sPgK[i] = clampi(a.k.pt[(int64_t)b * a.k.max_pages + (tok >> a.k.ps_log2)], 0, a.k.num_pages - 1);
            if (a.v.pt)
                sPgV[i] = clampi(a.v.pt[(int64_t)b * a.v.max_pages + (tok >> a.v.ps_log2)], 0, a.v.num_pages - 1);
        }
    }

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
            const uint16_t *p = a.q + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + quad * S::QD;
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
    __syncthreads();                  // token table ready

    f32x4 acc[S::DVT][QT];
#pragma unroll
    for (int i = 0; i < S::DVT; ++i)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            acc[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref[QT], lrun[QT];         // reference max (log2 units) and running sum per query
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        mref[qt] = -INFINITY;
        lrun[qt] = 0.f;
    }

    const int ntile = (cnt + 15) >> 4;
    const int mine = ntile > w ? (ntile - w + 3) >> 2 : 0;    // tiles w, w+4, ... of this wave
    uint8_t *wring = lds + S::TAB + w * R * S::SLOT;           // this wave's ring of tile slots

    // Tile jj of this wave into ring slot jj % R by LDS DMA: lane (quad, li) moves the
    // quarter `quad` of row li of K and of V, 16 bytes per instruction (lane i's bytes
    // land at slot + 16*i).  Issued for every step, also past the end (then it re-reads
    // the split's last row into a slot nobody reads), so the waits count exactly.
    auto dma = [&](int jj) {
        const int rel = min(((w + 4 * jj) << 4) + li, cnt - 1);
        const int tok = sTok[rel];
        int64_t ko, vo;
        if (a.k.pt)
            ko = (int64_t)sPgK[rel] * a.k.sp + (int64_t)(tok & ((1 << a.k.ps_log2) - 1)) * a.k.st;
        else
            ko = (int64_t)b * a.k.sb + (int64_t)tok * a.k.st;
        if (a.v.pt)
            vo = (int64_t)sPgV[rel] * a.v.sp + (int64_t)(tok & ((1 << a.v.ps_log2) - 1)) * a.v.st;
        else
            vo = (int64_t)b * a.v.sb + (int64_t)tok * a.v.st;
        const uint16_t *kp = a.k.base + ko + (int64_t)g * a.k.sh + quad * S::QD;
        const uint16_t *vp = a.v.base + vo + (int64_t)g * a.v.sh + quad * S::QD;
        uint8_t *slot = wring + (jj % R) * S::SLOT;
#pragma unroll
        for (int i = 0; i < S::KS; ++i)
            __builtin_amdgcn_global_load_lds(kp + i * 8, (lds_void *)(slot + i * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < S::KS; ++i)
            __builtin_amdgcn_global_load_lds(vp + i * 8, (lds_void *)(slot + (S::KS + i) * 1024), 16, 0, 0);
    };

    if (mine > 0) {
#pragma unroll
        for (int jj = 0; jj < R - 1; ++jj)
            dma(jj);
        for (int jj = 0; jj < mine; ++jj) {
            dma(jj + R - 1);
            wait_vmcnt<2 * S::KS * (R - 1)>();      // tile jj has landed; R-1 tiles stay in flight
            __builtin_amdgcn_sched_barrier(0);
            const uint8_t *slot = wring + (jj % R) * S::SLOT;
            const int pos0 = p0 + ((w + 4 * jj) << 4);

            // S^T = K Q^T: the lane's own K bytes are its A operand
            u32x4 kop[S::KS];
#pragma unroll
            for (int i = 0; i < S::KS; ++i)
                kop[i] = *reinterpret_cast<const u32x4 *>(slot + i * 1024 + lane * 16);
            f32x4 s[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                s[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < S::KS; ++ks)
                    s[qt] = mfma_bf16(kop[ks], qop[qt][ks], s[qt]);
            }
            // lane holds tokens pos0 + 4*quad + r (r = 0..3) for query row qt*16 + li
            const bool full = pos0 + 16 <= full_end;
            u32x2 pb[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                if (full) {
                    s[qt] *= a.scale_log2;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int pos = pos0 + 4 * quad + r;
                        const bool ok = (pos < p1) & ((pos < nsel) | (pos - nsel <= qrow_t[qt]));
                        s[qt][r] = ok ? s[qt][r] * a.scale_log2 : -INFINITY;
                    }
                }
                float mx = fmaxf(fmaxf(s[qt][0], s[qt][1]), fmaxf(s[qt][2], s[qt][3]));
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                if (__any(mx > mref[qt] + kLazy)) {
                    const float mnew = fmaxf(mref[qt], mx);
                    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref[qt] - mnew);
                    mref[qt] = mnew;
                    lrun[qt] *= alpha;
#pragma unroll
                    for (int i = 0; i < S::DVT; ++i)
                        acc[i][qt] *= alpha;
                }
                const float muse = mref[qt] == -INFINITY ? 0.f : mref[qt];
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p[r] = fast_exp2(s[qt][r] - muse);
                lrun[qt] += (p[0] + p[1]) + (p[2] + p[3]);
                pb[qt] = u32x2{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])};
            }
            // O^T += V^T P^T: V read transposed out of the DMA'd tile — column dv of rows
            // 4*quad + j sits in DMA instruction (dv % QD) / 8 of lane group dv / QD
            const uint8_t *vslot = slot + S::KS * 1024;
#pragma unroll
            for (int dt = 0; dt < S::DVT; ++dt) {
                const int dv = dt * 16 + li;
                const int within = dv % S::QD;
                const uint8_t *col = vslot + (within >> 3) * 1024 + ((dv / S::QD) * 16 + 4 * quad) * 16 + (within & 7) * 2;
                const uint32_t e0 = *reinterpret_cast<const uint16_t *>(col);
                const uint32_t e1 = *reinterpret_cast<const uint16_t *>(col + 16);
                const uint32_t e2 = *reinterpret_cast<const uint16_t *>(col + 32);
                const uint32_t e3 = *reinterpret_cast<const uint16_t *>(col + 48);
                const u32x2 vop{e0 | (e1 << 16), e2 | (e3 << 16)};
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    acc[dt][qt] = mfma_bf16_k16(vop, pb[qt], acc[dt][qt]);
            }
        }
        wait_vmcnt<0>();              // trailing DMAs done before the LDS is reused
    }

    // ---- merge the four waves: row sums over lane groups, then waves 1..3 into wave 0 ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        lrun[qt] += __shfl_xor(lrun[qt], 16);
        lrun[qt] += __shfl_xor(lrun[qt], 32);
    }
    float *mAcc = reinterpret_cast<float *>(lds + S::TAB);
    float *mM = mAcc + 64 * S::ACC;
    float *mL = mM + S::QR;
    for (int src = 1; src < 4; ++src) {
        __syncthreads();              // ring / previous round no longer read
        if (w == src) {
#pragma unroll
            for (int i = 0; i < S::DVT; ++i)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    *reinterpret_cast<f32x4 *>(mAcc + ((i * QT + qt) * 64 + lane) * 4) = acc[i][qt];
            if (quad == 0) {
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    mM[qt * 16 + li] = mref[qt];
                    mL[qt * 16 + li] = lrun[qt];
                }
            }
        }
        __syncthreads();
        if (w == 0) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const float m2 = mM[qt * 16 + li];
                const float M = fmaxf(mref[qt], m2);
                const float f1 = M == -INFINITY ? 0.f : fast_exp2(mref[qt] - M);
                const float f2 = M == -INFINITY ? 0.f : fast_exp2(m2 - M);
                lrun[qt] = lrun[qt] * f1 + mL[qt * 16 + li] * f2;
                mref[qt] = M;
#pragma unroll
                for (int i = 0; i < S::DVT; ++i)
                    acc[i][qt] = acc[i][qt] * f1 +
                                 *reinterpret_cast<const f32x4 *>(mAcc + ((i * QT + qt) * 64 + lane) * 4) * f2;
            }
        }
    }
    if (w != 0)
        return;

    if (a.splits == 1) {
        // ---- final output straight from registers ----
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int row = qg * S::QR + qt * 16 + li;
            if (row >= a.GV)
                continue;
            const int t = row / a.G;
            const int h = g * a.G + (row - t * a.G);
            const float inv = 1.f / lrun[qt];
            uint16_t *o = a.out + ((int64_t)(b * a.nv + t) * a.Hq + h) * D;
#pragma unroll
            for (int i = 0; i < S::DVT; ++i) {
                const int dv = i * 16 + 4 * quad;
                *reinterpret_cast<u32x2 *>(o + dv) =
                    u32x2{pack_bf16x2(acc[i][qt][0] * inv, acc[i][qt][1] * inv),
                          pack_bf16x2(acc[i][qt][2] * inv, acc[i][qt][3] * inv)};
            }
            if (quad == 0)
                a.lse[((int64_t)b * a.Hq + h) * a.nv + t] = (mref[qt] + __log2f(lrun[qt])) * kLn2;
        }
        return;
    }

    // ---- split partial for the merge kernel: acc [QR][D], then m [QR], l [QR] ----
    const int64_t pstride = (int64_t)S::QR * D + 2 * S::QR;
    float *part = a.part + ((int64_t)pair * a.splits + split) * pstride;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int q = qt * 16 + li;
        if (qg * S::QR + q >= a.GV)
            continue;                 // padding rows are never merged
#pragma unroll
        for (int i = 0; i < S::DVT; ++i)
            *reinterpret_cast<f32x4 *>(part + (int64_t)q * D + i * 16 + 4 * quad) = acc[i][qt];
        if (quad == 0) {
            part[S::QR * D + q] = mref[qt];
            part[S::QR * D + S::QR + q] = lrun[qt];
        }
    }
}

// Merges the split partials of one (pair, 16-row query tile) in fixed split order:
// O = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s, LSE = M + log sum_s e^{m_s - M} l_s.
// Every (row, 4-column) item is one thread; the per-split maxima and sums of a row are
// read by all of its threads (cache hits), so there is a single round of loads.
template <int D, int QT>
__global__ __launch_bounds__(kThreads) void verify_attn_merge_kernel(AttnArgs a)
{
    constexpr int QR = QT * 16;
    constexpr int kPre = 8;           // splits whose partials are fetched before any math
    const int pair = blockIdx.x / QT;
    const int qt = blockIdx.x - pair * QT;
    const int qg = pair % a.qgroups;
    const int bg = pair / a.qgroups;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;
    const int row0 = qg * QR + qt * 16;
    const int rows = min(16, a.GV - row0);
    const int64_t pstride = (int64_t)QR * D + 2 * QR;
    const float *base = a.part + (int64_t)pair * a.splits * pstride;
    for (int item = threadIdx.x; item < rows * (D / 4); item += kThreads) {
        const int r = item / (D / 4);
        const int dv = (item - r * (D / 4)) * 4;
        const int q = qt * 16 + r;
        float ms[kPre], ls[kPre];
        f32x4 as[kPre];
#pragma unroll
        for (int sp = 0; sp < kPre; ++sp) {
            if (sp < a.splits) {
                const float *ps = base + sp * pstride;
                ms[sp] = ps[QR * D + q];
                ls[sp] = ps[QR * D + QR + q];
                as[sp] = *reinterpret_cast<const f32x4 *>(ps + (int64_t)q * D + dv);
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < kPre; ++sp)
            if (sp < a.splits)
                M = fmaxf(M, ms[sp]);
        for (int sp = kPre; sp < a.splits; ++sp)
            M = fmaxf(M, base[sp * pstride + QR * D + q]);
        f32x4 num{0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
#pragma unroll
        for (int sp = 0; sp < kPre; ++sp) {
            if (sp < a.splits) {
                const float wgt = fast_exp2(ms[sp] - M);
                num += wgt * as[sp];
                den += wgt * ls[sp];
            }
        }
        for (int sp = kPre; sp < a.splits; ++sp) {
            const float *ps = base + sp * pstride;
            const float wgt = fast_exp2(ps[QR * D + q] - M);
            num += wgt * *reinterpret_cast<const f32x4 *>(ps + (int64_t)q * D + dv);
            den += wgt * ps[QR * D + QR + q];
        }
        const float inv = 1.f / den;
        const int row = row0 + r;
        const int t = row / a.G;
        const int h = g * a.G + (row - t * a.G);
        uint16_t *o = a.out + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + dv;
        *reinterpret_cast<u32x2 *>(o) =
            u32x2{pack_bf16x2(num[0] * inv, num[1] * inv), pack_bf16x2(num[2] * inv, num[3] * inv)};
        if (dv == 0)
            a.lse[((int64_t)b * a.Hq + h) * a.nv + t] = (M + __log2f(den)) * kLn2;
    }
}

template <int D, int QT, int R>
hipError_t launch_qt(const AttnArgs &a, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL((verify_attn_split_kernel<D, QT, R>), grid, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1)
        return e;
    hipLaunchKernelGGL((verify_attn_merge_kernel<D, QT>), dim3((unsigned)(a.pairs * QT)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D, int R>
hipError_t launch_r(const AttnArgs &a, int qt, dim3 grid, hipStream_t st)
{
    switch (qt) {
    case 1: return launch_qt<D, 1, R>(a, grid, st);
    case 2: return launch_qt<D, 2, R>(a, grid, st);
    case 3: return launch_qt<D, 3, R>(a, grid, st);
    case 4: return launch_qt<D, 4, R>(a, grid, st);
    default: return launch_qt<D, 5, R>(a, grid, st);
    }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, int qt, int ring, dim3 grid, hipStream_t st)
{
    return ring >= 3 ? launch_r<D, 3>(a, qt, grid, st) : launch_r<D, 2>(a, qt, grid, st);
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
    const int list = max(1, max_list);
    int s = (target_wgs + p.pairs - 1) / max(1, p.pairs);
    s = max(s, (list + kSplitMax - 1) / kSplitMax);        // the token table holds kSplitMax positions
    s = max(1, min(min(s, (list + 15) / 16), kMaxSplits));
    p.spl = ((list + s - 1) / s + 15) / 16 * 16;
    p.splits = (list + p.spl - 1) / p.spl;
    p.part_floats = p.splits > 1 ? (size_t)p.pairs * p.splits * ((size_t)p.qt * 16 * 128 + 2 * p.qt * 16) : 0;
    p.grid = (size_t)((p.pairs + 7) / 8) * 8 * p.splits;
    return p;
}

hipError_t launch_attn(const AttnArgs &a, int head_dim, int qt, int ring, hipStream_t st)
{
    const dim3 grid((unsigned)(((a.pairs + 7) / 8) * 8 * a.splits));
    return head_dim == 64 ? launch_d<64>(a, qt, ring, grid, st) : launch_d<128>(a, qt, ring, grid, st);
}

}  // namespace dustin
