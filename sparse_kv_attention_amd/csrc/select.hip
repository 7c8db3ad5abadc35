// Hybrid budgeted selection of I_verify (English Dustin summary, "Methodology" 1, last
// two sentences): sinks and a recent window are always kept, then the top-m tokens by
// the draft score, then the best remaining tokens by the target score, for a set of
// fixed size.  Ties go to the smaller position; -0 and +0 compare equal.
//
// The two tiers run on two workgroups of one sequence at once when both are non-empty
// (and r + m <= kSelectCombineCap): the best r target picks outside the draft tier D are
// the best r of T' \ D, where T' is the best r + m of the same candidates by the target
// score (at most m of T' can be in D).  Workgroup 0 takes D by the draft score and
// workgroup 1 takes T' by the target score; each publishes its position mask and counts
// itself in on the sequence's counter (a device-scope atomic after a device-scope
// release), and the second to arrive reads the other's mask, takes the best r of T' \ D
// and writes the ordered set.  Neither waits for the other.  Otherwise one workgroup runs
// both tiers in turn.
//
// A tier's workgroup has 1024 threads.  Thread t owns the contiguous positions
// [t*E, t*E + E) and keeps their order-preserving 32-bit keys in registers.  Each tier
// finds its threshold key with an LDS radix select of up to four 8-bit passes (32
// histogram copies indexed by lane mod 32, with a padded stride: at most two lanes of a
// wave share a counter, and lanes counting the same digit hit different banks).  It
// takes every eligible key above the threshold plus the first `need` keys equal to it in
// position order (block-wide exclusive scan); when every key of the chosen digit bin is
// needed, the search stops there and takes the keys at or above that prefix.  The final
// set is compacted in ascending position order with one more block scan, staged in LDS
// and written with coalesced stores.  Integer-only after the key transform, so the
// result is bit-reproducible.
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kWaves = kSelectThreads / 64;
constexpr int kCopies = 32;              // lane-slot histogram copies
constexpr int kHistStride = 257;         // padded so copies sit in different banks

__device__ __forceinline__ uint32_t ord_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;                               // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one int across the 64 lanes of a wave, by DPP: shifts by 1, 2, 4 and
// 8 lanes within each row of 16 (lanes shifted in from outside the row add 0), then the
// last lane of row 0 (and of row 2) is broadcast into row 1 (and row 3), and the last lane
// of row 1 into rows 2 and 3.
__device__ __forceinline__ int wave_scan_incl(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return x;
}

// A sequence's selection parameters, clamped as the contract states; `parallel`: the two
// tiers run on two workgroups (both decide it alike).
struct SeqPlan {
    int N, k, s, w, md, r;
    bool parallel;
};

__device__ __forceinline__ SeqPlan seq_plan(const SelectArgs &a, int n_raw, int k_raw, int s_raw, int w_raw,
                                            int m_raw)
{
    SeqPlan p;
    p.N = clampi(n_raw, 0, a.n_max);
    p.k = clampi(k_raw, 0, min(p.N, a.k_max));
    p.s = clampi(s_raw, 0, p.k);
    p.w = clampi(w_raw, 0, p.k - p.s);
    p.md = a.score_draft ? clampi(m_raw, 0, p.k - p.s - p.w) : 0;
    p.r = p.k - p.s - p.w - p.md;
    p.parallel = a.ws != nullptr && p.k < p.N && p.md > 0 && p.r > 0 && p.r + p.md <= kSelectCombineCap;
    return p;
}

// masks of the lowest n bits, n in [0, 64]
__device__ __forceinline__ uint64_t low_bits(int n) { return n >= 64 ? ~0ull : (1ull << n) - 1; }

// Exclusive scan of one int per thread over a block of NT threads (NT / 64 waves).
template <int NT = kSelectThreads>
__device__ int block_scan(int v, int &total, int *sScan)
{
    constexpr int NWV = NT / 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int x = wave_scan_incl(v);
    if (lane == 63)
        sScan[wid] = x;
    __syncthreads();
    if (wid == 0) {
        const int t = lane < NWV ? sScan[lane] : 0;
        const int y = wave_scan_incl(t);
        if (lane < NWV)
            sScan[lane] = y - t;
        if (lane == NWV - 1)
            sScan[NWV] = y;
    }
    __syncthreads();
    const int r = sScan[wid] + x - v;
    total = sScan[NWV];
    __syncthreads();
    return r;
}

struct SelShared {
    uint32_t hist[2][kCopies * kHistStride];   // alternating: one is counted, the other cleared
    int part[kSelectThreads / 256][256];       // per-bin sums over a quarter of the copies
    int scan[kWaves + 1];
    int bcast[3];
    int32_t lpos[kSelectCombineCap];           // two-workgroup path: T' \ D in position order
    unsigned long long tw[kSelectThreads];     // ... and T: bit e of word t = position t*E + e
};

// arrival counter word of the two-workgroup path: [63:24] tag, [15:0] arrivals.  A word
// without the tag (a fresh or foreign workspace) counts as zero arrivals.
constexpr unsigned long long kSelTag = 0x5e1ec7d2a9ull << 24;
constexpr unsigned long long kSelTagMask = ~0ull << 24;

// Threshold of the `kth` largest eligible key (1 <= kth <= #eligible): returns the
// threshold key and, in `need`, how many keys equal to it belong to the top kth.  When,
// before the last pass, every key of the digit bin just chosen belongs to the top kth, the
// search stops there: `whole` is set, and the top kth are exactly the keys >= the returned
// prefix (its lower digits zero).
// Per 8-bit pass: every thread counts its keys into the current histogram (lane-slot
// copies, one atomic per counted key); barrier; every thread sums one bin over
// a quarter of the copies and clears its share of the other histogram (for the next
// pass); barrier; wave 0 adds the four quarters of its 4 bins per lane, scans the bins
// from the top with shuffles and picks the digit; a last barrier publishes it.  hist[0]
// must be zero on entry and is zero again on return (an odd pass counts into hist[1],
// which the next call's first pass clears; a stop after an even pass clears hist[0]).
template <int E>
__device__ uint32_t radix_select(const uint32_t (&key)[E], uint64_t elig, int kth, int &need,
                                 bool &whole, SelShared &sh)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int slot = lane % kCopies;
    uint32_t prefix = 0;
    need = kth;
    whole = false;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        uint32_t *hist = sh.hist[pass & 1];
        uint32_t *other = sh.hist[(pass + 1) & 1];
        // every eligible key that agrees with the prefix found so far adds one to its
        // digit's counter (a masked LDS atomic per key, no branches around it)
        const uint32_t hmask = pass == 0 ? 0u : ~0u << (shift + 8);
        const uint32_t want = prefix & hmask;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (((elig >> e) & 1) && (key[e] & hmask) == want)
                atomicAdd(&hist[slot * kHistStride + ((key[e] >> shift) & 255)], 1u);
        }
        __syncthreads();
        {
            constexpr int kQ = kSelectThreads / 256;          // quarters of the copies
            constexpr int kPerQ = kCopies / kQ;
            const int bin = tid & 255, q = tid >> 8;
            int v = 0;
#pragma unroll
            for (int cp = 0; cp < kPerQ; ++cp)
                v += (int)hist[(q * kPerQ + cp) * kHistStride + bin];
            sh.part[q][bin] = v;
            for (int i = tid; i < kCopies * kHistStride; i += kSelectThreads)
                other[i] = 0;
        }
        __syncthreads();
        if (tid < 64) {
            // lane holds bins 255-4l .. 252-4l (descending)
            int c[4], tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int bin = 255 - 4 * lane - j;
                int v = 0;
#pragma unroll
                for (int q = 0; q < kSelectThreads / 256; ++q)
                    v += sh.part[q][bin];
                c[j] = v;
                tot += v;
            }
            const int incl = wave_scan_incl(tot);
            int before = incl - tot;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (before < need && before + c[j] >= need) {
                    sh.bcast[0] = 255 - 4 * lane - j;
                    sh.bcast[1] = need - before;
                    sh.bcast[2] = c[j];
                }
                before += c[j];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh.bcast[0] << shift;
        need = sh.bcast[1];
        if (pass < 3 && need == sh.bcast[2]) {   // the whole bin is taken (uniform)
            whole = true;
            if ((pass & 1) == 0) {
                for (int i = tid; i < kCopies * kHistStride; i += kSelectThreads)
                    hist[i] = 0;
                __syncthreads();
            }
            break;
        }
    }
    return prefix;
}

// Marks the top `kth` eligible keys (threshold + position-ordered ties).
template <int E>
__device__ uint64_t take_top(const uint32_t (&key)[E], uint64_t elig, int kth, SelShared &sh)
{
    int need;
    bool whole;
    const uint32_t thr = radix_select<E>(key, elig, kth, need, whole, sh);
    uint64_t sel = 0;
    if (whole) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            sel |= (uint64_t)(((elig >> e) & 1) && key[e] >= thr) << e;
        return sel;
    }
    int eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {   // branch-free
        const bool el = (elig >> e) & 1;
        sel |= (uint64_t)(el && key[e] > thr) << e;
        eq += (el && key[e] == thr) ? 1 : 0;
    }
    int total;
    int before = block_scan(eq, total, sh.scan);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool tie = ((elig >> e) & 1) && key[e] == thr;
        sel |= (uint64_t)(tie && before < need) << e;
        before += tie ? 1 : 0;
    }
    return sel;
}

// The raw bits of the thread's E scores (positions base .. base+E-1 of one score row):
// 16-byte loads when the row is 16-byte aligned and the range lies inside it, else scalar
// loads at clamped positions (n_max >= 1).
template <int E>
__device__ __forceinline__ void load_raw(uint32_t (&raw)[E], const float *row, int base, int n_max)
{
    if ((n_max & 3) == 0 && base + E <= n_max) {
        const float4 *p = reinterpret_cast<const float4 *>(row + base);
        float4 v[E / 4];
#pragma unroll
        for (int i = 0; i < E / 4; ++i)
            v[i] = p[i];
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            raw[4 * i] = __float_as_uint(v[i].x);
            raw[4 * i + 1] = __float_as_uint(v[i].y);
            raw[4 * i + 2] = __float_as_uint(v[i].z);
            raw[4 * i + 3] = __float_as_uint(v[i].w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            raw[e] = __float_as_uint(row[min(base + e, n_max - 1)]);
    }
}

// Raw score bits -> order-preserving keys, 0 outside `valid`.
template <int E>
__device__ __forceinline__ void to_keys(uint32_t (&key)[E], uint64_t valid)
{
#pragma unroll
    for (int e = 0; e < E; ++e)
        key[e] = ((valid >> e) & 1) ? ord_key(__uint_as_float(key[e])) : 0u;
}

// The best r of the `total` listed candidates (C contiguous list entries per thread, so
// list order, which is position order, breaks ties) by the target score: their bits are
// set in the T mask.
template <int C, int E>
__device__ void take_listed(const SelectArgs &a, int b, int total, int r, SelShared &sh)
{
    const int tid = threadIdx.x;
    const float *row = a.score_target + (int64_t)b * a.n_max;
    int32_t p2[C];
    uint32_t k2[C];
    uint64_t e2 = 0;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int li = tid * C + i;
        const bool ok = li < total;
        p2[i] = ok ? sh.lpos[li] : 0;
        e2 |= (uint64_t)ok << i;
    }
#pragma unroll
    for (int i = 0; i < C; ++i)
        k2[i] = ((e2 >> i) & 1) ? ord_key(row[p2[i]]) : 0u;
    const uint64_t s2 = take_top<C>(k2, e2, r, sh);
#pragma unroll
    for (int i = 0; i < C; ++i)
        if ((s2 >> i) & 1)
            atomicOr(&sh.tw[p2[i] / E], 1ull << (p2[i] % E));
}

// The second workgroup of the two-workgroup path: thread t holds word t of D and of T'
// (positions [t*E, t*E + E)); T' \ D is listed in position order and the best r of it
// (r <= |T' \ D| <= r + m <= kSelectCombineCap) are returned as this thread's word of T.
template <int E>
__device__ uint64_t finish_target(const SelectArgs &a, int b, int base, uint64_t d, uint64_t tp, int r,
                                  SelShared &sh)
{
    const int tid = threadIdx.x;
    const uint64_t cw = tp & ~d;
    int total;
    int off = block_scan(__popcll(cw), total, sh.scan);
    uint64_t m = cw;
    while (m) {
        const int e = __builtin_ctzll(m);
        m &= m - 1;
        if (off < kSelectCombineCap)
            sh.lpos[off] = base + e;
        ++off;
    }
    sh.tw[tid] = 0;
    __syncthreads();
    total = min(total, kSelectCombineCap);
    if (total <= 2 * kSelectThreads)
        take_listed<2, E>(a, b, total, r, sh);
    else
        take_listed<4, E>(a, b, total, r, sh);
    __syncthreads();
    return sh.tw[tid];
}

template <int E>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a)
{
    __shared__ SelShared sh;
    // With two workgroups per sequence, blocks 16o + j (j < 8) take the draft tier of
    // sequence 8o + j and blocks 16o + 8 + j its target superset: both have the same
    // blockIdx % 8 and so run on one XCD (workgroups are dispatched round-robin over the
    // XCDs), where the masks are exchanged through that XCD's L2.
    const bool two = a.ws != nullptr && a.score_draft != nullptr;
    const int x = blockIdx.x;
    const int b = two ? (x >> 4) * 8 + (x & 7) : x;
    const int role = two ? (x >> 3) & 1 : 0;   // 0: the draft tier, or both in turn; 1: the target superset
    if (b >= a.B)
        return;
    const int tid = threadIdx.x;
    const int base = tid * E;
    // the workgroup's first scores are requested first, before the sequence's arguments are
    // known
    uint32_t key[E];
    const float *first = role == 0 ? a.score_draft : a.score_target;
    if (first && a.n_max > 0)
        load_raw<E>(key, first + (int64_t)b * a.n_max, base, a.n_max);
    // every per-sequence argument in one round of loads
    const int n_raw = a.ctx_len[b], k_raw = a.budget[b], s_raw = a.n_sink[b], w_raw = a.n_window[b];
    const int m_raw = a.score_draft ? a.m[b] : 0;
    const SeqPlan P = seq_plan(a, n_raw, k_raw, s_raw, w_raw, m_raw);
    if (role == 1 && !P.parallel) {
        wait_vmcnt<0>();   // the early score loads
        return;
    }
    const int N = P.N, k = P.k;
    int32_t *out = a.idx + (int64_t)b * a.k_max;
    if (role == 0 && tid == 0)
        a.count[b] = k;
    if (k == N) {
        for (int i = tid; i < a.k_max; i += kSelectThreads)
            out[i] = i < N ? i : -1;
        wait_vmcnt<0>();   // the early score loads
        return;
    }
    const int s = P.s, w = P.w, md = P.md, r = P.r;

    // the thread's positions base + e: valid below N, protected below s (sinks) or at N - w
    // and above (window)
    const uint64_t valid = low_bits(clampi(N - base, 0, E));
    const uint64_t prot = low_bits(clampi(s - base, 0, E)) | (valid & ~low_bits(clampi(N - w - base, 0, E)));
    for (int i = tid; i < kCopies * kHistStride; i += kSelectThreads)
        sh.hist[0][i] = 0;
    __syncthreads();
    // the two tiers run the same code (one loop body): the selection code is fetched into
    // the instruction cache once, not once per tier
    // On the two-workgroup path this workgroup runs its own tier alone: D, the best md by
    // the draft score (role 0), or T', the best r + md by the target score (role 1, with
    // its scores already requested); the second to finish does the rest.
    uint64_t selD = 0, selT = 0;
    const int t_lo = P.parallel ? role : 0, t_hi = P.parallel ? role + 1 : 2;
#pragma unroll 1
    for (int tier = t_lo; tier < t_hi; ++tier) {
        const int kth = tier == 0 ? md : (P.parallel ? r + md : r);
        if (kth <= 0)
            continue;
        // the thread's position and masks are made opaque to the compiler at the top of
        // the body, so what is formed from them per key (addresses, mask tests) is formed
        // in the loop rather than hoisted out of it and held, or spilled, through the tiers
        int bs = base;
        uint64_t vl = valid, pr = prot;
        asm volatile("" : "+v"(bs), "+v"(vl), "+v"(pr));
        if (tier == 1 && !P.parallel) {
            const float *row = a.score_target + (int64_t)b * a.n_max;
            asm volatile("" : "+s"(row));
            load_raw<E>(key, row, bs, a.n_max);
        }
        to_keys<E>(key, vl);
        const uint64_t sel = take_top<E>(key, vl & ~pr & ~selD, kth, sh);
        if (tier == 0)
            selD = sel;
        else
            selT = sel;
    }
    if (P.parallel) {
        // publish this tier's mask, then count in; the second workgroup to arrive has both
        unsigned long long *wsb = a.ws + (int64_t)b * 2 * kSelectThreads;
        wsb[role * kSelectThreads + tid] = role == 0 ? selD : selT;
        wait_vmcnt<0>();   // this wave's mask store is acknowledged
        __syncthreads();   // ... and every wave's
        if (tid == 0) {
            unsigned long long *ctr = a.ws + (int64_t)a.B * 2 * kSelectThreads + b;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // the masks before the count
            unsigned long long old = kSelTag, nw = 0;
            for (;;) {   // compare-and-swap; retries only when the other workgroup arrived meanwhile
                const unsigned long long cur = (old & kSelTagMask) == kSelTag ? old : kSelTag;
                nw = cur + 1;
                if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT))
                    break;
            }
            const bool second = (nw & 0xffff) >= 2;
            if (second) {   // both have arrived: the next call starts from zero
                __hip_atomic_store(ctr, kSelTag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other mask after the count
            }
            sh.bcast[0] = second ? 1 : 0;
        }
        __syncthreads();
        if (sh.bcast[0] == 0)
            return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const uint64_t other = wsb[(1 - role) * kSelectThreads + tid];
        if (role == 0)
            selT = other;
        else
            selD = other;
        selT = finish_target<E>(a, b, base, selD, selT, r, sh);
    }
    const uint64_t fin = prot | selD | selT;
    int total;
    int o = block_scan(__popcll(fin), total, sh.scan);
    constexpr int kStageWords = 2 * kCopies * kHistStride;
    if (a.k_max <= kStageWords) {
        // the histograms are no longer needed: the positions are placed there in order and
        // then written out with coalesced stores
        int32_t *stage = reinterpret_cast<int32_t *>(&sh.hist[0][0]);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (((fin >> e) & 1) && o < a.k_max)
                stage[o++] = base + e;
        __syncthreads();
        const int n_out = min(total, a.k_max);
        for (int i = tid; i < a.k_max; i += kSelectThreads) {
            if (i >= k)
                out[i] = -1;
            else if (i < n_out)
                out[i] = stage[i];
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (((fin >> e) & 1) && o < a.k_max)
            out[o++] = base + e;
    for (int i = k + tid; i < a.k_max; i += kSelectThreads)
        out[i] = -1;
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t st)
{
    const int e = (a.n_max + kSelectThreads - 1) / kSelectThreads;
    // the second workgroup of a sequence only when a draft tier can exist and the
    // workspace holds the masks
    const dim3 grid(a.ws != nullptr && a.score_draft != nullptr ? 16u * (unsigned)((a.B + 7) / 8) : (unsigned)a.B);
    const dim3 block(kSelectThreads);
    if (e <= 4)
        hipLaunchKernelGGL(select_kernel<4>, grid, block, 0, st, a);
    else if (e <= 8)
        hipLaunchKernelGGL(select_kernel<8>, grid, block, 0, st, a);
    else if (e <= 16)
        hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, st, a);
    else if (e <= 32)
        hipLaunchKernelGGL(select_kernel<32>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(select_kernel<64>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace dustin
