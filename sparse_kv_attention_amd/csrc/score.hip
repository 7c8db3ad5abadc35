// SRH importance scoring (English Dustin summary, "Methodology" 1 and 2: attention scores
// of the target-historical and draft-lookahead queries, computed on the semantic
// retrieval heads only, summed into one importance value per context token; German
// Vegas summary 2A/2B for the logit-sum mode over the first and bonus queries).
//
// Softmax mode (PROB_SUM), two kernels:
//   srh_prob_logits  one workgroup per (share of a stream's tiles, group, sequence); the
//                    grid is one resident round of CU-filling workgroups.  Each wave
//                    claims 64-token tiles from the workgroup's counter, reads a tile's
//                    key rows with coalesced non-temporal 16-byte loads into its own LDS
//                    area, and keeps the next tile in flight in registers; no workgroup
//                    barrier is taken per tile.  Dot products run on the matrix cores
//                    (bf16 in, one fp32 sum per 32-element chunk of the head dim, the
//                    chunks added in fp64).  Logits are stored as fp32 offsets from the
//                    maximum of their 64-token statistics tile, so tokens near the
//                    maximum — the ones that carry probability mass — keep full relative
//                    precision even when logits are large.  Every tile leaves its maximum
//                    and sum of exp2 per pair; every workgroup folds its tiles, in tile
//                    order, into one (max, sum of exp2) per pair.
//   srh_finalize     one workgroup per (1024 tokens, sequence): per pair, the global max
//                    and 1/Z from the workgroup partials (one wave per pair, loads of
//                    several pairs in flight together), then per token the sum over pairs
//                    of exp2(offset + tile max - max) / Z.
// Logit-sum modes (LOGIT_SUM2: queries 0 and n_q-1; LOGIT_SUM_ALL: every query):
// srh_logit_sum computes the raw scaled logits on MFMA (bf16 in, fp32 accumulate; the
// sum's tolerance scales with the sum of |logits|), adds a group's pairs in registers and
// writes one row per group; the finalize kernel sums the groups per token.
// Every pass streams: the K stream is read once, the logit workspace written once and
// read once.
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kThreads = 256;

// Whole-wave reductions without LDS: quad_perm xor 1 and xor 2, row_half_mirror (the other
// quad of the 8 lanes), row_mirror (the other half of the 16-lane row), then the
// permlane16 / permlane32 swaps across rows.  Every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ double dpp64(double v)
{
    const uint64_t u = __double_as_longlong(v);
    const uint64_t lo = dpp32<CTRL>((uint32_t)u), hi = dpp32<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ __forceinline__ double swap_max_f64(double v, bool wide)
{
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto a = wide ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = wide ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const double x = __longlong_as_double((long long)(((uint64_t)b[0] << 32) | a[0]));
    const double y = __longlong_as_double((long long)(((uint64_t)b[1] << 32) | a[1]));
    return fmax(x, y);
}

// In-place max (MAX) or sum over each 16-lane row of N values per lane; every lane of a
// row ends with its row's results.
template <int N, bool MAX>
__device__ __forceinline__ void row16_reduce_f32(float (&v)[N])
{
    auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = op(v[i], __uint_as_float(dpp32<0xB1>(__float_as_uint(v[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = op(v[i], __uint_as_float(dpp32<0x4E>(__float_as_uint(v[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = op(v[i], __uint_as_float(dpp32<0x141>(__float_as_uint(v[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = op(v[i], __uint_as_float(dpp32<0x140>(__float_as_uint(v[i]))));
}

__device__ __forceinline__ double wave_max_f64_dpp(double v)
{
    v = fmax(v, dpp64<0xB1>(v));
    v = fmax(v, dpp64<0x4E>(v));
    v = fmax(v, dpp64<0x141>(v));
    v = fmax(v, dpp64<0x140>(v));
    v = swap_max_f64(v, false);
    return swap_max_f64(v, true);
}

__device__ __forceinline__ double swap_add_f64(double v, bool wide)
{
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto a = wide ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = wide ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const double x = __longlong_as_double((long long)(((uint64_t)b[0] << 32) | a[0]));
    const double y = __longlong_as_double((long long)(((uint64_t)b[1] << 32) | a[1]));
    return x + y;
}

// Sum over the 64 lanes, every lane ending with it: the same exchange pattern as
// wave_max_f64_dpp (pairs, quads, half rows, rows, then the row and half swaps).
__device__ __forceinline__ double wave_sum_f64_dpp(double v)
{
    v += dpp64<0xB1>(v);
    v += dpp64<0x4E>(v);
    v += dpp64<0x141>(v);
    v += dpp64<0x140>(v);
    v = swap_add_f64(v, false);
    return swap_add_f64(v, true);
}

// Waves per workgroup of the softmax-mode logit kernel: two per SIMD.  One workgroup
// fills a CU, so all of a CU's waves draw tiles from one counter and none is left running
// alone at the end.
constexpr int kProbWaves = 8;

// The 32-lane halves of a wave exchanged (permlane32 swap), then the 16-lane rows within
// each half (permlane16 swap): combines the four lanes l % 16 + 16 k, for N values per
// lane; every lane ends with its column's results.
template <int N, bool MAX>
__device__ __forceinline__ void column_reduce_f32(float (&v)[N])
{
    auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t u = __float_as_uint(v[i]);
        const auto t = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v[i] = op(__uint_as_float(t[0]), __uint_as_float(t[1]));
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t u = __float_as_uint(v[i]);
        const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v[i] = op(__uint_as_float(t[0]), __uint_as_float(t[1]));
    }
}

// Pages of one workgroup's share the softmax-mode kernel resolves into LDS at its start.
constexpr int kPageCache = 4096;

// LDS bytes of one wave's staged tile at head dim D (row stride 2D + 16: conflict-free
// 16-byte row reads)
__host__ __device__ constexpr int prob_tile_bytes(int D) { return kStatTile * (2 * D + 16); }

// One workgroup of the softmax-mode logit kernel for group G (head dim D).  sK: the waves'
// tile areas (kProbWaves x prob_tile_bytes(D)); sNext: the workgroup's tile counter.
// FLAT: every group's view is unpaged with a row stride below 4 GiB, so a row address is a
// per-workgroup base plus token x stride (one 32x32->64 multiply-add per load).
// setup: zero the tile counter (and fill the page cache) behind a workgroup barrier; a
// caller that zeroed the counter at kernel start passes false (unpaged views only).
// wave_bytes: the stride of the waves' LDS areas (at least prob_tile_bytes(D)).  sDone:
// nullptr, or a zeroed LDS counter of the waves done with the group: then no barrier ends
// the group, and the last wave to finish folds it alone while the others go on.
template <int D, bool FLAT>
__device__ __forceinline__ void prob_logits(const ScoreArgs &a, const ScoreGroup &G, int b, int part, uint8_t *sK,
                                            int &sNext, int *sPage, bool setup = true,
                                            int wave_bytes = prob_tile_bytes(D), int *sDone = nullptr)
{
    constexpr int NW = kProbWaves;
    constexpr int NT = 64 * NW;
    constexpr int KS = D / 32;          // MFMA k-steps of a row (32 elements each)
    constexpr int kDepth = FLAT ? 2 : 1;   // tiles in flight in registers per wave
    constexpr int RB = D * 2;           // bytes per key row
    constexpr int RSTR = RB + 16;       // LDS row stride
    constexpr int CPR = RB / 16;        // 16-byte chunks per row
    constexpr int LPT = kStatTile * CPR / 64;   // 16-byte loads per lane per 64-token tile
    const ScoreSig &S = a.sig[G.sig];
    const int N = clampi(a.ctx_len[b], 0, S.ctx_clamp);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane >> 4;
    const int li = lane & 15;
    // 64-token tiles holding context tokens; this workgroup takes an equal share of them
    const int n_live = (N + kStatTile - 1) / kStatTile;
    const int q_lo = (int)((int64_t)n_live * part / G.parts);
    const int q_hi = (int)((int64_t)n_live * (part + 1) / G.parts);

    // statistics tiles past the live tiles: empty
    for (int st = n_live + part; st < a.n_tiles; st += G.parts)
        for (int p = tid; p < G.n_pairs; p += NT) {
            const int64_t e = ((int64_t)b * S.total_pairs + G.pair0 + p) * a.n_tiles + st;
            S.tile_max[e] = -INFINITY;
        }
    if (q_lo >= q_hi) {
        // the empty partial in this workgroup's slot and the slots past the group's
        // workgroups that it covers
        for (int p = tid; p < G.n_pairs; p += NT) {
            const int64_t e = ((int64_t)b * S.total_pairs + G.pair0 + p) * a.n_parts;
            for (int x = part; x < a.n_parts; x += G.parts) {
                S.part_max[e + x] = -INFINITY;
                S.part_sum[e + x] = 0.0;
            }
        }
        return;
    }
    // The group's queries as the MFMA B operand, in registers for every tile: lane holds
    // pair li (zero past the group's pairs), head-dim elements 32 ks + 8 quad .. +8
    u32x4 qop[KS];
    {
        const int p = li;
        const uint16_t *qp = nullptr;
        if (p < G.n_pairs) {
            const int hl = p / S.n_q;
            const int j = p - hl * S.n_q;
            qp = S.q + ((int64_t)(b * S.total_qheads + G.q_head0 + hl) * S.n_q + j) * D + quad * 8;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[ks] = qp ? load16(qp + ks * 32) : u32x4{0, 0, 0, 0};
    }
    // Paged views: the pages of this workgroup's share, resolved once into LDS (clamped page
    // ids), so a row's address needs no page-table load of its own; shares spanning more
    // pages than the cache holds look each row's page up.  Rows past the share read row N-1
    // through its own offset.
    bool cached = false;
    int pfirst = 0;
    int64_t off_last = 0;
    if constexpr (!FLAT) {
        off_last = kv_offset(G.k, b, N - 1, G.kv_head);
        if (G.k.pt) {
            const int ps = G.k.ps_log2;
            pfirst = (q_lo * kStatTile) >> ps;
            const int plast = (min(q_hi * kStatTile, N) - 1) >> ps;
            cached = plast - pfirst + 1 <= kPageCache;
            if (cached)
                for (int i = tid; i <= plast - pfirst; i += NT)
                    sPage[i] = clampi(G.k.pt[(int64_t)b * G.k.max_pages + pfirst + i], 0, G.k.num_pages - 1);
        }
    }
    if (setup) {
        if (tid == 0)
            sNext = 0;
        __syncthreads();              // the tile counter and the page cache ready
    }
    uint8_t *myK = sK + w * wave_bytes;

    // A wave's tile is 64 tokens: lane l loads chunks l + 64 i (row = chunk / CPR) of the
    // tile's rows (whole rows per instruction: the coalescing the matrix-core operand
    // layout would not give), all issued at once, kDepth tiles in flight in registers per
    // lane.  Loads are unconditional (positions past the context, and tiles past the
    // workgroup's share, read row N-1, which is discarded), so the waits count exactly.
    const char *flat_base = reinterpret_cast<const char *>(G.k.base + (int64_t)b * G.k.sb + (int64_t)G.kv_head * G.k.sh) +
                            (lane % CPR) * 16;
    const uint32_t flat_st = (uint32_t)(G.k.st * 2);
    auto issue = [&](u32x4 (&kr)[LPT], int tile) {
        const int t0 = tile * kStatTile;
        // a tile past the share (the last claims of every wave) reads row N-1 only: its
        // rows may be live rows of the next workgroup's share, which would then be fetched
        // twice
        const bool mine = tile < q_hi;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = lane + i * 64;
            const int r = c / CPR;
            const int t = mine ? min(t0 + r, N - 1) : N - 1;
            const u32x4 *src;
            if constexpr (FLAT) {
                src = reinterpret_cast<const u32x4 *>(flat_base + (uint64_t)(uint32_t)t * flat_st);
            } else {
                int64_t off;
                if (!mine || t0 + r >= N)
                    off = off_last;
                else if (cached)
                    off = (int64_t)sPage[(t >> G.k.ps_log2) - pfirst] * G.k.sp +
                          (int64_t)(t & ((1 << G.k.ps_log2) - 1)) * G.k.st + (int64_t)G.kv_head * G.k.sh;
                else
                    off = kv_offset(G.k, b, t, G.kv_head);
                src = reinterpret_cast<const u32x4 *>(G.k.base + off + (c - r * CPR) * 8);
            }
            kr[i] = __builtin_nontemporal_load(src);
        }
    };
    // Only the wave itself reads its LDS tile, and a wave's LDS accesses complete in
    // order, so no workgroup barrier is needed; the fences keep the compiler from moving
    // LDS accesses across the staging.
    auto stage = [&](const u32x4 (&kr)[LPT]) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = lane + i * 64;
            const int r = c / CPR;
            *reinterpret_cast<u32x4 *>(&myK[r * RSTR + (c - r * CPR) * 16]) = kr[i];
        }
        wait_lgkm0();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };
    // One staged 64-token tile.  Dot products on the matrix cores: row block rb (16
    // tokens) times the 16 pairs, one v_mfma_f32_16x16x32_bf16 per 32-element chunk of the
    // head dim, each from a zero accumulator; the chunk sums are added in fp64.  The bf16
    // products are exact in fp32 and the instruction rounds each 32-term sum once (terms
    // far below its largest product can be dropped), so a logit's error is a few fp32 ulps
    // of its largest 32-term partial sum.  Lane l ends with pair l % 16 of tokens
    // 16 rb + 4 (l / 16) + r, r < 4.
    auto process = [&](int tile) {
        double lg[4][4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            f32x4 c[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 kop = *reinterpret_cast<const u32x4 *>(&myK[(16 * rb + li) * RSTR + (ks * 4 + quad) * 16]);
                c[ks] = mfma_bf16(kop, qop[ks], f32x4{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                double v = (double)c[0][r];
#pragma unroll
                for (int ks = 1; ks < KS; ++ks)
                    v += (double)c[ks][r];
                lg[rb][r] = v;
            }
        }
        // ---- the 64 tokens are one statistics tile: per pair, the maximum of the
        // fp32-rounded logits (rounding is monotonic, so it is the rounded true maximum)
        // as the tile's reference, offsets against it formed in fp64, sum of exp2 ----
        const int tok0 = tile * kStatTile + 4 * quad;          // + 16 rb + r
        double lp[4][4];
        float red[1] = {-INFINITY};
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lp[rb][r] = tok0 + 16 * rb + r < N ? lg[rb][r] * S.mul : -INFINITY;
                red[0] = fmaxf(red[0], (float)lp[rb][r]);
            }
        column_reduce_f32<1, true>(red);
        const float mx = red[0];
        float off[4][4];
        red[0] = 0.f;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool vld = tok0 + 16 * rb + r < N;
                off[rb][r] = vld ? (float)(lp[rb][r] - (double)mx) : -INFINITY;
                red[0] += vld ? fast_exp2(off[rb][r]) : 0.f;
            }
        column_reduce_f32<1, false>(red);
        if (li < G.n_pairs) {
            const int64_t row = (int64_t)b * S.total_pairs + G.pair0 + li;
            // four consecutive tokens per store; tok0 + 16 rb < N <= n_pad, both multiples
            // of four, so the four stay inside the row
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                if (tok0 + 16 * rb < N)
                    *reinterpret_cast<f32x4 *>(S.logits + row * a.n_pad + tok0 + 16 * rb) =
                        f32x4{off[rb][0], off[rb][1], off[rb][2], off[rb][3]};
            if (quad == 0 && tile < a.n_tiles) {
                S.tile_max[row * a.n_tiles + tile] = (double)mx;
                S.tile_sum[row * a.n_tiles + tile] = (double)red[0];
            }
        }
    };
    // Tiles are claimed one at a time from the workgroup's counter, so a wave that gets
    // less of the SIMDs than its neighbours simply takes fewer tiles.  A wave's claims
    // increase, so the loop ends at the first claim past the share, and every later buffer
    // of the round holds a tile past it too (single exit: the compiler's waits then keep
    // the other kDepth-1 tiles in flight).
    auto claim = [&]() {
        int v = 0;
        if (lane == 0)
            v = atomicAdd(&sNext, 1);
        return q_lo + __builtin_amdgcn_readfirstlane(v);
    };
    int qs[kDepth];
    u32x4 kr[kDepth][LPT];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        qs[d] = claim();
        __builtin_amdgcn_sched_barrier(0);   // tile d's loads after tile d-1's, as in the loop
        issue(kr[d], qs[d]);
    }
    while (qs[0] < q_hi) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            stage(kr[d]);
            const int nq = claim();
            issue(kr[d], nq);
            if (d == 0 || qs[d] < q_hi)
                process(qs[d]);
            qs[d] = nq;
        }
    }
    // This workgroup's (max, sum of exp2(l - max)) per pair over its tiles, folded in a
    // fixed order whichever wave took a tile, so the result does not depend on the claims:
    // one wave per pair (or the last wave every pair), lane i folding tiles q_lo + i,
    // q_lo + i + 64, ... in order (both values of a tile requested together), then the
    // lanes combined by a fixed butterfly.
    int p_first = w, p_step = NW;
    if (sDone) {
        // this wave's tile records are stored; the last wave to count in has them all
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        int v = 0;
        if (lane == 0)
            v = atomicAdd(sDone, 1);
        if (__builtin_amdgcn_readfirstlane(v) != NW - 1)
            return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        p_first = 0;
        p_step = 1;
    } else {
        __syncthreads();              // every tile's (max, sum) is stored
    }
    for (int p = p_first; p < G.n_pairs; p += p_step) {
        const int64_t row = ((int64_t)b * S.total_pairs + G.pair0 + p) * a.n_tiles;
        double Ml = -INFINITY, Sl = 0.0;
        for (int t = q_lo + lane; t < q_hi; t += 64) {
            const double m = S.tile_max[row + t], sm = S.tile_sum[row + t];
            if (m > -INFINITY) {
                const double M1 = fmax(Ml, m);
                Sl = (Ml > -INFINITY ? Sl * (double)fast_exp2((float)(Ml - M1)) : 0.0) +
                     sm * (double)fast_exp2((float)(m - M1));
                Ml = M1;
            }
        }
        const double M = wave_max_f64_dpp(Ml);
        const double Z = wave_sum_f64_dpp(Ml > -INFINITY ? Sl * (double)fast_exp2((float)(Ml - M)) : 0.0);
        if (lane == 0) {
            const int64_t e = ((int64_t)b * S.total_pairs + G.pair0 + p) * a.n_parts;
            S.part_max[e + part] = M;
            S.part_sum[e + part] = Z;
            // the record's slots beyond the group's workgroups hold the empty partial, so
            // the finalize folds every slot without knowing the group's count
            for (int x = G.parts + part; x < a.n_parts; x += G.parts) {
                S.part_max[e + x] = -INFINITY;
                S.part_sum[e + x] = 0.0;
            }
        }
    }
}


// One workgroup's share of group G, on the path of the group's head dim (DM: the head dim
// of every group launched, or 0 when both occur).
template <int DM, bool FLAT>
__device__ __forceinline__ void prob_group(const ScoreArgs &a, const ScoreGroup &G, int b, int part, uint8_t *sK,
                                           int &sNext, int *sPage)
{
    if constexpr (DM == 64) {
        prob_logits<64, FLAT>(a, G, b, part, sK, sNext, sPage);
    } else if constexpr (DM == 128) {
        prob_logits<128, FLAT>(a, G, b, part, sK, sNext, sPage);
    } else {
        if (a.sig[G.sig].head_dim == 64)
            prob_logits<64, FLAT>(a, G, b, part, sK, sNext, sPage);
        else
            prob_logits<128, FLAT>(a, G, b, part, sK, sNext, sPage);
    }
}

// DM: the head dim of every group launched (64 or 128), or 0 when the launch holds groups
// of both head dims (each workgroup then takes its group's path; the LDS is sized for 128).
template <int DM, bool FLAT>
__global__ __launch_bounds__(64 * kProbWaves)
__attribute__((amdgpu_waves_per_eu(kProbWaves / 4))) void srh_prob_logits_kernel(ScoreArgs a)
{
    __shared__ __align__(16) uint8_t sK[kProbWaves * prob_tile_bytes(DM == 64 ? 64 : 128)];
    __shared__ int sNext;               // tiles claimed so far by the workgroup's waves
    __shared__ int sPage[FLAT ? 1 : kPageCache];
    const int x = blockIdx.x;
    // workgroup -> (group, sequence, part): the groups' workgroups are consecutive ranges
    int gi = a.prob_g0;
    for (int g = a.prob_g0 + 1; g < a.prob_g0 + a.prob_ng; ++g)
        gi = x >= a.grp[g].wg0 ? g : gi;
    const ScoreGroup &G = a.grp[gi];
    const int r = x - G.wg0;
    const int b = r / G.parts;
    const int part = r - b * G.parts;
    prob_group<DM, FLAT>(a, G, b, part, sK, sNext, sPage);
}

// The softmax-mode kernel when the launch pairs the groups of two signals (head dims D1
// for the first half of the groups, D2 for the second, D1 != D2): workgroup -> (pair i,
// sequence, part), one share of group i of the first half, then the same share of group i
// of the second half (every group has the same parts), so every workgroup moves the same
// bytes.  A kernel of its own: with both paths in one kernel, the tile arrays of its four
// inlined copies ended up in scratch memory.
template <int D1, int D2, bool FLAT>
__global__ __launch_bounds__(64 * kProbWaves)
__attribute__((amdgpu_waves_per_eu(kProbWaves / 4))) void srh_prob_pair_kernel(ScoreArgs a)
{
    __shared__ __align__(16) uint8_t sK[kProbWaves * prob_tile_bytes(D1 > D2 ? D1 : D2)];
    __shared__ int sNext[2];
    __shared__ int sDone;
    __shared__ int sPage[FLAT ? 1 : kPageCache];
    const int x = blockIdx.x;
    const int half = a.prob_ng / 2;
    const ScoreGroup &G0 = a.grp[a.prob_g0];
    const int per = a.B * G0.parts;
    const int i = x / per;
    const int b = (x - i * per) / G0.parts;
    const int part = x - i * per - b * G0.parts;
    if constexpr (FLAT) {
        // a tile counter per group, both zeroed up front, and every wave's LDS area the same
        // for both head dims: a wave goes from its last tile of the first group straight
        // to the second, and the last one to finish the first group folds it meanwhile
        if (threadIdx.x == 0) {
            sNext[0] = sNext[1] = 0;
            sDone = 0;
        }
        __syncthreads();
        constexpr int kWave = prob_tile_bytes(D1 > D2 ? D1 : D2);
        prob_logits<D1, FLAT>(a, a.grp[a.prob_g0 + i], b, part, sK, sNext[0], sPage, false, kWave, &sDone);
        prob_logits<D2, FLAT>(a, a.grp[a.prob_g0 + half + i], b, part, sK, sNext[1], sPage, false, kWave);
    } else {
        prob_logits<D1, FLAT>(a, a.grp[a.prob_g0 + i], b, part, sK, sNext[0], sPage);
        __syncthreads();              // the LDS areas and the page cache are free again
        prob_logits<D2, FLAT>(a, a.grp[a.prob_g0 + half + i], b, part, sK, sNext[1], sPage);
    }
}

// ---- logit-sum mode: raw scaled logits on MFMA -------------------------------------
constexpr int kSumTile = 512;              // tokens per workgroup
constexpr int kPerWave = kSumTile / 4;
constexpr int kSub = kPerWave / 16;
constexpr int kBatch = 4;

template <int D, int PT>
__global__ __launch_bounds__(kThreads) void srh_logit_sum_kernel(ScoreArgs a, int sidx)
{
    constexpr int KS = D / 32;
    const int tile = blockIdx.x;
    const ScoreSig &S = a.sig[sidx];
    const ScoreGroup &G = a.grp[S.g0 + blockIdx.y];
    const int b = blockIdx.z;
    const int N = clampi(a.ctx_len[b], 0, S.ctx_clamp);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane >> 4;
    const int li = lane & 15;
    const int t0 = tile * kSumTile;
    if (t0 >= N)
        return;
    // pair p of the group = (query head p / nqe, query p % nqe); LOGIT_SUM2 maps the
    // second query slot to the last query
    const bool all_q = S.mode == DUSTIN_SCORE_LOGIT_SUM_ALL;
    const int nqe = all_q ? S.n_q : min(2, S.n_q);
    const float mul = (float)S.mul;

    // SRH queries as the MFMA B operand: lane holds pair pt*16 + li, its quarter of d
    u32x4 qop[PT][KS];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const int p = pt * 16 + li;
        if (p < G.n_pairs) {
            const int hl = p / nqe;
            const int jj = p - hl * nqe;
            const int j = all_q || jj == 0 ? jj : S.n_q - 1;
            const uint16_t *qp =
                S.q + ((int64_t)(b * S.total_qheads + G.q_head0 + hl) * S.n_q + j) * D + quad * (D / 4);
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
            // column li of the product is pair pt*16 + li (zero queries past n_pairs): the
            // group's sum over pairs is a sum over the 16 lanes of the lane's row
            float c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mfma_bf16(kop[u][ks], qop[pt][ks], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    c[r] += acc[r] * mul;
            }
            row16_reduce_f32<4, false>(c);
            if (li == 0 && tb < N) {
                float *dst = S.logits + ((int64_t)b * S.logit_rows + blockIdx.y) * a.n_pad + tb;
                if (tb + 3 < N) {
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{c[0], c[1], c[2], c[3]};
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

constexpr int kFinTokens = 1024;          // = kThreads * 4: every thread sums four tokens
constexpr int kFinTiles = kFinTokens / kStatTile;
constexpr int kFinBatch = 5;               // pairs per wave whose statistics loads are in flight together
constexpr int kFinChunk = 20;              // pairs whose logits one finalize thread holds at once (rows past a signal's last repeat it)

__global__ __launch_bounds__(kThreads) void srh_finalize_kernel(ScoreArgs a)
{
    static_assert(kFinTokens == 4 * kThreads, "one f32x4 of tokens per thread");
    __shared__ float sOff[kMaxGroups * kMaxProbPairsPerGroup][kFinTiles];
    __shared__ float sInvZ[kMaxGroups * kMaxProbPairsPerGroup];
    const ScoreSig &S = a.sig[blockIdx.z];
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int N = clampi(a.ctx_len[b], 0, S.ctx_clamp);
    const bool prob = S.mode == DUSTIN_SCORE_PROB_SUM;
    const int tile0 = blockIdx.x * kFinTiles;
    // this thread's 4 tokens: the statistics of the wave's first kFinBatch pairs are
    // requested first and the logits of the first kFinChunk pairs right behind them, all
    // as unconditional loads at clamped addresses (values outside the ranges are replaced
    // after the loads), so the statistics can be reduced while the logits are in flight
    const int P = prob ? S.total_pairs : S.n_groups;   // logit rows summed per token
    const int tb = blockIdx.x * kFinTokens + tid * 4;
    const bool live = tb < N;
    const float *lg = S.logits + (int64_t)b * S.logit_rows * a.n_pad + (live ? tb : 0);
    const int p_last = max(P - 1, 0);
    f32x4 lv[kFinChunk];
    auto fetch = [&](int p0) {
#pragma unroll
        for (int j = 0; j < kFinChunk; ++j)
            lv[j] = *reinterpret_cast<const f32x4 *>(lg + (int64_t)min(p0 + j, p_last) * a.n_pad);
    };
    if (prob) {
        // one wave per pair, kFinBatch pairs at a time: lanes take the workgroup partials
        // (at most kScoreParts) for the pair's max (fp64) and normaliser (fp32 exp2 of the
        // fp64 difference, summed in fp64), and lanes below kFinTiles the maxima of this
        // block's statistics tiles
        const int w = tid >> 6, lane = tid & 63;
        const int tc = min(tile0 + min(lane, kFinTiles - 1), a.n_tiles - 1);   // lanes past the block's tiles repeat its last
        const int pi = min(lane, max(a.n_parts, 1) - 1);
        const int row_last = max(S.total_pairs - 1, 0);
        double pm[kFinBatch], ps[kFinBatch], tm[kFinBatch];
        auto load_stats = [&](int p0) {
            // every slot of the pair's record (slots past its group's workgroups hold the
            // empty partial)
#pragma unroll
            for (int k = 0; k < kFinBatch; ++k) {
                const int64_t row = (int64_t)b * S.total_pairs + min(p0 + 4 * k, row_last);
                pm[k] = S.part_max[row * a.n_parts + pi];
                ps[k] = S.part_sum[row * a.n_parts + pi];
                tm[k] = S.tile_max[row * a.n_tiles + tc];
            }
        };
        auto reduce_stats = [&](int p0) {
            // the batch's pairs in three branch-free passes (their reduction chains
            // interleave), then the stores
            double M[kFinBatch], Z[kFinBatch];
#pragma unroll
            for (int k = 0; k < kFinBatch; ++k) {
                const bool ok = p0 + 4 * k < S.total_pairs && lane < a.n_parts;
                pm[k] = ok ? pm[k] : -INFINITY;
                ps[k] = ok ? ps[k] : 0.0;
                M[k] = wave_max_f64_dpp(pm[k]);
            }
#pragma unroll
            for (int k = 0; k < kFinBatch; ++k)
                Z[k] = wave_sum_f64_dpp(ps[k] > 0.0 ? ps[k] * (double)fast_exp2((float)(pm[k] - M[k])) : 0.0);
            float iz[kFinBatch], off[kFinBatch];
#pragma unroll
            for (int k = 0; k < kFinBatch; ++k) {
                const bool tok = lane < kFinTiles && tile0 + lane < a.n_tiles && tm[k] > -INFINITY;
                iz[k] = Z[k] > 0.0 ? (float)(1.0 / Z[k]) : 0.f;
                off[k] = tok ? (float)(tm[k] - M[k]) : 0.f;
            }
#pragma unroll
            for (int k = 0; k < kFinBatch; ++k) {
                const int p = p0 + 4 * k;
                if (p < S.total_pairs) {
                    if (lane == 0)
                        sInvZ[p] = iz[k];
                    if (lane < kFinTiles)
                        sOff[p][lane] = off[k];
                }
            }
        };
        // the first batch with the logits requested right behind its statistics (no branch
        // between them, so the wait for the statistics leaves the logits in flight)
        load_stats(w);
        fetch(0);
        __builtin_amdgcn_sched_barrier(0);   // every load issued before the first wait
        reduce_stats(w);
        for (int p0 = w + 4 * kFinBatch; p0 < S.total_pairs; p0 += 4 * kFinBatch) {
            load_stats(p0);
            reduce_stats(p0);
        }
        __syncthreads();
    } else {
        fetch(0);
    }
    if (tb >= a.n_max)
        return;
    const int tl = (tid * 4) / kStatTile;   // statistics tile of these 4 tokens within the block
    f32x4 v{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < P; p0 += kFinChunk) {
        if (p0 > 0)
            fetch(p0);
#pragma unroll
        for (int j = 0; j < kFinChunk; ++j) {
            const int p = p0 + j;
            if (p < P) {
                if (prob) {
                    const float c = sOff[p][tl], iz = sInvZ[p];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] += fast_exp2(lv[j][r] + c) * iz;
                } else {
                    v += lv[j];
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (tb + r >= N)
            v[r] = 0.f;
    float *dst = S.score + (int64_t)b * a.n_max + tb;
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
hipError_t launch_logit_sum(const ScoreArgs &a, int sidx, int pt, dim3 grid, hipStream_t st)
{
    switch (pt) {
    case 1: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 1>), grid, dim3(kThreads), 0, st, a, sidx); break;
    case 2: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 2>), grid, dim3(kThreads), 0, st, a, sidx); break;
    case 3: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 3>), grid, dim3(kThreads), 0, st, a, sidx); break;
    default: hipLaunchKernelGGL((srh_logit_sum_kernel<D, 4>), grid, dim3(kThreads), 0, st, a, sidx); break;
    }
    return hipGetLastError();
}

// The softmax-mode kernel over the softmax-mode signals' groups (grp[a.prob_g0 ..
// + n_groups)).  Its grid is one resident round: as many workgroups per CU as the
// variant's registers and LDS allow (asked of the runtime once per variant), each taking
// an equal share of its stream's tiles.  a.n_parts comes in as the workspace's maximum and
// leaves as the count launched (the finalize reads that many).
template <int DM, bool FLAT>
hipError_t launch_prob_variant(ScoreArgs &a, int cus, hipStream_t st)
{
    constexpr int nt = 64 * kProbWaves;
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, srh_prob_logits_kernel<DM, FLAT>, nt, 0) !=
                hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    // one resident round of workgroups, shared among the groups in proportion to their
    // bytes per token (the head dim), at least one and at most the workspace's count each
    const int slots = std::max(1, per_cu * cus / std::max(1, a.B));
    // Two signals with the same number of groups and different head dims (the draft's and
    // the target's): whole parts per group cannot match bytes per workgroup (64 against
    // 128 would need 2.67 and 5.33 shares of 32), so every workgroup takes the same share
    // of one group of each, and every workgroup moves the same bytes.
    if (DM == 0 && a.prob_ng % 2 == 0) {
        const int half = a.prob_ng / 2;
        const int parts = std::min(a.n_parts, slots / half);
        bool ok = parts >= 1;
        for (int i = 0; i < half && ok; ++i) {
            const ScoreGroup &A = a.grp[a.prob_g0 + i], &Bg = a.grp[a.prob_g0 + half + i];
            ok = a.sig[A.sig].head_dim == a.sig[a.grp[a.prob_g0].sig].head_dim &&
                 a.sig[Bg.sig].head_dim == a.sig[a.grp[a.prob_g0 + half].sig].head_dim &&
                 a.sig[A.sig].head_dim != a.sig[Bg.sig].head_dim;
        }
        if (ok) {
            int wg = 0;
            for (int g = a.prob_g0; g < a.prob_g0 + a.prob_ng; ++g) {
                a.grp[g].parts = parts;
                a.grp[g].wg0 = g < a.prob_g0 + half ? wg : a.grp[g - half].wg0;
                if (g < a.prob_g0 + half)
                    wg += parts * a.B;
            }
            a.n_parts = parts;
            if (a.sig[a.grp[a.prob_g0].sig].head_dim == 64)
                hipLaunchKernelGGL((srh_prob_pair_kernel<64, 128, FLAT>), dim3((unsigned)wg), dim3(nt), 0, st, a);
            else
                hipLaunchKernelGGL((srh_prob_pair_kernel<128, 64, FLAT>), dim3((unsigned)wg), dim3(nt), 0, st, a);
            return hipGetLastError();
        }
    }
    int dsum = 0;
    for (int g = a.prob_g0; g < a.prob_g0 + a.prob_ng; ++g)
        dsum += a.sig[a.grp[g].sig].head_dim;
    int wg = 0, pmax = 1;
    for (int g = a.prob_g0; g < a.prob_g0 + a.prob_ng; ++g) {
        ScoreGroup &G = a.grp[g];
        const int d = a.sig[G.sig].head_dim;
        G.parts = std::max(1, std::min(a.n_parts, (slots * d + dsum / 2) / dsum));
        G.wg0 = wg;
        wg += G.parts * a.B;
        pmax = std::max(pmax, G.parts);
    }
    a.n_parts = pmax;
    hipLaunchKernelGGL((srh_prob_logits_kernel<DM, FLAT>), dim3((unsigned)wg), dim3(nt), 0, st, a);
    return hipGetLastError();
}

template <int DM>
hipError_t launch_prob(ScoreArgs &a, bool flat, int cus, hipStream_t st)
{
    return flat ? launch_prob_variant<DM, true>(a, cus, st) : launch_prob_variant<DM, false>(a, cus, st);
}

}  // namespace

// Softmax-mode signals share one logit launch (their groups are contiguous: signals are
// stored in order); each logit-sum signal has its own; one finalize launch serves every
// signal (grid z = signal).
hipError_t launch_score(ScoreArgs a, int cus, hipStream_t st)
{
    hipError_t e = hipSuccess;
    int pg0 = -1, png = 0, dims = 0;
    bool flat = true;
    for (int s = 0; s < a.n_sig; ++s) {
        const ScoreSig &S = a.sig[s];
        if (S.mode != DUSTIN_SCORE_PROB_SUM)
            continue;
        if (pg0 < 0)
            pg0 = S.g0;
        png += S.n_groups;
        dims |= S.head_dim == 64 ? 1 : 2;
        for (int g = S.g0; g < S.g0 + S.n_groups; ++g)
            flat = flat && !a.grp[g].k.pt && a.grp[g].k.st >= 0 && a.grp[g].k.st * 2 < (int64_t)1 << 32;
    }
    if (png > 0) {
        a.prob_g0 = pg0;
        a.prob_ng = png;
        e = dims == 1 ? launch_prob<64>(a, flat, cus, st)
                      : (dims == 2 ? launch_prob<128>(a, flat, cus, st) : launch_prob<0>(a, flat, cus, st));
        if (e != hipSuccess)
            return e;
    }
    for (int s = 0; s < a.n_sig; ++s) {
        const ScoreSig &S = a.sig[s];
        if (S.mode == DUSTIN_SCORE_PROB_SUM)
            continue;
        int max_pairs = 1;
        for (int g = S.g0; g < S.g0 + S.n_groups; ++g)
            max_pairs = std::max(max_pairs, a.grp[g].n_pairs);
        const dim3 g1((unsigned)((a.n_max + kSumTile - 1) / kSumTile), (unsigned)S.n_groups, (unsigned)a.B);
        const int pt = (max_pairs + 15) / 16;
        e = S.head_dim == 64 ? launch_logit_sum<64>(a, s, pt, g1, st) : launch_logit_sum<128>(a, s, pt, g1, st);
        if (e != hipSuccess)
            return e;
    }
    const dim3 g2((unsigned)((a.n_max + kFinTokens - 1) / kFinTokens), (unsigned)a.B, (unsigned)a.n_sig);
    hipLaunchKernelGGL(srh_finalize_kernel, g2, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dustin
