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
//   workgroup = (b, g, query group, split of the selected positions).  The split's
//   positions (at most 2048) are resolved once into an LDS table of 64-bit row offsets
//   (page tables are looked up there), then each wave streams its own 32-position steps
//   (steps w, w+4, ...) with no workgroup barrier inside the loop:
//     - a step's K and V rows are moved into one of the wave's two LDS ring slots by LDS
//       DMA (non-temporal; every 64-lane instruction moves whole rows), with 16-byte
//       chunks XOR-swizzled per row so that the operand reads are bank-conflict free; a
//       slot is refilled as soon as its operands are in registers;
//     - S^T = K Q^T is formed for all (up to QT*16) queries of the KV head's group on
//       v_mfma_f32_16x16x32_bf16 (fp32 accumulate); the S^T output layout of a lane is
//       exactly the B operand of the PV product, so P never leaves registers;
//     - V^T comes from transposing LDS reads (ds_read_b64_tr_b16) and O^T += V^T P^T is
//       accumulated on 16x16x32 over the whole head dim; the online softmax is in base 2
//       with a lazy rescale;
//     - the new-token block (at most 16 rows, causal among themselves) is one 16-row
//       step of wave 3 of the last split, loaded first into its own LDS area.
//   The four waves merge their (max, sum, O) in one LDS exchange at the end; splits of
//   one pair are merged by a second kernel with log-sum-exp weights in fixed split order
//   (a kernel boundary, not per-workgroup device-scope fences, which write back and
//   invalidate the XCD's L2).  Block ids are mapped so that all splits of one pair run
//   on one XCD (blocks are dispatched round-robin over the 8 XCDs).
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;          // list positions per wave step
constexpr int kNewWave = 3;        // wave of the last split that takes the new-token step (it
                                   // has the fewest ring steps)
constexpr float kLazy = 8.f;       // rescale O only when a tile's max exceeds the reference by 2^8

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// max over the four lanes l, l^16, l^32, l^48 (v_permlane32_swap / v_permlane16_swap)
__device__ __forceinline__ float max_over_quads(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS transposing read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i receives
// 16-bit element i % 4 of the 8-byte words addressed by lanes i / 4, 4 + i / 4, 8 + i / 4
// and 12 + i / 4 of its group, in that order.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t *p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Geometry of one wave step for head dim D.  A step covers kTile list positions; its K
// rows and V rows are each moved into LDS by NI DMA instructions of 64 lanes x 16 bytes,
// instruction n covering LDS rows n*RPI .. n*RPI + RPI - 1 with whole rows per lane group
// (fully coalesced reads).  LDS row rho holds list row tau(rho) = (rho % RPI) * NI +
// rho / RPI of the step, so the NI rows one lane moves are consecutive list positions.
// Chunks (16 bytes) of a row are stored XOR-swizzled: K chunk c of row rho sits at
// c ^ (rho % CPR), V chunk c at c ^ (2 rho % CPR), which makes the MFMA operand reads
// (K: 16 rows x one chunk; V transposed: 8 rows x two chunks per half-wave) bank-conflict free.
template <int D>
struct Geo {
    static constexpr int RB = 2 * D;            // bytes of one row of one head
    static constexpr int CPR = RB / 16;         // 16-byte chunks per row
    static constexpr int RPI = 1024 / RB;       // rows per DMA instruction
    static constexpr int NI = kTile / RPI;      // DMA instructions per tensor per step
    static constexpr int KS = D / 32;           // k-steps of QK^T (16x16x32)
    static constexpr int DVT = D / 16;          // 16-wide head-dim tiles of PV
    static constexpr int HALF = kTile * RB;     // bytes of the K (or V) rows of a step
    static constexpr int SLOT = 2 * HALF;
    __device__ static constexpr int tau(int rho) { return (rho % RPI) * NI + rho / RPI; }
};

template <int D, int QT, int R>
struct AttnShape {
    using G = Geo<D>;
    static constexpr int QR = QT * 16;          // padded query rows
    static constexpr int ACC = G::DVT * QT * 4; // O accumulator floats per lane
    static constexpr int TAB = (kSplitMax + 32) * 8;   // + the new-token rows' K and V offsets
    static constexpr int RING = 4 * R * G::SLOT;
    // The four waves' accumulators are exchanged in one pass, or in two (half of the
    // head-dim tiles each) where one pass would not fit the LDS (five query tiles at head
    // dim 128).
    static constexpr int MRG1 = 4 * 64 * ACC * 4 + 2 * 4 * QR * 4;
    static constexpr int PH = TAB + (RING > MRG1 ? RING : MRG1) + 2 * 16 * G::RB > 160 * 1024 ? 2 : 1;
    static constexpr int MRG = 4 * 64 * (ACC / PH) * 4 + 2 * 4 * QR * 4;
    static constexpr int NEW = TAB + (RING > MRG ? RING : MRG);   // new-token rows: 16 K, 16 V
    static constexpr int LDS = NEW + 2 * 16 * G::RB;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D, int QT, int R>
__global__ __launch_bounds__(kThreads) void verify_attn_split_kernel(AttnArgs a)
{
    using S = AttnShape<D, QT, R>;
    using G = Geo<D>;
    __shared__ __align__(16) uint8_t lds[S::LDS];
    int64_t *sOffK = reinterpret_cast<int64_t *>(lds);
    int64_t *sOffV = a.kv_same ? sOffK : sOffK + kSplitMax / 2;

    // ---- block -> (sequence, KV head, query group, split).  Every workgroup of one
    //      (sequence, KV head) has the same blockIdx % 8, i.e. runs on the same XCD, and
    //      the query groups of one split are dispatched back to back, so the groups
    //      re-reading a split's rows find them in that XCD's L2 ----
    const int x = blockIdx.x;
    const int hi = x >> 3;
    const int qg = hi % a.qgroups;
    const int t2 = hi / a.qgroups;
    const int split = t2 % a.splits;
    const int bg = (t2 / a.splits) * 8 + (x & 7);
    if (bg >= a.B * a.Hkv)
        return;
    const int pair = bg * a.qgroups + qg;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane >> 4;   // MFMA lane group
    const int li = lane & 15;
    const int p0 = split * a.spl;

    // ---- one round trip: the split's index entries, the sequence's length and count,
    //      and Q; none of these loads depends on another ----
    constexpr int PT = (kSplitMax + kThreads - 1) / kThreads;
    int raw[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        const int i = tid + k * kThreads;
        const int pos = p0 + i;
        raw[k] = (a.idx && i < a.spl && pos < a.k_max) ? a.idx[(int64_t)b * a.k_max + pos] : 0;
    }
    const int n_raw = a.ctx_len[b];
    const int c_raw = a.idx ? a.count[b] : 0;

    // Q as the B operand of S^T = K Q^T: lane holds q-row qt*16 + li, head-dim elements
    // ks*32 + quad*8 .. +8 for k-step ks.  A negative scale is moved into Q (exact sign
    // flip), so the kernel only ever multiplies logits by c = |scale| log2(e) >= 0.  Q is
    // loaded after the first K/V step has been requested (it is needed only by the math).
    const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
    const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    u32x4 qop[QT][G::KS];
    int qrow_t[QT];   // verify index t of the lane's query row (large for padding rows)
    const uint16_t *qptr[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int row = qg * S::QR + qt * 16 + li;
        qrow_t[qt] = 1 << 20;
        qptr[qt] = nullptr;
        if (row < a.GV) {
            const int t = row / a.G;
            const int h = g * a.G + (row - t * a.G);
            qptr[qt] = a.q + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + quad * 8;
            qrow_t[qt] = t;
        }
    }
    auto load_q = [&]() {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks)
                qop[qt][ks] = qptr[qt] ? (load16(qptr[qt] + ks * 32) ^ qsign) : u32x4{0, 0, 0, 0};
    };

    // ---- sequence geometry; every device value is clamped ----
    const int N = clampi(n_raw, 0, a.ctx_clamp);
    const int nsel = a.idx ? clampi(c_raw, 0, min(a.k_max, N)) : N;
    // split ranges cover the selected positions; the new-token block (nv <= 16 rows,
    // list positions nsel .. nsel+nv-1) is a separate 16-row step of one wave of the last
    // split, loaded at the start into its own LDS area so that no wave's ring carries an
    // extra step
    const int p1 = min(p0 + a.spl, nsel);
    const int cnt = max(p1 - p0, 0);
    const int ntile = (cnt + kTile - 1) / kTile;
    const bool new_here = split == a.splits - 1 && w == kNewWave;

    // ---- row offsets of the split's positions; the padding of the last step points at
    //      token N (the first new token, always present), whose scores are masked.  Paged
    //      caches: every entry's page is fetched before any is used (one round trip) ----
    int tokv[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        const int i = tid + k * kThreads;
        const int pos = p0 + i;
        int tok = N;
        if (i < cnt)
            tok = a.idx ? clampi(raw[k], 0, N - 1) : pos;
        tokv[k] = tok;
    }
    int pgK[PT], pgV[PT];
    if (a.k.pt) {
#pragma unroll
        for (int k = 0; k < PT; ++k)
            pgK[k] = a.k.pt[(int64_t)b * a.k.max_pages + (tokv[k] >> a.k.ps_log2)];
    }
    if (a.v.pt && !a.kv_same) {
#pragma unroll
        for (int k = 0; k < PT; ++k)
            pgV[k] = a.v.pt[(int64_t)b * a.v.max_pages + (tokv[k] >> a.v.ps_log2)];
    }
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        const int i = tid + k * kThreads;
        if (i < ntile * kTile) {
            const int tok = tokv[k];
            sOffK[i] = a.k.pt ? (int64_t)clampi(pgK[k], 0, a.k.num_pages - 1) * a.k.sp +
                                    (int64_t)(tok & ((1 << a.k.ps_log2) - 1)) * a.k.st
                              : (int64_t)b * a.k.sb + (int64_t)tok * a.k.st;
            if (!a.kv_same)
                sOffV[i] = a.v.pt ? (int64_t)clampi(pgV[k], 0, a.v.num_pages - 1) * a.v.sp +
                                        (int64_t)(tok & ((1 << a.v.ps_log2) - 1)) * a.v.st
                                  : (int64_t)b * a.v.sb + (int64_t)tok * a.v.st;
        }
    }
    // the new-token rows' offsets (last split): entry e of 16 is LDS row (e % n') * RPI +
    // e / n' of the new-token area (n' = NI/2 DMA instructions), i.e. new token min(row,
    // nv-1); K entries first, then V
    if (split == a.splits - 1 && tid < 32) {
        constexpr int NH = G::NI / 2;
        const int e = tid & 15;
        const int tok = N + min((e % NH) * G::RPI + e / NH, a.nv - 1);
        sOffK[kSplitMax + tid] = tid < 16 ? kv_offset(a.k, b, tok, 0) : kv_offset(a.v, b, tok, 0);
    }
    __syncthreads();                  // offset tables ready

    f32x4 acc[G::DVT][QT];
#pragma unroll
    for (int i = 0; i < G::DVT; ++i)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            acc[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref[QT], lrun[QT];         // reference max (scaled log2 units) and running sum
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        mref[qt] = -INFINITY;
        lrun[qt] = 0.f;
    }

    const int mine = ntile > w ? (ntile - w + 3) >> 2 : 0;    // steps w, w+4, ... of this wave
    uint8_t *wring = lds + S::TAB + w * R * G::SLOT;          // this wave's ring of step slots
    const uint16_t *kbase = a.k.base + (int64_t)g * a.k.sh;
    const uint16_t *vbase = a.v.base + (int64_t)g * a.v.sh;
    const int dg = lane / G::CPR;     // DMA: row group of the lane within an instruction
    const int dc = lane % G::CPR;     // DMA: LDS chunk of the lane within its row

    // ni instructions each of K and V rows into dst (V at dst + voff): the lane moves table
    // entries tk[dg*ni + n] / tv[dg*ni + n] (n < ni) to LDS rows n*RPI + dg.  Loads are
    // non-temporal: every row is read once.
    auto dma_to = [&](const int64_t *tk, const int64_t *tv, uint8_t *dst, int voff, int ni) {
#pragma unroll
        for (int n = 0; n < G::NI; ++n) {
            if (n < ni) {
                const int rho = n * G::RPI + dg;
                const int ck = dc ^ (rho % G::CPR);
                __builtin_amdgcn_global_load_lds(kbase + tk[dg * ni + n] + ck * 8, (lds_void *)(dst + n * 1024), 16, 0,
                                                 kLoadNonTemporal);
            }
        }
#pragma unroll
        for (int n = 0; n < G::NI; ++n) {
            if (n < ni) {
                const int rho = n * G::RPI + dg;
                const int cv = dc ^ ((2 * rho) % G::CPR);
                __builtin_amdgcn_global_load_lds(vbase + tv[dg * ni + n] + cv * 8, (lds_void *)(dst + voff + n * 1024),
                                                 16, 0, kLoadNonTemporal);
            }
        }
    };
    // Step jj of this wave into ring slot jj % R (table entries of the step's 32 positions).
    auto dma = [&](int jj) {
        const int e0 = (w + 4 * jj) * kTile;
        dma_to(sOffK + e0, sOffV + e0, wring + (jj % R) * G::SLOT, G::HALF, G::NI);
    };

    // per-lane LDS byte offsets of the operand reads (slot-relative)
    int koff[2][G::KS];               // K: row 16h + li, chunk ks*4 + quad
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const int rho = 16 * h + li;
            koff[h][ks] = rho * G::RB + (((ks * 4 + quad) ^ (rho % G::CPR)) << 4);
        }
    // V^T: source lane s = li of group quad reads row 16h + 4*quad + s/4, head-dim
    // columns dt*16 + 4*(s%4) .. +3, i.e. chunk 2*dt + (s%4)/2, byte 8*(s%2) of it
    int vrow[2], vf2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rho = 16 * h + 4 * quad + (li >> 2);
        vrow[h] = G::HALF + rho * G::RB + (((li >> 1) & 1) << 4) + ((li & 1) << 3);
        vf2[h] = rho % (G::CPR / 2);
    }
    // list row of the lane's S^T entries (h, r): LDS row 16h + 4*quad + r
    int trow[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            trow[h][r] = G::tau(16 * h + 4 * quad + r);

    // The softmax and O^T update of one step, given its K and V^T operands.  S^T entry
    // (h, r) is LDS row 16h + 4*quad + r of the step; its list position is pos0 +
    // tau(row) for ring steps and pos0 + row for the new-token step (direct).  Entries at
    // list positions >= pend, and new tokens after the query row's own, are masked.
    auto math = [&](const u32x4 (&kop)[2][G::KS], const u32x4 (&vop)[G::DVT], bool full, int pos0,
                    bool direct, int pend) {
        // S^T = K Q^T for both 16-row halves of the step
        f32x4 s[2][QT];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                s[h][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks)
                    s[h][qt] = mfma_bf16(kop[h][ks], qop[qt][ks], s[h][qt]);
            }

        u32x4 pb[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            if (!full) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int pos = pos0 + (direct ? 16 * h + 4 * quad + r : trow[h][r]);
                        const bool ok = (pos < pend) & ((pos < nsel) | (pos - nsel <= qrow_t[qt]));
                        s[h][qt][r] = ok ? s[h][qt][r] : -INFINITY;
                    }
            }
            float mx = fmaxf(fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), fmaxf(s[0][qt][2], s[0][qt][3])),
                             fmaxf(fmaxf(s[1][qt][0], s[1][qt][1]), fmaxf(s[1][qt][2], s[1][qt][3])));
            mx = max_over_quads(mx) * c;
            if (__any(mx > mref[qt] + kLazy)) {
                const float mnew = fmaxf(mref[qt], mx);
                const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref[qt] - mnew);
                mref[qt] = mnew;
                lrun[qt] *= alpha;
#pragma unroll
                for (int i = 0; i < G::DVT; ++i)
                    acc[i][qt] *= alpha;
            }
            const float nm = mref[qt] == -INFINITY ? 0.f : -mref[qt];
            float p[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p[h][r] = fast_exp2(fmaf(s[h][qt][r], c, nm));
            lrun[qt] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
            pb[qt] = u32x4{cvt_pk_bf16(p[0][0], p[0][1]), cvt_pk_bf16(p[0][2], p[0][3]),
                           cvt_pk_bf16(p[1][0], p[1][1]), cvt_pk_bf16(p[1][2], p[1][3])};
        }
        // O^T += V^T P^T over the 32 positions (16x16x32: k-slot (quad, 4h + r) is LDS
        // row 16h + 4*quad + r in both operands)
#pragma unroll
        for (int dt = 0; dt < G::DVT; ++dt)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                acc[dt][qt] = mfma_bf16(vop[dt], pb[qt], acc[dt][qt]);
    };

    // The new-token rows, requested first: LDS row rho (< 16) holds new token min(rho,
    // nv-1) in the swizzled layout of a step's first half; the V rows follow the K rows.
    uint8_t *nslot = lds + S::NEW;
    if (new_here)
        dma_to(sOffK + kSplitMax, sOffK + kSplitMax + 16, nslot, 16 * G::RB, G::NI / 2);

    // All R slots are in flight while a step computes: a slot is refilled as soon as its K
    // and V operands have been read into registers, before the step's math.
    if (mine > 0)
        dma(0);
    load_q();
    if (mine > 0) {
#pragma unroll
        for (int jj = 1; jj < R; ++jj)
            if (jj < mine)
                dma(jj);
        for (int jj = 0; jj < mine; ++jj) {
            if (jj + R - 1 < mine)
                wait_vmcnt<2 * G::NI * (R - 1)>();   // step jj has landed, R-1 later steps in flight
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_sched_barrier(0);
            const uint8_t *slot = wring + (jj % R) * G::SLOT;
            const int pos0 = p0 + (w + 4 * jj) * kTile;

            u32x4 kop[2][G::KS];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks)
                    kop[h][ks] = *reinterpret_cast<const u32x4 *>(slot + koff[h][ks]);
            // V^T operands (16-bit transposing reads)
            u32x4 vop[G::DVT];
#pragma unroll
            for (int dt = 0; dt < G::DVT; ++dt) {
                const u32x2 v0 = lds_read_tr16(slot + vrow[0] + ((dt ^ vf2[0]) << 5));
                const u32x2 v1 = lds_read_tr16(slot + vrow[1] + ((dt ^ vf2[1]) << 5));
                vop[dt] = u32x4{v0[0], v0[1], v1[0], v1[1]};
            }
            if (jj + R < mine) {
                wait_lgkm0();                        // the slot's reads are done
                __builtin_amdgcn_sched_barrier(0);
                dma(jj + R);
            }
            math(kop, vop, pos0 + kTile <= p1, pos0, false, p1);
        }
    }
    if (new_here) {
        // the new-token step: rows 16..31 have zero operands and are masked
        wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        u32x4 kop[2][G::KS];
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            kop[0][ks] = *reinterpret_cast<const u32x4 *>(nslot + koff[0][ks]);
            kop[1][ks] = u32x4{0, 0, 0, 0};
        }
        u32x4 vop[G::DVT];
#pragma unroll
        for (int dt = 0; dt < G::DVT; ++dt) {
            const u32x2 v0 = lds_read_tr16(nslot + vrow[0] - G::HALF + 16 * G::RB + ((dt ^ vf2[0]) << 5));
            vop[dt] = u32x4{v0[0], v0[1], 0, 0};
        }
        math(kop, vop, false, nsel, true, nsel + a.nv);
    }

    // ---- merge the four waves through LDS: every wave publishes its maxima, sums and
    //      O^T accumulators (all head-dim tiles, or half of them per phase), then wave w
    //      merges a quarter of the published tiles of every row and writes them ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        lrun[qt] += __shfl_xor(lrun[qt], 16);
        lrun[qt] += __shfl_xor(lrun[qt], 32);
    }
    constexpr int DVTP = G::DVT / S::PH;   // head-dim tiles exchanged per phase
    constexpr int DPW = DVTP / 4;          // head-dim tiles merged by each wave per phase
    float *xAcc = reinterpret_cast<float *>(lds + S::TAB);   // [wave][dv tile of the phase][qt][lane][4]
    float *xM = xAcc + 4 * 64 * (S::ACC / S::PH);             // [wave][QR]
    float *xL = xM + 4 * S::QR;
    __syncthreads();                  // every wave is done with its ring
    if (quad == 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            xM[w * S::QR + qt * 16 + li] = mref[qt];
            xL[w * S::QR + qt * 16 + li] = lrun[qt];
        }
    }
    const int64_t pstride = (int64_t)S::QR * D + 2 * S::QR;
    float *part = a.part + ((int64_t)pair * a.splits + split) * pstride;
#pragma unroll
    for (int ph = 0; ph < S::PH; ++ph) {
        if (ph > 0)
            __syncthreads();          // the previous phase's tiles have been read
#pragma unroll
        for (int i = 0; i < DVTP; ++i)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                *reinterpret_cast<f32x4 *>(xAcc + (((w * DVTP + i) * QT + qt) * 64 + lane) * 4) = acc[ph * DVTP + i][qt];
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int q = qt * 16 + li;
            const int row = qg * S::QR + q;
            if (row >= a.GV)
                continue;             // padding rows are never written
            float mw[4], M = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                mw[v] = xM[v * S::QR + q];
                M = fmaxf(M, mw[v]);
            }
            float f[4], l = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                f[v] = M == -INFINITY ? 0.f : fast_exp2(mw[v] - M);
                l += f[v] * xL[v * S::QR + q];
            }
            const int t = row / a.G;
            const int h = g * a.G + (row - t * a.G);
            const float inv = 1.f / l;
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                const int i = w * DPW + j;
                f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    o += f[v] * *reinterpret_cast<const f32x4 *>(xAcc + (((v * DVTP + i) * QT + qt) * 64 + lane) * 4);
                const int dv = (ph * DVTP + i) * 16 + 4 * quad;
                if (a.splits == 1) {
                    uint16_t *op = a.out + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + dv;
                    *reinterpret_cast<u32x2 *>(op) =
                        u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
                } else {
                    *reinterpret_cast<f32x4 *>(part + (int64_t)q * D + dv) = o;
                }
            }
            if (ph == 0 && w == 0 && quad == 0) {
                if (a.splits == 1) {
                    a.lse[((int64_t)b * a.Hq + h) * a.nv + t] = (M + __log2f(l)) * kLn2;
                } else {
                    part[S::QR * D + q] = M;
                    part[S::QR * D + S::QR + q] = l;
                }
            }
        }
    }
}

// Merges the split partials of one (pair, query tile) in fixed split order:
// O = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s, LSE = M + log sum_s e^{m_s - M} l_s.
// Every (row, 4-column) item is one thread (D/64 blocks per 16-row tile); the per-split
// maxima and sums of a row are read by all of its threads (cache hits), so there is a
// single round of loads.
template <int D, int QT, int kPre>   // kPre: splits whose partials are fetched before any math
__global__ __launch_bounds__(kThreads) void verify_attn_merge_kernel(AttnArgs a)
{
    constexpr int QR = QT * 16;
    constexpr int BPQ = D / 64;       // blocks per 16-row query tile
    // blocks of a pair run on the XCD that ran its split workgroups (blockIdx % 8)
    const int x = blockIdx.x;
    const int hi = x >> 3;
    const int k = hi % (QT * BPQ);
    const int t2 = hi / (QT * BPQ);
    const int qg = t2 % a.qgroups;
    const int bg = (t2 / a.qgroups) * 8 + (x & 7);
    if (bg >= a.B * a.Hkv)
        return;
    const int pair = bg * a.qgroups + qg;
    const int qt = k / BPQ;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;
    const int item = (k - qt * BPQ) * kThreads + threadIdx.x;
    const int r = item / (D / 4);
    const int dv = (item - r * (D / 4)) * 4;
    const int row = qg * QR + qt * 16 + r;
    if (row >= a.GV)
        return;
    const int q = qt * 16 + r;
    const int64_t pstride = (int64_t)QR * D + 2 * QR;
    const float *base = a.part + (int64_t)pair * a.splits * pstride;
    // the first kPre splits' partials are loaded unconditionally (split index clamped, the
    // copies weighted 0), so all their loads are in flight together
    float ms[kPre], ls[kPre];
    f32x4 as[kPre];
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) {
        const float *ps = base + min(sp, a.splits - 1) * pstride;
        ms[sp] = ps[QR * D + q];
        ls[sp] = ps[QR * D + QR + q];
        as[sp] = *reinterpret_cast<const f32x4 *>(ps + (int64_t)q * D + dv);
    }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp)
        M = fmaxf(M, sp < a.splits ? ms[sp] : -INFINITY);
    for (int sp = kPre; sp < a.splits; ++sp)
        M = fmaxf(M, base[sp * pstride + QR * D + q]);
    f32x4 num{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) {
        const float wgt = (sp < a.splits && M != -INFINITY) ? fast_exp2(ms[sp] - M) : 0.f;
        num += wgt * as[sp];
        den += wgt * ls[sp];
    }
    for (int sp = kPre; sp < a.splits; ++sp) {
        const float *ps = base + sp * pstride;
        const float wgt = M == -INFINITY ? 0.f : fast_exp2(ps[QR * D + q] - M);
        num += wgt * *reinterpret_cast<const f32x4 *>(ps + (int64_t)q * D + dv);
        den += wgt * ps[QR * D + QR + q];
    }
    const float inv = 1.f / den;
    const int t = row / a.G;
    const int h = g * a.G + (row - t * a.G);
    uint16_t *o = a.out + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + dv;
    *reinterpret_cast<u32x2 *>(o) =
        u32x2{pack_bf16x2(num[0] * inv, num[1] * inv), pack_bf16x2(num[2] * inv, num[3] * inv)};
    if (dv == 0)
        a.lse[((int64_t)b * a.Hq + h) * a.nv + t] = (M + __log2f(den)) * kLn2;
}

template <int D, int QT, int R>
hipError_t launch_qt(const AttnArgs &a, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL((verify_attn_split_kernel<D, QT, R>), grid, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1)
        return e;
    const dim3 mgrid((unsigned)((a.B * a.Hkv + 7) / 8 * 8 * a.qgroups * QT * (D / 64)));
    if (a.splits <= 4)
        hipLaunchKernelGGL((verify_attn_merge_kernel<D, QT, 4>), mgrid, dim3(kThreads), 0, st, a);
    else if (a.splits <= 8)
        hipLaunchKernelGGL((verify_attn_merge_kernel<D, QT, 8>), mgrid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((verify_attn_merge_kernel<D, QT, 16>), mgrid, dim3(kThreads), 0, st, a);
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
    if constexpr (D == 64)
        return ring >= 3 ? launch_r<D, 3>(a, qt, grid, st) : launch_r<D, 2>(a, qt, grid, st);
    else
        return launch_r<D, 2>(a, qt, grid, st);   // two 16 KB slots per wave fill the LDS
}

}  // namespace

AttnPlan plan_attn(int B, int Hkv, int G, int nv, int max_list, int target_wgs, int split_cap)
{
    AttnPlan p;
    const int gv = G * nv;
    const int qt_total = (gv + 15) / 16;
    const int base = B * Hkv;
    // Splits are sized on the selected positions (the whole context when dense); the
    // new-token block is a separate step, so a split holds at most split_cap positions.
    const int sel = max(1, max_list - nv);
    const int target = max(1, target_wgs);
    const int min_s = (sel + split_cap - 1) / split_cap;
    // Query-row groups only as needed for the register budget: every group streams the
    // pair's K/V rows again.
    const int qg = (qt_total + kMaxQT - 1) / kMaxQT;
    p.qt = (qt_total + qg - 1) / qg;
    p.qgroups = (qt_total + p.qt - 1) / p.qt;
    p.pairs = base * p.qgroups;
    // Token splits: the minimum, unless the grid would leave more than half of a round
    // idle; then rounded up to whole rounds.
    int s = min_s;
    if ((long)p.pairs * s * 2 <= target)
        s = (target + p.pairs - 1) / p.pairs;
    if ((long)p.pairs * s > target) {
        const long rounds = ((long)p.pairs * s + target - 1) / target;
        s = max(s, (int)(rounds * target / p.pairs));
    }
    const int max_s = min((sel + kTile - 1) / kTile, kMaxSplits);
    s = max(1, min(s, max_s));
    s = max(s, min_s);
    p.spl = ((sel + s - 1) / s + kTile - 1) / kTile * kTile;
    p.splits = (sel + p.spl - 1) / p.spl;
    p.part_floats = p.splits > 1 ? (size_t)p.pairs * p.splits * ((size_t)p.qt * 16 * 128 + 2 * p.qt * 16) : 0;
    p.grid = (size_t)((base + 7) / 8) * 8 * p.qgroups * p.splits;
    return p;
}

hipError_t launch_attn(const AttnArgs &a, int head_dim, int qt, int ring, hipStream_t st)
{
    const dim3 grid((unsigned)(((a.B * a.Hkv + 7) / 8) * 8 * a.qgroups * a.splits));
    return head_dim == 64 ? launch_d<64>(a, qt, ring, grid, st) : launch_d<128>(a, qt, ring, grid, st);
}

}  // namespace dustin
