// Verification attention over a gathered token list (sparse) or the whole context (dense).
//
// Computes, for every sequence b, verify query t and query head h (KV head g = h / G):
//   out = softmax(scale * q . K[x]) V[x] over x in I_b u {ctx_len[b] + j : j <= t}
// (English Dustin summary, Verification Workflow steps 3-4: the draft block is verified
// against the selected tokens only; the selected rows are gathered by position, never
// copied into a compacted cache, because the method keeps the full history resident —
// "Significance and Limitations" 2).
//
// Work decomposition (gfx950, 64-wide waves, 4 waves per workgroup, one workgroup per CU):
//   workgroup = (b, g, query group, split of the list).  Wave w takes the 32-position
//   steps w, w+4, ... of its split and keeps R of them in flight in its LDS ring:
//     - a step's K and V rows are moved into a ring slot by LDS DMA (non-temporal; every
//       64-lane instruction moves whole rows; 16-byte chunks XOR-swizzled per row so the
//       operand reads are bank-conflict free); a slot is refilled as soon as its
//       operands are in registers;
//     - the wait for a step is an explicit vmcnt of the instructions issued after it.
//       The loop holds no load whose result the compiler tracks, and the slot reads are
//       inline-assembly blocks that end with their own LDS wait, so the compiler adds no
//       conservative wait for the LDS DMA in flight: the ring stays R steps deep.
//   List entries (sparse) reach a per-wave LDS table by LDS DMA, together with Q (staged
//   once per workgroup in the ring area, then held in registers); paged caches are
//   resolved once through the page tables into row numbers in that table.
//   S^T = K Q^T for all (up to QT*16) queries of the KV head's group on
//   v_mfma_f32_16x16x32_bf16; the S^T output layout of a lane is exactly the B operand
//   of the PV product, so P never leaves registers; online softmax in base 2 with a lazy
//   rescale; V^T comes from transposing LDS reads (ds_read_b64_tr_b16) and O^T += V^T P^T.
//   The new-token block (at most 16 rows, causal among themselves) is one 16-row step of
//   wave 3 of the last split, loaded first into its own LDS area.
//   The four waves merge through LDS at the end.  Splits of one (b, g, query group) are
//   merged inside the same kernel: each split writes its (O, max, sum) partial, counts
//   itself in on the pair's counter (a device-scope atomic), and the last split to arrive
//   merges every partial in fixed split order, so the result does not depend on arrival
//   order.  All splits of a pair have the same blockIdx % 8 and so run on one XCD
//   (workgroups are dispatched round-robin over the XCDs), where the partials are
//   exchanged through that XCD's L2 with no device-scope cache write-back.  The counter
//   records the XCDs its arrivals ran on; if they ever differ, the merge writes NaN
//   instead of reading partials another L2 may still hold.  With fused_merge off, a
//   second kernel merges instead.
#include "device.hpp"
#include "launch.hpp"

namespace dustin {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;          // list positions per wave step
constexpr int kNewWave = 3;        // wave of the last split that takes the new-token step
constexpr float kLazy = 8.f;       // rescale O only when a tile's max exceeds the reference by 2^8
// counter word: [63:24] tag, [23:16] XCDs of the arrivals (bit per XCD), [15:0] arrivals.
// A word without the tag (a fresh or foreign workspace) counts as zero arrivals.
constexpr unsigned long long kCtrTag = 0xd5571a7e93ull << 24;
constexpr unsigned long long kCtrTagMask = ~0ull << 24;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// max over the four lanes l, l^16, l^32, l^48 (v_permlane32_swap / v_permlane16_swap)
// In-place sum over each 16-lane row of N values per lane (quad_perm xor 1 and xor 2,
// row_half_mirror, row_mirror); every lane of a row ends with its row's sums.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int N>
__device__ __forceinline__ void row16_sum(float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += dpp_f32<0xB1>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += dpp_f32<0x4E>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += dpp_f32<0x141>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += dpp_f32<0x140>(v[i]);
}

__device__ __forceinline__ float max_over_quads(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}


// LDS byte address of a pointer into the kernel's __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)(const lds_u8 *)(p);
}

__device__ __forceinline__ uint32_t xcc_id()
{
    uint32_t id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
    return id & 7u;
}

// One ring step's MFMA operands out of LDS, in one inline-assembly block that ends with
// its own wait (so every output is complete when the block ends): K as the A operand of
// S^T = K Q^T (ka: 2 halves x KS k-steps, 16-byte reads) and V^T as the A operand of
// O^T += V^T P^T (va: 2 halves x DVT head-dim tiles, transposing 8-byte reads).  The
// transposing read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives 16-bit
// element i % 4 of the 8-byte words addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4 of its group, in that order.
__device__ __forceinline__ void read_step_ops(const uint32_t (&ka)[8], const uint32_t (&va)[16], u32x4 (&k)[8],
                                              u32x2 (&v)[16])
{
    asm volatile(
        "ds_read_b128 %0, %24\n ds_read_b128 %1, %25\n ds_read_b128 %2, %26\n ds_read_b128 %3, %27\n"
        "ds_read_b128 %4, %28\n ds_read_b128 %5, %29\n ds_read_b128 %6, %30\n ds_read_b128 %7, %31\n"
        "ds_read_b64_tr_b16 %8, %32\n ds_read_b64_tr_b16 %9, %33\n ds_read_b64_tr_b16 %10, %34\n"
        "ds_read_b64_tr_b16 %11, %35\n ds_read_b64_tr_b16 %12, %36\n ds_read_b64_tr_b16 %13, %37\n"
        "ds_read_b64_tr_b16 %14, %38\n ds_read_b64_tr_b16 %15, %39\n ds_read_b64_tr_b16 %16, %40\n"
        "ds_read_b64_tr_b16 %17, %41\n ds_read_b64_tr_b16 %18, %42\n ds_read_b64_tr_b16 %19, %43\n"
        "ds_read_b64_tr_b16 %20, %44\n ds_read_b64_tr_b16 %21, %45\n ds_read_b64_tr_b16 %22, %46\n"
        "ds_read_b64_tr_b16 %23, %47\n s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]),
          "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
          "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]),
          "=&v"(v[15])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7]),
          "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]),
          "v"(va[8]), "v"(va[9]), "v"(va[10]), "v"(va[11]), "v"(va[12]), "v"(va[13]), "v"(va[14]), "v"(va[15]));
}

__device__ __forceinline__ void read_step_ops(const uint32_t (&ka)[4], const uint32_t (&va)[8], u32x4 (&k)[4],
                                              u32x2 (&v)[8])
{
    asm volatile(
        "ds_read_b128 %0, %12\n ds_read_b128 %1, %13\n ds_read_b128 %2, %14\n ds_read_b128 %3, %15\n"
        "ds_read_b64_tr_b16 %4, %16\n ds_read_b64_tr_b16 %5, %17\n ds_read_b64_tr_b16 %6, %18\n"
        "ds_read_b64_tr_b16 %7, %19\n ds_read_b64_tr_b16 %8, %20\n ds_read_b64_tr_b16 %9, %21\n"
        "ds_read_b64_tr_b16 %10, %22\n ds_read_b64_tr_b16 %11, %23\n s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
          "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]),
          "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]));
}

// N consecutive ints at LDS byte address a (16-byte aligned), in one block with its wait
__device__ __forceinline__ void read_ints(int (&o)[8], uint32_t a)
{
    u32x4 x, y;
    asm volatile("ds_read_b128 %0, %2\n ds_read_b128 %1, %2 offset:16\n s_waitcnt lgkmcnt(0)"
                 : "=&v"(x), "=&v"(y)
                 : "v"(a));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[i] = (int)x[i];
        o[4 + i] = (int)y[i];
    }
}

__device__ __forceinline__ void read_ints(int (&o)[4], uint32_t a)
{
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(a));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = (int)x[i];
}

// Geometry of one wave step for head dim D.  A step covers kTile list positions; its K
// rows and V rows are each moved into LDS by NI DMA instructions of 64 lanes x 16 bytes,
// instruction n covering LDS rows n*RPI .. n*RPI + RPI - 1 with whole rows per lane
// group (fully coalesced reads).  LDS row rho holds list row tau(rho) = (rho % RPI) * NI +
// rho / RPI of the step, so the NI rows one lane group moves are consecutive list
// positions.  Chunks (16 bytes) of a row are stored XOR-swizzled: K chunk c of row rho
// sits at c ^ (rho % CPR), V chunk c at c ^ (2 rho % CPR), which makes the MFMA operand
// reads (K: 16 rows x one chunk; V transposed: 8 rows x two chunks per half-wave)
// bank-conflict free.
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
    static constexpr int GOPS = 2 * NI;         // memory instructions one step issues
    __device__ static constexpr int tau(int rho) { return (rho % RPI) * NI + rho / RPI; }
};

template <int D, int QT>
struct AttnShape {
    using G = Geo<D>;
    // ring slots per wave: the ring holds 128 KB per workgroup (16 KB steps at head dim
    // 128, 8 KB at 64)
    static constexpr int R = D == 64 ? 4 : 2;
    static constexpr int QR = QT * 16;          // padded query rows
    static constexpr int ACC = G::DVT * QT * 4; // O accumulator floats per lane
    static constexpr int RING = 4 * R * G::SLOT;
    static constexpr int TAB = 4 * kAttnStepsMaxW * kTile * 4;   // list entries / row numbers of the 4 waves
    static constexpr int NEWB = 2 * 16 * G::RB; // new-token rows: 16 K, then 16 V
    // The four waves' accumulators are exchanged through the ring area, each wave's through
    // its own ring slots (free as soon as its own loop has ended), in one pass or in two
    // (half of the head-dim tiles each) where one would not fit.
    static constexpr int XW = RING / 4 / 4;     // floats of one wave's exchange area
    static constexpr int MRG1 = 64 * ACC * 4 + 2 * QR * 4;
    static constexpr int PH = MRG1 > RING / 4 ? 2 : 1;
    static constexpr int MRG = 64 * (ACC / PH) * 4 + 2 * QR * 4;
    static_assert(MRG <= RING / 4, "exchange fits a wave's ring slots");
    static constexpr int OFF_TAB = RING;
    static constexpr int OFF_NEW = OFF_TAB + TAB;
    static constexpr int OFF_FLAG = OFF_NEW + NEWB;
    static constexpr int LDS = OFF_FLAG + 16;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert((R - 1) * G::GOPS < 64, "vmcnt range");
};

// Record of one split's partial result: O (unnormalised, relative to m) [QR][D], m [QR]
// (base-2 scaled logits), l [QR]; padded to 256 bytes so no cache line holds two records.
__host__ __device__ constexpr int64_t part_stride(int qr, int d)
{
    return ((int64_t)qr * d + 2 * qr + 63) / 64 * 64;
}

// Split partials are combined in fixed split order 0, 1, ..., splits-1 (the same
// operations in the fused merge and in the merge kernel, so both give the same bits):
// with split s's (m_s, l_s, acc_s), M = max_s m_s, w_s = e^{m_s - M},
//   O = sum_s w_s acc_s / sum_s w_s l_s,  LSE = M + log sum_s w_s l_s
// (base-2 scaled logits, natural-log LSE).  The weights depend on the row only.
struct SplitSum {
    float M, den;
    f32x4 num;
};

__device__ __forceinline__ float split_weight(float m, float M) { return M == -INFINITY ? 0.f : fast_exp2(m - M); }

// Writes one (row, 4 head-dim columns) item of the merged result (NaN when poisoned).
template <int D>
__device__ __forceinline__ void split_write(const AttnArgs &a, const SplitSum &t, int b, int g, int row, int dv,
                                           bool poison)
{
    const float inv = 1.f / t.den;
    const int tq = row / a.G;
    const int h = g * a.G + (row - tq * a.G);
    uint16_t *o = a.out + ((int64_t)(b * a.nv + tq) * a.Hq + h) * D + dv;
    u32x2 ov = u32x2{pack_bf16x2(t.num[0] * inv, t.num[1] * inv), pack_bf16x2(t.num[2] * inv, t.num[3] * inv)};
    float lse = (t.M + __log2f(t.den)) * kLn2;
    if (poison) {
        ov = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
        lse = __uint_as_float(0x7fc00000u);
    }
    *reinterpret_cast<u32x2 *>(o) = ov;
    if (dv == 0)
        a.lse[((int64_t)b * a.Hq + h) * a.nv + tq] = lse;
}

// EMIT: also write the Collect-2 logit sums of the list rows (a.logit2)
template <int D, int QT, bool EMIT>
__global__ __launch_bounds__(kThreads) void verify_attn_kernel(AttnArgs a)
{
    using S = AttnShape<D, QT>;
    using G = Geo<D>;
    constexpr int R = S::R;
    __shared__ __align__(16) uint8_t lds[S::LDS];

    // The argument fields the prologue and the ring need, requested from the kernel
    // argument segment in one batch with one wait (left to itself the compiler loads each
    // where it is first used, one dependent round trip after another).
    asm volatile("" ::"s"(a.B), "s"(a.Hkv), "s"(a.qgroups), "s"(a.splits), "s"(a.spl), "s"(a.GV), "s"(a.G),
                 "s"(a.nv), "s"(a.Hq), "s"(a.q), "s"(a.idx), "s"(a.count), "s"(a.ctx_len), "s"(a.k_max),
                 "s"(a.k.base), "s"(a.k.sb), "s"(a.k.st), "s"(a.k.sh), "s"(a.v.base), "s"(a.v.sb), "s"(a.v.st),
                 "s"(a.v.sh), "s"(a.kv_same), "s"(a.rows_mode), "s"(a.ctx_clamp));

    // ---- block -> (sequence, KV head, query group, split).  Every workgroup of one
    //      (sequence, KV head) has the same blockIdx % 8, i.e. runs on the same XCD ----
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
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int lane = tid & 63;
    const int quad = lane >> 4;   // MFMA lane group
    const int li = lane & 15;
    const int dg = lane / G::CPR; // DMA: row group of the lane within an instruction
    const int dc = lane % G::CPR; // DMA: LDS chunk of the lane within its row
    const int p0 = split * a.spl;
    const bool sparse = a.idx != nullptr;

    // ---- per-sequence values, as vector loads (an opaque zero index keeps them off the
    //      scalar path) so they travel in the same round trip as Q and the list entries:
    //      a scalar load here would cost its own round trip before the first DMA ----
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int n_v = a.ctx_len[b + zero];
    const int c_v = sparse ? a.count[b + zero] : 0;

    // ---- Q of the query group into the ring area (not yet in use) by LDS DMA, a quarter
    //      of the rows per wave, chunk c of row r at c ^ (r % CPR); padding rows copy the
    //      group's first row and are never written out ----
    {
        constexpr int NQI = S::QR * G::RB / 1024;
        for (int n = w; n < NQI; n += 4) {
            const int r = n * G::RPI + dg;
            const int row = qg * S::QR + r;
            const int rr = row < a.GV ? row : qg * S::QR;
            const int t = rr / a.G;
            const int h = g * a.G + (rr - t * a.G);
            const int ck = dc ^ (r % G::CPR);
            __builtin_amdgcn_global_load_lds((const void *)(a.q + ((int64_t)(b * a.nv + t) * a.Hq + h) * D + ck * 8),
                                             (lds_void *)(lds + n * 1024), 16, 0, 0);
        }
    }
    // Collect-2 emission (one query group holds every row of the pair): lane column li of
    // tile qt counts when its query row is a real row of verify query 0 or n_verify-1
    constexpr bool emit = EMIT;
    float wq[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int row = qt * 16 + li;
        const int t = row / a.G;
        wq[qt] = emit && row < a.GV && (t == 0 || t == a.nv - 1) ? 1.f : 0.f;
    }
    int qrow_t[QT];   // verify index t of the lane's query row (large for padding rows)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int row = qg * S::QR + qt * 16 + li;
        qrow_t[qt] = row < a.GV ? row / a.G : 1 << 20;
    }

    // ---- this wave's list entries (as many steps as the split can hold: the count is
    //      not known yet) into its LDS table by DMA, one dword per lane, in the same round
    //      trip as Q ----
    const int tiles_max = (a.spl + kTile - 1) / kTile;
    const int steps_max = tiles_max > w ? (tiles_max - w + 3) >> 2 : 0;
    const bool tab_mode = sparse || a.rows_mode;   // per-step rows come from the table
    int32_t *tab = reinterpret_cast<int32_t *>(lds + S::OFF_TAB) + w * kAttnStepsMaxW * kTile;
    // rows mode with K and V rows at different places: V rows in the second half of the
    // table (the plan halves the split capacity then)
    int32_t *tabV = a.kv_same ? tab : tab + kAttnStepsMaxW * kTile / 2;
    if (sparse && a.k_max > 0) {
        const int32_t *row = a.idx + (int64_t)b * a.k_max;
        for (int i0 = 0; i0 < steps_max * kTile; i0 += 64) {
            const int i = i0 + lane;
            const int pos = min(p0 + (w + 4 * (i / kTile)) * kTile + i % kTile, a.k_max - 1);
            __builtin_amdgcn_global_load_lds((const void *)(row + pos), (lds_void *)(tab + i0), 4, 0, 0);
        }
    }
    wait_vmcnt<0>();                  // Q and the list entries have landed
    __syncthreads();                  // every wave's share of Q
    // Q as the B operand of S^T = K Q^T: lane holds q-row qt*16 + li, head-dim elements
    // ks*32 + quad*8 .. +8 for k-step ks (no LDS DMA is in flight here)
    u32x4 qop[QT][G::KS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
            qop[qt][ks] = *reinterpret_cast<const u32x4 *>(
                lds + (qt * 16 + li) * G::RB + (((ks * 4 + quad) ^ ((qt * 16 + li) % G::CPR)) << 4));

    // ---- sequence geometry; every device value is clamped ----
    const int N = clampi(__builtin_amdgcn_readfirstlane(n_v), 0, a.ctx_clamp);
    const int nsel = sparse ? clampi(__builtin_amdgcn_readfirstlane(c_v), 0, min(a.k_max, N)) : N;
    const int p1 = min(p0 + a.spl, nsel);
    const int cnt = max(p1 - p0, 0);
    const int ntile = (cnt + kTile - 1) / kTile;
    const int mine = ntile > w ? (ntile - w + 3) >> 2 : 0;    // steps w, w+4, ... of this wave
    const bool new_here = split == a.splits - 1 && w == kNewWave;
    // token of list row j of wave step s: positions past the split's end read token N
    // (the first new token, always present), whose scores are masked
    auto token = [&](int s, int j, int raw) {
        const int pos = p0 + (w + 4 * s) * kTile + j;
        return pos >= p1 ? N : (sparse ? clampi(raw, 0, N - 1) : pos);
    };

    if (a.rows_mode) {
        // paged caches: every entry resolved through the page tables (all loads of the
        // wave in one round), stored back as a row number (element offset / stride_token).
        // No LDS DMA is in flight here.
        constexpr int EPL = kAttnStepsMaxW * kTile / 64;
        const int n_ent = min(steps_max * kTile, a.kv_same ? kAttnStepsMaxW * kTile : kAttnStepsMaxW * kTile / 2);
        int tk[EPL], pk[EPL], pv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int i = e * 64 + lane;
            tk[e] = token(i / kTile, i % kTile, i < n_ent && sparse ? tab[i] : 0);
            pk[e] = a.k.pt && i < n_ent ? a.k.pt[(int64_t)b * a.k.max_pages + (tk[e] >> a.k.ps_log2)] : 0;
            pv[e] = a.v.pt && i < n_ent && !a.kv_same ? a.v.pt[(int64_t)b * a.v.max_pages + (tk[e] >> a.v.ps_log2)] : 0;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int i = e * 64 + lane;
            if (i < n_ent) {
                const uint32_t rk = a.k.pt ? (uint32_t)clampi(pk[e], 0, a.k.num_pages - 1) * (uint32_t)a.k.rows_per_page +
                                                 (uint32_t)(tk[e] & ((1 << a.k.ps_log2) - 1))
                                           : (uint32_t)b * (uint32_t)a.k.rows_per_batch + (uint32_t)tk[e];
                tab[i] = (int32_t)rk;
                if (!a.kv_same) {
                    const uint32_t rv = a.v.pt ? (uint32_t)clampi(pv[e], 0, a.v.num_pages - 1) * (uint32_t)a.v.rows_per_page +
                                                     (uint32_t)(tk[e] & ((1 << a.v.ps_log2) - 1))
                                               : (uint32_t)b * (uint32_t)a.v.rows_per_batch + (uint32_t)tk[e];
                    tabV[i] = (int32_t)rv;
                }
            }
        }
        wait_lgkm0();
        __builtin_amdgcn_wave_barrier();
    }

    const uint16_t *kbase = a.k.base + (int64_t)g * a.k.sh;
    const uint16_t *vbase = a.v.base + (int64_t)g * a.v.sh;
    const float c = a.scale_log2;     // logits are multiplied by scale * log2(e), any sign

    wait_lgkm0();
    __syncthreads();                  // every wave holds Q: the ring area is free
    // ---- the new-token rows first (wave 3 of the last split): LDS row rho (< 16) of the
    //      new-token area holds new token min(rho, nv-1), K rows then V rows ----
    uint8_t *nslot = lds + S::OFF_NEW;
    if (new_here) {
#pragma unroll
        for (int n = 0; n < G::NI / 2; ++n) {
            const int rho = n * G::RPI + dg;
            const int tok = N + min(rho, a.nv - 1);
            const int ck = dc ^ (rho % G::CPR);
            const int cv = dc ^ ((2 * rho) % G::CPR);
            __builtin_amdgcn_global_load_lds((const void *)(a.k.base + kv_offset(a.k, b, tok, g) + ck * 8),
                                             (lds_void *)(nslot + n * 1024), 16, 0, kLoadNonTemporal);
            __builtin_amdgcn_global_load_lds((const void *)(a.v.base + kv_offset(a.v, b, tok, g) + cv * 8),
                                             (lds_void *)(nslot + 16 * G::RB + n * 1024), 16, 0, kLoadNonTemporal);
        }
    }

    // ---- the ring: step s of this wave into slot r.  Lane group dg moves list rows
    //      dg*NI + n (n < NI) of the step. ----
    uint8_t *wring = lds + w * R * G::SLOT;
    auto issue = [&](int s, int r) {
        uint8_t *dst = wring + r * G::SLOT;
        int64_t ok[G::NI], ov[G::NI];
        {
            int raw[G::NI], rawv[G::NI];
            if (tab_mode) {
                read_ints(raw, lds_addr(reinterpret_cast<uint8_t *>(tab + s * kTile + dg * G::NI)));
                if (a.rows_mode && !a.kv_same)
                    read_ints(rawv, lds_addr(reinterpret_cast<uint8_t *>(tabV + s * kTile + dg * G::NI)));
            }
#pragma unroll
            for (int n = 0; n < G::NI; ++n) {
                if (a.rows_mode) {
                    ok[n] = (int64_t)(uint32_t)raw[n] * a.k.st;
                    ov[n] = (int64_t)(uint32_t)(a.kv_same ? raw[n] : rawv[n]) * a.v.st;
                } else {
                    const int tok = token(s, dg * G::NI + n, sparse ? raw[n] : 0);
                    ok[n] = (int64_t)b * a.k.sb + (int64_t)tok * a.k.st;
                    ov[n] = (int64_t)b * a.v.sb + (int64_t)tok * a.v.st;
                }
            }
        }
#pragma unroll
        for (int n = 0; n < G::NI; ++n) {
            const int rho = n * G::RPI + dg;
            const int ck = dc ^ (rho % G::CPR);
            __builtin_amdgcn_global_load_lds((const void *)(kbase + ok[n] + ck * 8), (lds_void *)(dst + n * 1024), 16, 0,
                                             kLoadNonTemporal);
        }
#pragma unroll
        for (int n = 0; n < G::NI; ++n) {
            const int rho = n * G::RPI + dg;
            const int cv = dc ^ ((2 * rho) % G::CPR);
            __builtin_amdgcn_global_load_lds((const void *)(vbase + ov[n] + cv * 8),
                                             (lds_void *)(dst + G::HALF + n * 1024), 16, 0, kLoadNonTemporal);
        }
    };

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

    // per-lane LDS byte offsets (slot-relative) of the operand reads: K row 16h + li,
    // chunk ks*4 + quad; V^T: source lane s = li of group quad reads row 16h + 4*quad +
    // s/4, head-dim columns dt*16 + 4*(s%4) .. +3, i.e. chunk 2*dt + (s%4)/2, byte 8*(s%2)
    uint32_t kq[2 * G::KS], vq[2 * G::DVT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const int rho = 16 * h + li;
            kq[h * G::KS + ks] = rho * G::RB + (((ks * 4 + quad) ^ (rho % G::CPR)) << 4);
        }
        const int rho = 16 * h + 4 * quad + (li >> 2);
        const int vrow = G::HALF + rho * G::RB + (((li >> 1) & 1) << 4) + ((li & 1) << 3);
        const int vf2 = rho % (G::CPR / 2);
#pragma unroll
        for (int dt = 0; dt < G::DVT; ++dt)
            vq[h * G::DVT + dt] = vrow + ((dt ^ vf2) << 5);
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
    auto math = [&](const u32x4 (&kop)[2][G::KS], const u32x4 (&vop)[G::DVT], bool full, int pos0, bool direct,
                    int pend) {
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

        // Collect-2 logits of the step's list rows: the emitted columns summed per row
        // (over the tiles, then over the 16 lanes of the row's quad), scaled to natural-log
        // units; lane 0 of each quad stores its 8 rows
        if (emit && !direct) {
            float e[8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = 0.f;
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt)
                        v += wq[qt] * s[h][qt][r];
                    e[4 * h + r] = v;
                }
            row16_sum<8>(e);
            if (li == 0) {
                float *dst = a.logit2 + ((int64_t)b * a.Hkv + g) * a.k_max;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int pos = pos0 + trow[h][r];
                        if (pos < pend)
                            dst[pos] = e[4 * h + r] * a.scale;
                    }
            }
        }

        u32x4 pb[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = s[h][qt][r] * c;
                    if (!full) {
                        const int pos = pos0 + (direct ? 16 * h + 4 * quad + r : trow[h][r]);
                        const bool ok = (pos < pend) & ((pos < nsel) | (pos - nsel <= qrow_t[qt]));
                        v = ok ? v : -INFINITY;
                    }
                    s[h][qt][r] = v;
                }
            float mx = fmaxf(fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), fmaxf(s[0][qt][2], s[0][qt][3])),
                             fmaxf(fmaxf(s[1][qt][0], s[1][qt][1]), fmaxf(s[1][qt][2], s[1][qt][3])));
            mx = max_over_quads(mx);
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
                    p[h][r] = fast_exp2(s[h][qt][r] + nm);
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

    // ---- issue the first R steps; then per step: wait for it (the explicit vmcnt of the
    //      steps issued after it: the loop holds no load the compiler tracks, and the slot
    //      reads are inline-assembly blocks with their own LDS wait, so no other wait is
    //      inserted), read its operands, refill its slot, compute ----
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < mine)
            issue(r, r);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (new_here) {
        // the new-token step first: its rows were requested before the ring's first steps,
        // which stay in flight (the wait counts exactly the ring loads issued after them)
        const int issued = min(mine, R);
        if (issued >= R)
            wait_vmcnt<R * G::GOPS>();
        else if (R > 3 && issued == 3)
            wait_vmcnt<(R > 3 ? 3 : 0) * G::GOPS>();
        else if (R > 2 && issued == 2)
            wait_vmcnt<(R > 2 ? 2 : 0) * G::GOPS>();
        else if (issued == 1)
            wait_vmcnt<G::GOPS>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        // rows 16..31 have zero operands and are masked.  The reads are one assembly block
        // (the first half's addresses twice), so the compiler adds no wait for the ring
        // loads still in flight.
        const uint32_t na = lds_addr(nslot);
        uint32_t ka[2 * G::KS], va[2 * G::DVT];
#pragma unroll
        for (int i = 0; i < 2 * G::KS; ++i)
            ka[i] = na + kq[i % G::KS];
#pragma unroll
        for (int i = 0; i < 2 * G::DVT; ++i)
            va[i] = na + vq[i % G::DVT] - G::HALF + 16 * G::RB;
        u32x4 kraw[2 * G::KS];
        u32x2 vraw[2 * G::DVT];
        read_step_ops(ka, va, kraw, vraw);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 kop[2][G::KS], vop[G::DVT];
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            kop[0][ks] = kraw[ks];
            kop[1][ks] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int dt = 0; dt < G::DVT; ++dt)
            vop[dt] = u32x4{vraw[dt][0], vraw[dt][1], 0, 0};
        math(kop, vop, false, nsel, true, nsel + a.nv);
    }
    for (int j0 = 0; j0 < mine; j0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int jj = j0 + r;
            if (jj >= mine)
                break;
            // steps issued after step jj: min(mine - 1 - jj, R - 1)
            const int later = min(mine - 1 - jj, R - 1);
            if (later >= R - 1)
                wait_vmcnt<(R - 1) * G::GOPS>();
            else if (R > 2 && later == 2)
                wait_vmcnt<(R > 2 ? 2 : 0) * G::GOPS>();
            else if (R > 1 && later == 1)
                wait_vmcnt<G::GOPS>();
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t sa = lds_addr(wring + r * G::SLOT);
            uint32_t ka[2 * G::KS], va[2 * G::DVT];
#pragma unroll
            for (int i = 0; i < 2 * G::KS; ++i)
                ka[i] = sa + kq[i];
#pragma unroll
            for (int i = 0; i < 2 * G::DVT; ++i)
                va[i] = sa + vq[i];
            u32x4 kraw[2 * G::KS];
            u32x2 vraw[2 * G::DVT];
            read_step_ops(ka, va, kraw, vraw);     // the slot's operands are in registers
            __builtin_amdgcn_sched_barrier(0);
            if (jj + R < mine)
                issue(jj + R, r);
            __builtin_amdgcn_sched_barrier(0);
            u32x4 kop[2][G::KS], vop[G::DVT];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks)
                    kop[h][ks] = kraw[h * G::KS + ks];
#pragma unroll
            for (int dt = 0; dt < G::DVT; ++dt)
                vop[dt] = u32x4{vraw[dt][0], vraw[dt][1], vraw[G::DVT + dt][0], vraw[G::DVT + dt][1]};
            const int pos0 = p0 + (w + 4 * jj) * kTile;
            math(kop, vop, pos0 + kTile <= p1, pos0, false, p1);
        }
    }
    wait_vmcnt<0>();                  // every ring load of the wave has landed

    // ---- merge the four waves through LDS: every wave publishes its maxima, sums and
    //      O^T accumulators (all head-dim tiles, or half of them per phase) into its own
    //      ring slots as soon as its loop has ended (no wait for the other waves), then
    //      wave w merges a quarter of the published tiles of every row ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        lrun[qt] += __shfl_xor(lrun[qt], 16);
        lrun[qt] += __shfl_xor(lrun[qt], 32);
    }
    constexpr int DVTP = G::DVT / S::PH;   // head-dim tiles exchanged per phase
    constexpr int DPW = DVTP / 4;          // head-dim tiles merged by each wave per phase
    // wave v's area: [dv tile of the phase][qt][lane][4] floats, then its maxima [QR] and
    // sums [QR]
    float *const xBase = reinterpret_cast<float *>(lds);
    auto xAcc = [&](int v) { return xBase + v * S::XW; };
    auto xM = [&](int v) { return xBase + v * S::XW + 64 * (S::ACC / S::PH); };
    auto xL = [&](int v) { return xBase + v * S::XW + 64 * (S::ACC / S::PH) + S::QR; };
    if (quad == 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            xM(w)[qt * 16 + li] = mref[qt];
            xL(w)[qt * 16 + li] = lrun[qt];
        }
    }
    const bool direct_out = a.splits == 1;
    const int64_t pstride = part_stride(S::QR, D);
    float *part = a.part + ((int64_t)pair * a.splits + split) * pstride;
    // this workgroup's result, per lane: rows q = qt*16 + li, head-dim tiles (ph, w*DPW + j)
    f32x4 res[S::PH][QT][DPW];
    float resM[QT], resL[QT];
#pragma unroll
    for (int ph = 0; ph < S::PH; ++ph) {
        if (ph > 0)
            __syncthreads();          // the previous phase's tiles have been read
#pragma unroll
        for (int i = 0; i < DVTP; ++i)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                *reinterpret_cast<f32x4 *>(xAcc(w) + ((i * QT + qt) * 64 + lane) * 4) = acc[ph * DVTP + i][qt];
        __syncthreads();              // every wave's tiles, maxima and sums are published
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int q = qt * 16 + li;
            float mw[4], M = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                mw[v] = xM(v)[q];
                M = fmaxf(M, mw[v]);
            }
            float f[4], l = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                f[v] = M == -INFINITY ? 0.f : fast_exp2(mw[v] - M);
                l += f[v] * xL(v)[q];
            }
            resM[qt] = M;
            resL[qt] = l;
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                const int i = w * DPW + j;
                f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    o += f[v] * *reinterpret_cast<const f32x4 *>(xAcc(v) + ((i * QT + qt) * 64 + lane) * 4);
                res[ph][qt][j] = o;
            }
        }
    }
    if (direct_out) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int row = qg * S::QR + qt * 16 + li;
            if (row >= a.GV)
                continue;             // padding rows are never written
            SplitSum t;
#pragma unroll
            for (int ph = 0; ph < S::PH; ++ph)
#pragma unroll
                for (int j = 0; j < DPW; ++j) {
                    t.M = resM[qt];
                    t.den = resL[qt];
                    t.num = res[ph][qt][j];
                    split_write<D>(a, t, b, g, row, (ph * DVTP + w * DPW + j) * 16 + 4 * quad, false);
                }
        }
        return;
    }
    // the partial record: O [QR][D], m [QR], l [QR]
#pragma unroll
    for (int ph = 0; ph < S::PH; ++ph)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int j = 0; j < DPW; ++j)
                *reinterpret_cast<f32x4 *>(part + (int64_t)(qt * 16 + li) * D + (ph * DVTP + w * DPW + j) * 16 +
                                           4 * quad) = res[ph][qt][j];
    if (w == 0 && quad == 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            part[S::QR * D + qt * 16 + li] = resM[qt];
            part[S::QR * D + S::QR + qt * 16 + li] = resL[qt];
        }
    }
    if (!a.fused_merge)
        return;

    // ---- split merge in this kernel: count in on the pair's counter once this
    //      workgroup's partial is complete in L2; the last arrival merges ----
    wait_vmcnt<0>();                  // this wave's partial stores are acknowledged
    __syncthreads();                  // ... and every wave's
    uint32_t *sflag = reinterpret_cast<uint32_t *>(lds + S::OFF_FLAG);
    if (tid == 0) {
        unsigned long long *ctr = a.counter + pair;
        const unsigned long long me = 1ull << (16 + xcc_id());
        unsigned long long old = kCtrTag, nw = 0;
        for (;;) {   // compare-and-swap; retries only when another split arrived meanwhile
            const unsigned long long cur = (old & kCtrTagMask) == kCtrTag ? old : kCtrTag;
            nw = (cur | me) + 1;
            if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
                break;
        }
        const bool last = (int)(nw & 0xffff) == a.splits;
        const uint32_t xm = (uint32_t)(nw >> 16) & 0xff;
        sflag[0] = last ? 1u : 0u;
        sflag[1] = (xm & (xm - 1)) == 0 ? 0u : 1u;     // arrivals on more than one XCD
        if (last)   // every split has arrived: the next call starts from zero
            __hip_atomic_store(ctr, kCtrTag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (sflag[0] == 0)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const bool poison = sflag[1] != 0;
    // The last arrival: every other split's values for this lane's items, the first kPre
    // splits requested in one round (index clamped; the copies are not used), then the
    // fixed-order combination with this workgroup's own values at its split.
    constexpr int kPre = 4;
    const float *base = a.part + (int64_t)pair * a.splits * pstride;
    f32x4 po[kPre][S::PH][QT][DPW];
    float pm[kPre][QT], pl[kPre][QT];
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) {
        const float *ps = base + min(sp, a.splits - 1) * pstride;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            pm[sp][qt] = ps[S::QR * D + qt * 16 + li];
            pl[sp][qt] = ps[S::QR * D + S::QR + qt * 16 + li];
#pragma unroll
            for (int ph = 0; ph < S::PH; ++ph)
#pragma unroll
                for (int j = 0; j < DPW; ++j)
                    po[sp][ph][qt][j] = *reinterpret_cast<const f32x4 *>(
                        ps + (int64_t)(qt * 16 + li) * D + (ph * DVTP + w * DPW + j) * 16 + 4 * quad);
        }
    }
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp)
        if (sp == split)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                pm[sp][qt] = resM[qt];
                pl[sp][qt] = resL[qt];
#pragma unroll
                for (int ph = 0; ph < S::PH; ++ph)
#pragma unroll
                    for (int j = 0; j < DPW; ++j)
                        po[sp][ph][qt][j] = res[ph][qt][j];
            }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int row = qg * S::QR + qt * 16 + li;
        if (row >= a.GV)
            continue;
        auto m_of = [&](int sp) -> float {
            if (sp < kPre)
                return pm[sp][qt];
            return sp == split ? resM[qt] : base[sp * pstride + S::QR * D + qt * 16 + li];
        };
        float M = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < kPre; ++sp)
            M = fmaxf(M, sp < a.splits ? pm[sp][qt] : -INFINITY);
        for (int sp = kPre; sp < a.splits; ++sp)
            M = fmaxf(M, m_of(sp));
        float wt[kPre], den = 0.f;
#pragma unroll
        for (int sp = 0; sp < kPre; ++sp) {
            wt[sp] = sp < a.splits ? split_weight(pm[sp][qt], M) : 0.f;
            den += wt[sp] * pl[sp][qt];
        }
        for (int sp = kPre; sp < a.splits; ++sp)
            den += split_weight(m_of(sp), M) *
                   (sp == split ? resL[qt] : base[sp * pstride + S::QR * D + S::QR + qt * 16 + li]);
#pragma unroll
        for (int ph = 0; ph < S::PH; ++ph)
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                const int dv = (ph * DVTP + w * DPW + j) * 16 + 4 * quad;
                SplitSum t;
                t.M = M;
                t.den = den;
                t.num = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sp = 0; sp < kPre; ++sp)
                    t.num += wt[sp] * po[sp][ph][qt][j];
                for (int sp = kPre; sp < a.splits; ++sp)
                    t.num += split_weight(m_of(sp), M) *
                             (sp == split ? res[ph][qt][j]
                                          : *reinterpret_cast<const f32x4 *>(base + sp * pstride +
                                                                             (int64_t)(qt * 16 + li) * D + dv));
                split_write<D>(a, t, b, g, row, dv, poison);
            }
    }
}

// The split merge as its own kernel (fused_merge off): one thread per (row, 4-column)
// item, D/64 blocks per 16-row tile, blocks of a pair on the XCD of its splits; the same
// fixed-order combination as the fused merge.
template <int D, int QT>
__global__ __launch_bounds__(kThreads) void verify_attn_merge_kernel(AttnArgs a)
{
    constexpr int QR = QT * 16;
    constexpr int BPQ = D / 64;       // blocks per 16-row query tile
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
    const int q = qt * 16 + item / (D / 4);
    const int dv = (item % (D / 4)) * 4;
    const int row = qg * QR + q;
    if (row >= a.GV)
        return;
    const int64_t pstride = part_stride(QR, D);
    const float *base = a.part + (int64_t)pair * a.splits * pstride;
    constexpr int kPre = 4;
    float pm[kPre], pl[kPre];
    f32x4 po[kPre];
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) {
        const float *ps = base + min(sp, a.splits - 1) * pstride;
        pm[sp] = ps[QR * D + q];
        pl[sp] = ps[QR * D + QR + q];
        po[sp] = *reinterpret_cast<const f32x4 *>(ps + (int64_t)q * D + dv);
    }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp)
        M = fmaxf(M, sp < a.splits ? pm[sp] : -INFINITY);
    for (int sp = kPre; sp < a.splits; ++sp)
        M = fmaxf(M, base[sp * pstride + QR * D + q]);
    float wt[kPre], den = 0.f;
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp) {
        wt[sp] = sp < a.splits ? split_weight(pm[sp], M) : 0.f;
        den += wt[sp] * pl[sp];
    }
    for (int sp = kPre; sp < a.splits; ++sp)
        den += split_weight(base[sp * pstride + QR * D + q], M) * base[sp * pstride + QR * D + QR + q];
    SplitSum t;
    t.M = M;
    t.den = den;
    t.num = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < kPre; ++sp)
        t.num += wt[sp] * po[sp];
    for (int sp = kPre; sp < a.splits; ++sp)
        t.num += split_weight(base[sp * pstride + QR * D + q], M) *
                 *reinterpret_cast<const f32x4 *>(base + sp * pstride + (int64_t)q * D + dv);
    split_write<D>(a, t, b, g, row, dv, false);
}

template <int D, int QT>
hipError_t launch_qt(const AttnArgs &a, dim3 grid, hipStream_t st)
{
    if (a.logit2)
        hipLaunchKernelGGL((verify_attn_kernel<D, QT, true>), grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((verify_attn_kernel<D, QT, false>), grid, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1 || a.fused_merge)
        return e;
    const dim3 mgrid((unsigned)((a.B * a.Hkv + 7) / 8 * 8 * a.qgroups * QT * (D / 64)));
    hipLaunchKernelGGL((verify_attn_merge_kernel<D, QT>), mgrid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs &a, int qt, dim3 grid, hipStream_t st)
{
    switch (qt) {
    case 1: return launch_qt<D, 1>(a, grid, st);
    case 2: return launch_qt<D, 2>(a, grid, st);
    case 3: return launch_qt<D, 3>(a, grid, st);
    case 4: return launch_qt<D, 4>(a, grid, st);
    default: return launch_qt<D, 5>(a, grid, st);
    }
}

}  // namespace

size_t attn_part_floats(int qt, int head_dim) { return (size_t)part_stride(qt * 16, head_dim); }

AttnPlan plan_attn(int B, int Hkv, int G, int nv, int head_dim, int max_list, int target_wgs, int split_cap)
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
    if (p.pairs <= 0) {               // an empty batch: nothing to launch, no workspace
        p.spl = kTile;
        p.splits = 1;
        p.part_floats = 0;
        p.counters = 0;
        p.grid = 0;
        return p;
    }
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
    p.part_floats = p.splits > 1 ? (size_t)p.pairs * p.splits * attn_part_floats(p.qt, head_dim) : 0;
    p.counters = p.splits > 1 ? (size_t)p.pairs : 0;
    p.grid = (size_t)((base + 7) / 8) * 8 * p.qgroups * p.splits;
    return p;
}

hipError_t launch_attn(const AttnArgs &a, int head_dim, int qt, hipStream_t st)
{
    const dim3 grid((unsigned)(((a.B * a.Hkv + 7) / 8) * 8 * a.qgroups * a.splits));
    return head_dim == 64 ? launch_d<64>(a, qt, grid, st) : launch_d<128>(a, qt, grid, st);
}

}  // namespace dustin
