// The gather floor of the verification attention: the K and V rows of a selected list read
// the way the attention reads them (16-byte non-temporal loads of one KV head's row slice,
// coalesced per row), with every row of a workgroup's share in flight at once and no
// arithmetic.  Its time per launch is the ceiling for those bytes as they lie in HBM, and
// the attention's time is measured against it.
#include "device.hpp"
#include "floor.hpp"

namespace dustin {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFloorThreads = 512;

// Workgroup x reads list entries [split * kFloorPositions, +kFloorPositions) of sequence b
// and KV head g, x = (b * splits + split) * Hkv + g: the KV heads of one stretch of the list
// go to consecutive workgroups (as in the attention).  Chunk c of the workgroup's
// 2 * kFloorPositions * CPR 16-byte chunks is chunk c % CPR of K row c / CPR (V rows after
// the K rows), so each row's chunks are read by consecutive lanes.
template <int D>
__global__ __launch_bounds__(kFloorThreads) void gather_floor_kernel(FloorArgs a)
{
    constexpr int CPR = D / 8;
    constexpr int NL = 2 * kFloorPositions * CPR / kFloorThreads;
    const int x = blockIdx.x;
    const int g = x % a.Hkv;
    const int rest = x / a.Hkv;
    const int split = rest % a.splits;
    const int b = rest / a.splits;
    const int j0 = split * kFloorPositions;
    const int32_t *list = a.idx + (int64_t)b * a.k_max;
    const uint16_t *kb = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
    const uint16_t *vb = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
    // the list entries first, with one wait (a K load and the V load NH instructions later
    // cover the same RPL entries); then every row load, unconditional (entries past k_max
    // in the last workgroup re-read the row of entry k_max - 1, served by the cache), so
    // all of them are in flight before the first wait; those entries are left out of the XOR
    constexpr int NH = NL / 2;                 // loads per tensor
    constexpr int RPL = kFloorThreads / CPR;   // rows one load instruction covers
    const int ch = (int)threadIdx.x % CPR;
    int tok[NH];
    bool live[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int j = j0 + h * RPL + (int)threadIdx.x / CPR;
        live[h] = j < a.k_max;
        tok[h] = list[min(j, a.k_max - 1)];
    }
    wait_vmcnt<0>();                           // the list entries have landed
    __builtin_amdgcn_sched_barrier(0);
    u32x4 r[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int h = i % NH;
        const int64_t t = min(max(tok[h], 0), a.n_tok - 1);
        const uint16_t *p = i < NH ? kb + t * a.k_st : vb + t * a.v_st;
        r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + ch * 8));
    }
    __builtin_amdgcn_sched_barrier(0);         // every row load is issued before the first use
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i)
        acc ^= live[i % NH] ? r[i][0] ^ r[i][1] ^ r[i][2] ^ r[i][3] : 0u;
    uint32_t *dst = a.checksum + (int64_t)b * a.Hkv + g;
    if (a.mode == 1) {
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1)
            acc ^= __shfl_xor(acc, s);
        if ((threadIdx.x & 63) == 0)
            atomicXor(dst, acc);
    } else if (acc == 0x9e3779b9u) {
        // timing mode: a store that depends on every word read keeps the loads, and in
        // practice never happens
        *dst = acc;
    }
}

}  // namespace

hipError_t launch_gather_floor(const FloorArgs &a, int head_dim, hipStream_t st)
{
    const dim3 grid((unsigned)((int64_t)a.B * a.splits * a.Hkv));
    if (head_dim == 128)
        hipLaunchKernelGGL(gather_floor_kernel<128>, grid, dim3(kFloorThreads), 0, st, a);
    else
        hipLaunchKernelGGL(gather_floor_kernel<64>, grid, dim3(kFloorThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dustin
