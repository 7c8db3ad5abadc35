// Device-side helpers shared by the gfx950 kernels of the sparse-verification library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dustin.h"

namespace dustin {

// ---- MFMA (gfx950 v_mfma_f32_16x16x32_bf16) ---------------------------------------------
// Operand layout relied on (lane l of the 64-lane wave, g = l / 16, j = 0..7):
//   A (16 x 32): lane l supplies A[row = l % 16][k-slot (g, j)]
//   B (32 x 16): lane l supplies B[k-slot (g, j)][col = l % 16]
//   C (16 x 16): lane l holds C[row = 4*g + r][col = l % 16], r = 0..3
// A k-slot (g, j) always pairs with B k-slot (g, j), so any fixed assignment of the
// contraction index to slots is valid as long as both operands use the same one.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- KV view addressing ---------------------------------------------------------------
struct KvView {
    const uint16_t *base;
    int64_t sb, st, sh, sp;
    const int32_t *pt;
    int32_t cap;        // tokens addressable per sequence
    int32_t ps_log2;    // paged: log2(page_size)
    int32_t max_pages;
    int32_t num_pages;
    int64_t rows_per_batch;   // stride_batch / stride_token (when a multiple)
    int64_t rows_per_page;    // stride_page / stride_token (when a multiple)
};

inline KvView make_view(const dustin_kv_view &v)
{
    KvView o;
    o.base = static_cast<const uint16_t *>(v.base);
    o.sb = v.stride_batch;
    o.st = v.stride_token;
    o.sh = v.stride_head;
    o.sp = v.stride_page;
    o.pt = v.page_table;
    o.ps_log2 = 0;
    o.max_pages = v.max_pages;
    o.num_pages = v.num_pages;
    o.rows_per_batch = v.stride_token > 0 && v.stride_batch % v.stride_token == 0 ? v.stride_batch / v.stride_token : -1;
    o.rows_per_page = v.stride_token > 0 && v.stride_page % v.stride_token == 0 ? v.stride_page / v.stride_token : -1;
    if (v.page_table) {
        while ((1 << o.ps_log2) < v.page_size)
            ++o.ps_log2;
        o.cap = v.max_pages * v.page_size;
    } else {
        o.cap = v.n_tokens;
    }
    return o;
}

// Element offset of row (b, t, h); t must already lie in [0, cap).
__device__ __forceinline__ int64_t kv_offset(const KvView &v, int b, int t, int h)
{
    if (v.pt) {
        int pg = v.pt[(int64_t)b * v.max_pages + (t >> v.ps_log2)];
        pg = clampi(pg, 0, v.num_pages - 1);
        return (int64_t)pg * v.sp + (int64_t)(t & ((1 << v.ps_log2) - 1)) * v.st + (int64_t)h * v.sh;
    }
    return (int64_t)b * v.sb + (int64_t)t * v.st + (int64_t)h * v.sh;
}

__device__ __forceinline__ u32x4 load16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// ---- LDS DMA (global_load_lds_dwordx4): lane i's 16 bytes land at lds + 16*i ---------
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kLoadNonTemporal = 2;   // cache-policy bit of the LDS DMA: rows read once

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): every LDS access of the wave has completed
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

}  // namespace dustin
