// Launch interface of the gather-floor measurement kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dustin {

constexpr int kFloorPositions = 512;   // list entries per workgroup

struct FloorArgs {
    int B, Hkv, k_max, n_tok, splits;  // splits = ceil(k_max / kFloorPositions)
    const uint16_t *k, *v;             // unpaged views
    int64_t k_sb, k_st, k_sh, v_sb, v_st, v_sh;
    const int32_t *idx;                // [B][k_max]
    uint32_t *checksum;                // [B][Hkv]
    int mode;                          // 0: timing, 1: XOR of the words read into checksum
};

hipError_t launch_gather_floor(const FloorArgs &a, int head_dim, hipStream_t st);

}  // namespace dustin
