// Kernel launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device.hpp"

namespace dustin {

// ---------------------------------------------------------------- attention
constexpr int kMaxQT = 5;          // 16-row query tiles held by one workgroup
constexpr int kAttnStepsMaxW = 16; // 32-position steps of one wave whose list entries (or row
                                   // numbers) the wave's LDS table holds
constexpr int kSplitMax = 4 * kAttnStepsMaxW * 32;   // positions of one workgroup when its steps
                                   // come from the table (sparse lists, paged caches); half as
                                   // many when K and V rows need a table each
constexpr int kMaxSplits = 256;    // splits of one (sequence, KV head, query group)
constexpr int kMaxList = 131072;   // longest list (selected positions + new tokens) accepted

struct AttnArgs {
    int B, Hq, Hkv, G, nv, GV;
    const uint16_t *q;
    KvView k, v;
    int kv_same;             // K and V rows of a token sit at the same element offsets
    int rows_mode;           // K or V paged: rows resolved through the page tables once
    const int32_t *ctx_len;
    const int32_t *idx;      // nullptr = dense: the list is [0, ctx_len[b])
    const int32_t *count;
    int k_max;
    int ctx_clamp;           // ctx_len is clamped to [0, ctx_clamp]
    float scale_log2;        // softmax scale * log2(e)
    uint16_t *out;
    float *lse;
    float *part;             // split partials
    unsigned long long *counter;   // per pair: arrivals of its splits (fused merge)
    int fused_merge;         // splits merged by their last arrival (else by a second kernel)
    float *logit2;           // optional [B][Hkv][k_max]: per selected token, scale * q.k summed over
                             //   the KV head's query heads and verify queries {0, n_verify-1}
    float scale;             // softmax scale (natural-log logits of logit2)
    int splits, spl, qgroups, pairs;   // spl: list positions per split; pairs = B*Hkv*qgroups
};

struct AttnPlan {
    int qt, qgroups, pairs, splits, spl;
    size_t part_floats;      // split partial records
    size_t counters;         // per-pair arrival counters
    size_t grid;
};

AttnPlan plan_attn(int B, int Hkv, int G, int nv, int head_dim, int max_list, int target_wgs, int split_cap);
hipError_t launch_attn(const AttnArgs &a, int head_dim, int qt, hipStream_t st);

// ---------------------------------------------------------------- scoring
constexpr int kMaxGroups = 16;
constexpr int kMaxPairsPerGroup = 64;       // logit-sum mode
constexpr int kMaxProbPairsPerGroup = 16;   // softmax mode
constexpr int kProbTile = 256;    // tokens per workgroup of the softmax-mode logit kernel
constexpr int kStatTile = 64;     // tokens per statistics tile (one maximum per pair)
constexpr int kScoreParts = 64;   // most workgroups per (group, sequence) of the softmax-mode logit kernel

struct ScoreGroup {
    KvView k;
    int kv_head;
    int sig;          // the signal the group belongs to
    int q_head0;      // first query head of the group in the signal's q
    int n_qheads;
    int pair0;        // first pair of the group in the signal's logit workspace
    int n_pairs;
    int parts;        // softmax mode: workgroups per sequence sharing the group's tiles
    int wg0;          // softmax mode: first workgroup of the group (then b * parts + part)
};

// One scored signal (draft lookahead or target historical queries).
struct ScoreSig {
    int n_groups, g0;        // its groups: grp[g0 .. g0 + n_groups)
    int n_q, mode, total_qheads, total_pairs, head_dim, ctx_clamp;
    int logit_rows;          // rows per sequence of `logits`: total_pairs (PROB_SUM), n_groups
    const uint16_t *q;
    double mul;              // PROB_SUM: scale*log2(e) (base-2 logits); logit sums: scale
    float *logits;           // [B][logit_rows][n_pad]: PROB_SUM l - tile max per pair; logit-sum
                             //   modes: per group, the sum of its pairs' logits
    double *tile_max;        // PROB_SUM: [B][total_pairs][n_tiles], n_tiles = ceil(n_max / kStatTile)
    double *tile_sum;        // PROB_SUM: [B][total_pairs][n_tiles], sum of exp2(l - tile max)
    double *part_max;        // PROB_SUM: [B][total_pairs][n_parts], one (max, sum of exp2(l - max))
    double *part_sum;        //   per workgroup of the logit kernel
    float *score;            // [B][n_max]
};

constexpr int kMaxSignals = 2;

struct ScoreArgs {
    int B, n_max, n_pad, n_tiles, n_parts, n_sig;
    int prob_g0, prob_ng;    // the softmax-mode launch covers grp[prob_g0 .. prob_g0 + prob_ng)
    const int32_t *ctx_len;
    ScoreSig sig[kMaxSignals];
    ScoreGroup grp[kMaxGroups];
};

// cus: compute units of the device (sizes the softmax-mode grid to one resident round)
hipError_t launch_score(ScoreArgs a, int cus, hipStream_t st);

// ---------------------------------------------------------------- selection
constexpr int kSelectThreads = 1024;
constexpr int kSelectMaxN = 65536;

struct SelectArgs {
    int B, n_max, k_max;
    const int32_t *ctx_len;
    const float *score_draft;   // may be nullptr: no draft tier
    const float *score_target;
    const int32_t *budget, *n_sink, *n_window, *m;
    int32_t *idx, *count;
    unsigned long long *ws;     // [B][2][kSelectThreads] chosen-position masks of the two tiers,
                                //   then [B] arrival counters (nullptr: one workgroup per
                                //   sequence runs both tiers)
};
constexpr int kSelectCombineCap = 4096;   // r + m up to which the tiers run on two workgroups

// bytes of the selection workspace for B sequences: the masks and the counters
inline size_t select_ws_bytes(int B)
{
    return (size_t)B * (2 * kSelectThreads + 1) * sizeof(unsigned long long);
}

hipError_t launch_select(const SelectArgs &a, hipStream_t st);

}  // namespace dustin
