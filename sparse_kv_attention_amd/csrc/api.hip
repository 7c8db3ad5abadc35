// C-ABI entry points: host-side validation, workspace layout and kernel launches.
// Nothing here touches device memory or synchronises; every check uses host values only.
#include <stdlib.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "dustin.h"
#include "floor.hpp"
#include "kv.hpp"
#include "launch.hpp"

using namespace dustin;

// The scratch of dustin_sparse_verify_attn_noalloc: a device array in the library's code
// object (zero at load; each device holds its own copy until the process ends).  Host code
// never uses the name as an address: the device address comes from hipGetSymbolAddress,
// taken once per device on the first call made with that device current.
static __device__ __align__(256) unsigned char scratch[DUSTIN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A view is usable for `heads` KV heads and at least `min_tokens` tokens per sequence.
bool view_ok(const dustin_kv_view *v, int heads, int min_tokens)
{
    if (!v || !v->base || !aligned16(v->base))
        return false;
    if (v->stride_token <= 0 || v->stride_head < 0 || v->stride_batch < 0 || v->n_heads < heads)
        return false;
    if ((v->stride_token | v->stride_head | v->stride_batch | v->stride_page) & 7)
        return false;
    if (v->page_table) {
        if (v->page_size <= 0 || (v->page_size & (v->page_size - 1)) || v->max_pages <= 0 ||
            v->num_pages <= 0 || v->stride_page <= 0)
            return false;
        if ((int64_t)v->max_pages * v->page_size > (1ll << 30))
            return false;
        return v->max_pages * v->page_size >= min_tokens;
    }
    return v->n_tokens >= min_tokens && v->n_tokens > 0;
}

int view_cap(const dustin_kv_view *v)
{
    return v->page_table ? v->max_pages * v->page_size : v->n_tokens;
}

int env_int(const char *name, int dflt)
{
    const char *s = getenv(name);
    if (!s || !*s)
        return dflt;
    const int v = atoi(s);
    return v > 0 ? v : dflt;
}

// A 0/1 switch from the environment ("0" turns it off; unset or anything else keeps dflt
// unless it is "1").
bool env_flag(const char *name, bool dflt)
{
    const char *s = getenv(name);
    if (!s || !*s)
        return dflt;
    if (s[0] == '0' && s[1] == 0)
        return false;
    if (s[0] == '1' && s[1] == 0)
        return true;
    return dflt;
}

// Compute units of the current device (cached per device id).
int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Workgroups per round of the attention grid: one resident workgroup per CU (the
// per-wave rings take most of the LDS).  The split count is rounded so the grid is a
// whole number of rounds.
int attn_target_wgs()
{
    return env_int("DUSTIN_ATTN_TARGET_WGS", device_cus());
}

struct AttnWs {
    AttnPlan plan;
    size_t ctr_off, part_off, bytes;
};

// Positions one attention workgroup can hold.  Sparse lists and paged caches take their
// rows from each wave's LDS table (K and V rows sharing one table when they sit at the
// same places, else half each); dense unpaged calls compute rows from positions and
// take any length.
int attn_split_cap(bool table, bool two_tables)
{
    return !table ? kMaxList : (two_tables ? kSplitMax / 2 : kSplitMax);
}

AttnWs attn_workspace(int B, int Hq, int Hkv, int head_dim, int n_verify, int max_list, int split_cap)
{
    AttnWs w;
    const int G = Hq / Hkv;
    w.plan = plan_attn(B, Hkv, G, n_verify, head_dim, max_list, attn_target_wgs(), split_cap);
    w.ctr_off = 0;
    w.part_off = align_up(sizeof(unsigned long long) * w.plan.counters);
    w.bytes = w.part_off + align_up(sizeof(float) * w.plan.part_floats);
    return w;
}

// Workspace bytes valid for every table layout (the size queries do not see the views).
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int head_dim, int n_verify, int max_list, bool sparse)
{
    size_t m = std::max(attn_workspace(B, Hq, Hkv, head_dim, n_verify, max_list, attn_split_cap(true, false)).bytes,
                        attn_workspace(B, Hq, Hkv, head_dim, n_verify, max_list, attn_split_cap(true, true)).bytes);
    if (!sparse)
        m = std::max(m, attn_workspace(B, Hq, Hkv, head_dim, n_verify, max_list, attn_split_cap(false, false)).bytes);
    return m;
}

bool same_rows(const KvView &k, const KvView &v)
{
    return k.sb == v.sb && k.st == v.st && k.sp == v.sp && k.pt == v.pt && k.ps_log2 == v.ps_log2 &&
           k.max_pages == v.max_pages && k.num_pages == v.num_pages;
}

// Paged calls keep row numbers (element offset / stride_token) in 32 bits: every offset
// of the view must be a multiple of stride_token and the largest row number below 2^32.
bool rows_representable(const KvView &v, int B)
{
    if (v.pt)
        return v.rows_per_page >= 0 && (uint64_t)v.num_pages * (uint64_t)v.rows_per_page + (1ull << v.ps_log2) <= (1ull << 32);
    return v.rows_per_batch >= 0 && (uint64_t)B * (uint64_t)v.rows_per_batch + (uint64_t)v.cap <= (1ull << 32);
}

bool attn_shape_ok(int B, int Hq, int Hkv, int head_dim, int n_verify, dustin_status &st)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || n_verify <= 0) {
        st = DUSTIN_ERR_INVALID_ARG;
        return false;
    }
    if (Hq % Hkv) {
        st = DUSTIN_ERR_INVALID_ARG;
        return false;
    }
    if ((head_dim != 64 && head_dim != 128) || n_verify > 16 || Hq / Hkv * n_verify > 1024) {
        st = DUSTIN_ERR_UNSUPPORTED;
        return false;
    }
    return true;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

dustin_status scratch_of_current_device(void *stream, void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return DUSTIN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return DUSTIN_ERR_UNSUPPORTED;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return DUSTIN_ERR_HIP;
        if (sdev != dev)
            return DUSTIN_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return DUSTIN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DUSTIN_OK;
}

dustin_status run_attn(int B, int Hq, int Hkv, int head_dim, int n_verify, const void *q,
                       const dustin_kv_view *k, const dustin_kv_view *v, const int32_t *ctx_len,
                       const int32_t *idx, const int32_t *count, int k_max, int n_max,
                       float scale, void *out, float *lse, void *ws, size_t ws_bytes, void *stream,
                       bool use_scratch = false, float *logit2 = nullptr)
{
    dustin_status st = DUSTIN_OK;
    if (!attn_shape_ok(B, Hq, Hkv, head_dim, n_verify, st))
        return st;
    if (B == 0)
        return DUSTIN_OK;
    const bool sparse = idx != nullptr || count != nullptr;
    if (!q || !ctx_len || !out || !lse || !aligned16(q) || !aligned16(out))
        return DUSTIN_ERR_INVALID_ARG;
    if (sparse && (!idx || !count || k_max < 0))
        return DUSTIN_ERR_INVALID_ARG;
    if (n_max < 0 || !std::isfinite(scale))
        return DUSTIN_ERR_INVALID_ARG;
    if (!view_ok(k, Hkv, n_verify) || !view_ok(v, Hkv, n_verify))
        return DUSTIN_ERR_INVALID_ARG;
    const int cap = std::min(view_cap(k), view_cap(v));
    const int ctx_clamp = std::min(cap - n_verify, sparse ? cap - n_verify : n_max);
    // the split plan depends on host sizes only, exactly as in the workspace-size queries
    const int max_list = (sparse ? k_max : n_max) + n_verify;
    if (max_list > kMaxList)
        return DUSTIN_ERR_UNSUPPORTED;
    const KvView kv = make_view(*k), vv = make_view(*v);
    const bool kv_same = same_rows(kv, vv);
    const bool rows_mode = kv.pt != nullptr || vv.pt != nullptr;
    if (rows_mode && (!rows_representable(kv, B) || !rows_representable(vv, B)))
        return DUSTIN_ERR_UNSUPPORTED;
    const AttnWs lay = attn_workspace(B, Hq, Hkv, head_dim, n_verify, max_list,
                                      attn_split_cap(sparse || rows_mode, rows_mode && !kv_same));
    // the Collect-2 emission needs every query row of a (sequence, KV head) in one workgroup
    if (logit2 && lay.plan.qgroups != 1)
        return DUSTIN_ERR_UNSUPPORTED;
    if (use_scratch) {
        // every host check has passed: only now the scratch of the current device
        if (lay.bytes > DUSTIN_NOALLOC_SCRATCH_BYTES)
            return DUSTIN_ERR_SCRATCH;
        const dustin_status sst = scratch_of_current_device(stream, &ws);
        if (sst != DUSTIN_OK)
            return sst;
        ws_bytes = DUSTIN_NOALLOC_SCRATCH_BYTES;
    }
    if (lay.bytes > 0 && (!ws || ws_bytes < lay.bytes || !aligned16(ws)))
        return DUSTIN_ERR_WORKSPACE;

    AttnArgs a;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.nv = n_verify;
    a.GV = a.G * n_verify;
    a.q = static_cast<const uint16_t *>(q);
    a.k = kv;
    a.v = vv;
    a.kv_same = kv_same ? 1 : 0;
    a.rows_mode = rows_mode ? 1 : 0;
    a.ctx_len = ctx_len;
    a.idx = sparse ? idx : nullptr;
    a.count = sparse ? count : nullptr;
    a.k_max = sparse ? k_max : 0;
    a.ctx_clamp = ctx_clamp;
    a.scale_log2 = scale * kLog2e;
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.counter = reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + lay.ctr_off);
    a.part = reinterpret_cast<float *>(static_cast<char *>(ws) + lay.part_off);
    a.fused_merge = env_flag("DUSTIN_ATTN_FUSED_MERGE", false) ? 1 : 0;
    a.logit2 = logit2;
    a.scale = scale;
    a.splits = lay.plan.splits;
    a.spl = lay.plan.spl;
    a.qgroups = lay.plan.qgroups;
    a.pairs = lay.plan.pairs;
    const hipError_t e = launch_attn(a, head_dim, lay.plan.qt, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

struct ScoreWs {
    int n_pad, n_tiles, n_parts, total_pairs, logit_rows;
    size_t logits_off, max_off, tsum_off, pmax_off, psum_off, bytes;
};

int pairs_per_qhead(int n_q, int mode) { return mode == DUSTIN_SCORE_LOGIT_SUM2 ? std::min(2, n_q) : n_q; }

bool score_mode_ok(int mode)
{
    return mode == DUSTIN_SCORE_PROB_SUM || mode == DUSTIN_SCORE_LOGIT_SUM2 || mode == DUSTIN_SCORE_LOGIT_SUM_ALL;
}

ScoreWs score_workspace(int B, int n_max, int total_qheads, int n_q, int mode)
{
    ScoreWs w;
    w.n_pad = (n_max + 3) / 4 * 4;
    w.n_tiles = std::max(1, (n_max + kStatTile - 1) / kStatTile);
    // room for up to kScoreParts workgroup partials per pair; the launch picks how many
    const int n_ld = std::max(1, (n_max + kProbTile - 1) / kProbTile);
    w.n_parts = std::min(kScoreParts, n_ld);
    w.total_pairs = total_qheads * pairs_per_qhead(n_q, mode);
    const bool prob = mode == DUSTIN_SCORE_PROB_SUM;
    // logit-sum modes keep one row per group (a group has at least one query head)
    w.logit_rows = prob ? w.total_pairs : total_qheads;
    const size_t stats = prob ? (size_t)B * w.total_pairs * w.n_tiles : 0;
    const size_t parts = prob ? (size_t)B * w.total_pairs * w.n_parts : 0;
    w.logits_off = 0;
    w.max_off = align_up(sizeof(float) * (size_t)B * w.logit_rows * w.n_pad);
    w.tsum_off = w.max_off + align_up(sizeof(double) * stats);
    w.pmax_off = w.tsum_off + align_up(sizeof(double) * stats);
    w.psum_off = w.pmax_off + align_up(sizeof(double) * parts);
    w.bytes = w.psum_off + align_up(sizeof(double) * parts);
    return w;
}

}  // namespace

extern "C" {

const char *dustin_status_string(dustin_status s)
{
    switch (s) {
    case DUSTIN_OK: return "ok";
    case DUSTIN_ERR_INVALID_ARG: return "invalid argument";
    case DUSTIN_ERR_WORKSPACE: return "workspace missing or too small";
    case DUSTIN_ERR_UNSUPPORTED: return "unsupported shape";
    case DUSTIN_ERR_HIP: return "HIP launch error";
    case DUSTIN_ERR_SCRATCH: return "needs more than the library's static scratch array";
    }
    return "unknown status";
}

dustin_status dustin_srh_score_workspace_size(int B, int n_max, int total_qheads, int n_q, int mode,
                                              size_t *bytes)
{
    if (!bytes || B < 0 || n_max < 0 || total_qheads < 0 || n_q <= 0 || n_q > 16 || !score_mode_ok(mode))
        return DUSTIN_ERR_INVALID_ARG;
    *bytes = score_workspace(B, n_max, total_qheads, n_q, mode).bytes;
    return DUSTIN_OK;
}

namespace {

// Host checks of one signal: sizes, mode, groups; its query heads and widest group.
dustin_status check_signal(const dustin_srh_signal &sg, int &total_qheads, int &max_pairs, int &ctx_clamp, int n_max)
{
    if (sg.n_q <= 0 || !std::isfinite(sg.scale) || !score_mode_ok(sg.mode) || sg.n_groups < 1 || !sg.groups)
        return DUSTIN_ERR_INVALID_ARG;
    if (sg.n_groups > kMaxGroups || (sg.head_dim != 64 && sg.head_dim != 128) || sg.n_q > 16)
        return DUSTIN_ERR_UNSUPPORTED;
    const int ppq = pairs_per_qhead(sg.n_q, sg.mode);
    total_qheads = 0;
    max_pairs = 0;
    ctx_clamp = n_max;
    for (int i = 0; i < sg.n_groups; ++i) {
        const dustin_srh_group &g = sg.groups[i];
        if (g.n_qheads <= 0 || g.kv_head < 0 || !view_ok(&g.k, g.kv_head + 1, 1))
            return DUSTIN_ERR_INVALID_ARG;
        if (g.n_qheads * ppq > (sg.mode == DUSTIN_SCORE_PROB_SUM ? kMaxProbPairsPerGroup : kMaxPairsPerGroup))
            return DUSTIN_ERR_UNSUPPORTED;
        total_qheads += g.n_qheads;
        max_pairs = std::max(max_pairs, g.n_qheads * ppq);
        ctx_clamp = std::min(ctx_clamp, view_cap(&g.k));
    }
    return DUSTIN_OK;
}

// Workspace of a set of signals: each signal's layout, one after the other.
size_t signals_workspace(int B, int n_max, int n_sig, const dustin_srh_signal *sigs, size_t *offs)
{
    size_t off = 0;
    for (int s = 0; s < n_sig; ++s) {
        int tq = 0;
        for (int i = 0; i < sigs[s].n_groups; ++i)
            tq += sigs[s].groups[i].n_qheads;
        if (offs)
            offs[s] = off;
        off += align_up(score_workspace(B, n_max, tq, sigs[s].n_q, sigs[s].mode).bytes);
    }
    return off;
}

dustin_status run_score(int B, int n_max, const int32_t *ctx_len, int n_sig, const dustin_srh_signal *sigs,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || n_max < 0 || n_sig < 1 || n_sig > kMaxSignals || !sigs)
        return DUSTIN_ERR_INVALID_ARG;
    int tq[kMaxSignals], mp[kMaxSignals], cc[kMaxSignals], groups = 0;
    for (int s = 0; s < n_sig; ++s) {
        const dustin_status st = check_signal(sigs[s], tq[s], mp[s], cc[s], n_max);
        if (st != DUSTIN_OK)
            return st;
        groups += sigs[s].n_groups;
    }
    if (groups > kMaxGroups)
        return DUSTIN_ERR_UNSUPPORTED;
    if (B == 0 || n_max == 0)
        return DUSTIN_OK;
    if (!ctx_len)
        return DUSTIN_ERR_INVALID_ARG;
    for (int s = 0; s < n_sig; ++s)
        if (!sigs[s].q || !sigs[s].score || !aligned16(sigs[s].q) || !aligned16(sigs[s].score))
            return DUSTIN_ERR_INVALID_ARG;
    size_t offs[kMaxSignals];
    const size_t need = signals_workspace(B, n_max, n_sig, sigs, offs);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return DUSTIN_ERR_WORKSPACE;

    ScoreArgs a;
    a.B = B;
    a.n_max = n_max;
    a.n_sig = n_sig;
    a.prob_g0 = 0;
    a.ctx_len = ctx_len;
    int g0 = 0;
    for (int s = 0; s < n_sig; ++s) {
        const dustin_srh_signal &in = sigs[s];
        const ScoreWs lay = score_workspace(B, n_max, tq[s], in.n_q, in.mode);
        char *base = static_cast<char *>(workspace) + offs[s];
        a.n_pad = lay.n_pad;       // the same for every signal (n_max)
        a.n_tiles = lay.n_tiles;
        a.n_parts = lay.n_parts;   // the most the workspace holds; the launch picks its count
        ScoreSig &S = a.sig[s];
        S.n_groups = in.n_groups;
        S.g0 = g0;
        S.n_q = in.n_q;
        S.mode = in.mode;
        S.total_qheads = tq[s];
        S.total_pairs = lay.total_pairs;
        S.head_dim = in.head_dim;
        S.ctx_clamp = cc[s];
        S.logit_rows = in.mode == DUSTIN_SCORE_PROB_SUM ? lay.total_pairs : in.n_groups;
        S.q = static_cast<const uint16_t *>(in.q);
        S.mul = in.mode == DUSTIN_SCORE_PROB_SUM ? (double)in.scale * 1.4426950408889634 : (double)in.scale;
        S.logits = reinterpret_cast<float *>(base + lay.logits_off);
        S.tile_max = reinterpret_cast<double *>(base + lay.max_off);
        S.tile_sum = reinterpret_cast<double *>(base + lay.tsum_off);
        S.part_max = reinterpret_cast<double *>(base + lay.pmax_off);
        S.part_sum = reinterpret_cast<double *>(base + lay.psum_off);
        S.score = in.score;
        const int ppq = pairs_per_qhead(in.n_q, in.mode);
        int qh = 0, pr = 0;
        for (int i = 0; i < in.n_groups; ++i) {
            ScoreGroup &sg = a.grp[g0 + i];
            sg.k = make_view(in.groups[i].k);
            sg.kv_head = in.groups[i].kv_head;
            sg.sig = s;
            sg.q_head0 = qh;
            sg.n_qheads = in.groups[i].n_qheads;
            sg.pair0 = pr;
            sg.n_pairs = in.groups[i].n_qheads * ppq;
            qh += sg.n_qheads;
            pr += sg.n_pairs;
        }
        g0 += in.n_groups;
    }
    const hipError_t e = launch_score(a, device_cus(), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

}  // namespace

dustin_status dustin_srh_score(int B, int n_max, const int32_t *ctx_len, int n_groups,
                               const dustin_srh_group *groups, int head_dim, const void *q, int n_q,
                               float scale, int mode, float *score, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    dustin_srh_signal sg;
    sg.n_groups = n_groups;
    sg.groups = groups;
    sg.head_dim = head_dim;
    sg.q = q;
    sg.n_q = n_q;
    sg.scale = scale;
    sg.mode = mode;
    sg.score = score;
    return run_score(B, n_max, ctx_len, 1, &sg, workspace, workspace_bytes, stream);
}

dustin_status dustin_srh_score_signals_workspace_size(int B, int n_max, int n_signals,
                                                      const dustin_srh_signal *signals, size_t *bytes)
{
    if (!bytes || B < 0 || n_max < 0 || n_signals < 1 || n_signals > kMaxSignals || !signals)
        return DUSTIN_ERR_INVALID_ARG;
    int groups = 0;
    for (int s = 0; s < n_signals; ++s) {
        int tq, mp, cc;
        const dustin_status st = check_signal(signals[s], tq, mp, cc, n_max);
        if (st != DUSTIN_OK)
            return st;
        groups += signals[s].n_groups;
    }
    if (groups > kMaxGroups)
        return DUSTIN_ERR_UNSUPPORTED;
    *bytes = signals_workspace(B, n_max, n_signals, signals, nullptr);
    return DUSTIN_OK;
}

dustin_status dustin_srh_score_signals(int B, int n_max, const int32_t *ctx_len, int n_signals,
                                       const dustin_srh_signal *signals, void *workspace,
                                       size_t workspace_bytes, void *stream)
{
    return run_score(B, n_max, ctx_len, n_signals, signals, workspace, workspace_bytes, stream);
}

dustin_status dustin_select_workspace_size(int B, int n_max, size_t *bytes)
{
    if (!bytes || B < 0 || n_max < 0)
        return DUSTIN_ERR_INVALID_ARG;
    // the two tiers' chosen-position masks and an arrival counter for every sequence
    *bytes = select_ws_bytes(B);
    return DUSTIN_OK;
}

dustin_status dustin_select(int B, int n_max, const int32_t *ctx_len, const float *score_draft,
                            const float *score_target, const int32_t *budget,
                            const int32_t *n_sink, const int32_t *n_window, const int32_t *m,
                            int k_max, int32_t *idx, int32_t *count, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    if (B < 0 || n_max < 0 || k_max < 0)
        return DUSTIN_ERR_INVALID_ARG;
    if (n_max > kSelectMaxN)
        return DUSTIN_ERR_UNSUPPORTED;
    if (B == 0)
        return DUSTIN_OK;
    if (!ctx_len || !score_target || !budget || !n_sink || !n_window || !m || !count ||
        (k_max > 0 && !idx))
        return DUSTIN_ERR_INVALID_ARG;
    // the kernels read score rows as 16-byte vectors
    if (!aligned16(score_target) || (score_draft && !aligned16(score_draft)))
        return DUSTIN_ERR_INVALID_ARG;
    // no workspace: one workgroup per sequence runs both tiers in turn
    if (workspace && (workspace_bytes < select_ws_bytes(B) || !aligned16(workspace)))
        return DUSTIN_ERR_WORKSPACE;
    SelectArgs a;
    a.B = B;
    a.n_max = n_max;
    a.k_max = k_max;
    a.ctx_len = ctx_len;
    a.score_draft = score_draft;
    a.score_target = score_target;
    a.budget = budget;
    a.n_sink = n_sink;
    a.n_window = n_window;
    a.m = m;
    a.idx = idx;
    a.count = count;
    a.ws = static_cast<unsigned long long *>(workspace);
    const hipError_t e = launch_select(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

dustin_status dustin_sparse_verify_attn_workspace_size(int B, int Hq, int Hkv, int head_dim,
                                                       int n_verify, int k_max, size_t *bytes)
{
    dustin_status st = DUSTIN_OK;
    if (!bytes || k_max < 0)
        return DUSTIN_ERR_INVALID_ARG;
    if (!attn_shape_ok(B, Hq, Hkv, head_dim, n_verify, st))
        return st;
    if (k_max + n_verify > kMaxList)
        return DUSTIN_ERR_UNSUPPORTED;
    *bytes = attn_workspace_bytes(B, Hq, Hkv, head_dim, n_verify, k_max + n_verify, true);
    return DUSTIN_OK;
}

dustin_status dustin_sparse_verify_attn(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                        const void *q, const dustin_kv_view *k,
                                        const dustin_kv_view *v, const int32_t *ctx_len,
                                        const int32_t *idx, const int32_t *count, int k_max,
                                        float scale, void *out, float *lse, void *workspace,
                                        size_t workspace_bytes, void *stream)
{
    if (!idx || !count)
        return DUSTIN_ERR_INVALID_ARG;
    return run_attn(B, Hq, Hkv, head_dim, n_verify, q, k, v, ctx_len, idx, count, k_max, 0, scale,
                    out, lse, workspace, workspace_bytes, stream);
}

dustin_status dustin_sparse_verify_attn_noalloc(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                                const void *q, const dustin_kv_view *k,
                                                const dustin_kv_view *v, const int32_t *ctx_len,
                                                const int32_t *idx, const int32_t *count, int k_max,
                                                float scale, void *out, float *lse, void *stream)
{
    size_t need = 0;
    const dustin_status st = dustin_sparse_verify_attn_workspace_size(B, Hq, Hkv, head_dim, n_verify, k_max, &need);
    if (st != DUSTIN_OK)
        return st;
    if (need > DUSTIN_NOALLOC_SCRATCH_BYTES)
        return DUSTIN_ERR_SCRATCH;
    if (!idx || !count)
        return DUSTIN_ERR_INVALID_ARG;
    return run_attn(B, Hq, Hkv, head_dim, n_verify, q, k, v, ctx_len, idx, count, k_max, 0, scale,
                    out, lse, nullptr, 0, stream, true);
}

dustin_status dustin_sparse_verify_attn_logits(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                               const void *q, const dustin_kv_view *k,
                                               const dustin_kv_view *v, const int32_t *ctx_len,
                                               const int32_t *idx, const int32_t *count, int k_max,
                                               float scale, void *out, float *lse, float *logit_sum2,
                                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (!idx || !count || !logit_sum2 || (reinterpret_cast<uintptr_t>(logit_sum2) & 3u))
        return DUSTIN_ERR_INVALID_ARG;
    return run_attn(B, Hq, Hkv, head_dim, n_verify, q, k, v, ctx_len, idx, count, k_max, 0, scale,
                    out, lse, workspace, workspace_bytes, stream, false, logit_sum2);
}

dustin_status dense_verify_attn_workspace_size(int B, int Hq, int Hkv, int head_dim, int n_verify,
                                               int n_max, size_t *bytes)
{
    dustin_status st = DUSTIN_OK;
    if (!bytes || n_max < 0)
        return DUSTIN_ERR_INVALID_ARG;
    if (!attn_shape_ok(B, Hq, Hkv, head_dim, n_verify, st))
        return st;
    if (n_max + n_verify > kMaxList)
        return DUSTIN_ERR_UNSUPPORTED;
    *bytes = attn_workspace_bytes(B, Hq, Hkv, head_dim, n_verify, n_max + n_verify, false);
    return DUSTIN_OK;
}

dustin_status dense_verify_attn(int B, int Hq, int Hkv, int head_dim, int n_verify, const void *q,
                                const dustin_kv_view *k, const dustin_kv_view *v,
                                const int32_t *ctx_len, int n_max, float scale, void *out,
                                float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    return run_attn(B, Hq, Hkv, head_dim, n_verify, q, k, v, ctx_len, nullptr, nullptr, 0, n_max,
                    scale, out, lse, workspace, workspace_bytes, stream);
}

dustin_status dustin_attn_plan(int B, int Hq, int Hkv, int head_dim, int n_verify, int n_positions, int layout,
                               int32_t *plan)
{
    dustin_status st = DUSTIN_OK;
    if (!plan || n_positions < 0 || layout < 0 || layout > 2)
        return DUSTIN_ERR_INVALID_ARG;
    if (!attn_shape_ok(B, Hq, Hkv, head_dim, n_verify, st))
        return st;
    if (n_positions + n_verify > kMaxList)
        return DUSTIN_ERR_UNSUPPORTED;
    const AttnWs lay = attn_workspace(B, Hq, Hkv, head_dim, n_verify, n_positions + n_verify,
                                      attn_split_cap(layout != 2, layout == 1));
    plan[0] = lay.plan.qt;
    plan[1] = lay.plan.qgroups;
    plan[2] = lay.plan.splits;
    plan[3] = (int32_t)lay.plan.grid;
    plan[4] = lay.plan.splits == 1 ? 0 : (env_flag("DUSTIN_ATTN_FUSED_MERGE", false) ? 2 : 1);
    return DUSTIN_OK;
}

dustin_status dustin_gather_floor(int B, int Hkv, int head_dim, const dustin_kv_view *k, const dustin_kv_view *v,
                                  const int32_t *idx, int k_max, uint32_t *checksum, int mode, void *stream)
{
    if (B < 0 || Hkv <= 0 || k_max < 0 || (mode != 0 && mode != 1))
        return DUSTIN_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128)
        return DUSTIN_ERR_UNSUPPORTED;
    if (B == 0 || k_max == 0)
        return DUSTIN_OK;
    if (!idx || !checksum || ((uintptr_t)checksum & 3))
        return DUSTIN_ERR_INVALID_ARG;
    if (!view_ok(k, Hkv, 1) || !view_ok(v, Hkv, 1))
        return DUSTIN_ERR_INVALID_ARG;
    if (k->page_table || v->page_table)
        return DUSTIN_ERR_UNSUPPORTED;
    const int splits = (k_max + kFloorPositions - 1) / kFloorPositions;
    if ((int64_t)B * splits * Hkv > 0x7fffffff)
        return DUSTIN_ERR_UNSUPPORTED;
    FloorArgs a;
    a.B = B;
    a.Hkv = Hkv;
    a.k_max = k_max;
    a.n_tok = std::min(k->n_tokens, v->n_tokens);
    a.splits = splits;
    a.k = static_cast<const uint16_t *>(k->base);
    a.v = static_cast<const uint16_t *>(v->base);
    a.k_sb = k->stride_batch;
    a.k_st = k->stride_token;
    a.k_sh = k->stride_head;
    a.v_sb = v->stride_batch;
    a.v_st = v->stride_token;
    a.v_sh = v->stride_head;
    a.idx = idx;
    a.checksum = checksum;
    a.mode = mode;
    const hipError_t e = launch_gather_floor(a, head_dim, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

dustin_status dustin_kv_write_block(int B, int Hkv, int head_dim, int n_new, const void *k_new,
                                    const void *v_new, const int32_t *ctx_len, const dustin_kv_view *k,
                                    const dustin_kv_view *v, void *stream)
{
    if (B < 0 || Hkv <= 0 || n_new <= 0)
        return DUSTIN_ERR_INVALID_ARG;
    if ((head_dim != 64 && head_dim != 128) || n_new > kMaxNewRows)
        return DUSTIN_ERR_UNSUPPORTED;
    if (B == 0)
        return DUSTIN_OK;
    if (!k_new || !v_new || !ctx_len || !aligned16(k_new) || !aligned16(v_new))
        return DUSTIN_ERR_INVALID_ARG;
    if (!view_ok(k, Hkv, n_new) || !view_ok(v, Hkv, n_new))
        return DUSTIN_ERR_INVALID_ARG;
    KvWriteArgs a;
    a.B = B;
    a.Hkv = Hkv;
    a.n_new = n_new;
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.k = make_view(*k);
    a.v = make_view(*v);
    a.ctx_len = ctx_len;
    a.ctx_clamp = std::min(view_cap(k), view_cap(v)) - n_new;
    const hipError_t e = launch_kv_write_block(a, head_dim, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

dustin_status dustin_kv_commit(int B, int n_new, const int32_t *n_accept, int32_t *ctx_len, void *stream)
{
    if (B < 0 || n_new <= 0)
        return DUSTIN_ERR_INVALID_ARG;
    if (n_new > kMaxNewRows)
        return DUSTIN_ERR_UNSUPPORTED;
    if (B == 0)
        return DUSTIN_OK;
    if (!n_accept || !ctx_len)
        return DUSTIN_ERR_INVALID_ARG;
    const hipError_t e = launch_kv_commit(B, n_new, n_accept, ctx_len, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

dustin_status dustin_attn_recovery(int n, const float *lse_sparse, const float *lse_dense, float *rec,
                                   void *stream)
{
    if (n < 0)
        return DUSTIN_ERR_INVALID_ARG;
    if (n == 0)
        return DUSTIN_OK;
    if (!lse_sparse || !lse_dense || !rec)
        return DUSTIN_ERR_INVALID_ARG;
    const hipError_t e = launch_attn_recovery(n, lse_sparse, lse_dense, rec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DUSTIN_OK : DUSTIN_ERR_HIP;
}

}  // extern "C"
