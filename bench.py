"""Benchmark of one sparse-verification step on one MI355X.

Workload: Qwen2.5-72B-shaped target (80 layers, 64 query heads, 8 KV heads, head dim
128, bf16), batch 8, 32768-token contexts, gamma = 4 (5 verify queries), budget 2048
(16 sinks, 256 window, m = 768), 4 draft + 4 target SRH streams.  All inputs are seeded
synthetic tensors resident in HBM before timing starts; every layer has its own K/V
buffers (86 GB in total), so no layer's gathered rows are served from the last-level
cache by an earlier layer.

One step = draft-SRH scoring + target-SRH scoring + selection + sparse verification
attention over all 80 layers.  `value` is the step's algorithmic HBM bytes divided by
the step time (GB/s); the step time itself is `step_us`.  The roofline entry is for the
dominant call, the sparse verification attention of one layer (a split kernel and, when
the list is split, a merge kernel): its algorithmic bytes per call divided by its average
duration, timed with HIP events on the stream it runs on.  `traffic` is the measured
HBM bytes per call (FETCH_SIZE + WRITE_SIZE counters, calibrated on a copy of known
size) from the committed counter summary, and null when the kernel source has changed
since those counters were taken.

`--counters` runs only a calibration copy and the attention calls, for counter passes.
`--estimator-sweep` times the naive all-heads estimator, dense attention and the SRH
scoring at contexts 1k..64k instead of the step (one JSON line of its own).
`--sweep` times sparse against dense attention (and each point's scoring and selection)
on one 72B-shaped layer at batch 64 over budgets 1024..4096 and gamma 2..8.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-verify step µs + achieved HBM GB/s (B=8, 32k ctx, budget 2048, γ=4)"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_qwen72b_b8_n32768_traffic.md")
ATTN_SOURCES = [os.path.join(ROOT, "sparse_kv_attention_amd", "csrc", f) for f in ("attn.hip", "launch.hpp", "device.hpp")]
CALIB_BYTES = 256 << 20


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention call from the committed counter summary, if it was taken
    on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    d = json.loads(line[len("traffic-json: "):])
                    if d.get("source_sha256_16") == attn_source_hash():
                        return d["bytes_per_call"]
    except OSError:
        pass
    return None


def attn_bytes(B, Hq, Hkv, d, nv, counts):
    """Algorithmic bytes of one verification-attention launch: the gathered K and V rows
    of the selected tokens and of the new block, Q, O, LSE and the index list."""
    rows = sum(int(c) + nv for c in counts)
    return rows * Hkv * d * 2 * 2 + 2 * B * nv * Hq * d * 2 + B * Hq * nv * 4 + sum(int(c) for c in counts) * 4


def score_bytes(B, n_ctx, streams_d, n_out):
    """Algorithmic bytes of scoring: every scored K row once, and the score vectors."""
    return sum(B * n_ctx * d * 2 for d in streams_d) + n_out * B * n_ctx * 4


def select_bytes(B, n_ctx, k):
    return 2 * B * n_ctx * 4 + B * k * 4 + B * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=80, help="target layers (80 = the whole 72B-shaped model)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--dense-layers", type=int, default=80,
                    help="layers of dense attention timed (all of them by default)")
    ap.add_argument("--counters", action="store_true", help="calibration copy + attention calls only")
    ap.add_argument("--estimator-sweep", action="store_true",
                    help="naive all-heads estimator vs dense attention vs SRH scoring, context 1k..64k")
    ap.add_argument("--sweep", action="store_true",
                    help="one 72B-shaped layer at B=64, 32k: sparse vs dense attention per (budget, gamma)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the sparse-verification path here is a single-GPU build)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_kv_attention_amd import workloads as W
    from sparse_kv_attention_amd.pipeline import SparseVerifyStep

    dev = torch.device("cuda:0")
    if args.estimator_sweep:
        estimator_sweep(dev, args)
        return
    if args.sweep:
        attention_sweep(dev, args)
        return
    w = W.QWEN72B
    if args.layers != w.target.layers:
        w = W.shrink(w, target=W.ModelShape(args.layers, w.target.hq, w.target.hkv, w.target.d),
                     srh_target=tuple((l % args.layers, h) for l, h in w.srh_target))
    t0 = time.time()
    inp = W.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s: {len(inp.k_cache)} layers", file=sys.stderr, flush=True)
    step = SparseVerifyStep(inp)
    T = w.target
    B, nv = w.batch, w.n_verify
    stream = torch.cuda.current_stream()

    if args.counters:
        # a plain copy of CALIB_BYTES (read CALIB_BYTES, write CALIB_BYTES), then ten
        # distinct-layer attention calls and the gather floor on the same ten layers
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        step.score()
        step.select()
        for l in step.layers[:10]:
            step.attn(l)
        from sparse_kv_attention_amd import dustin as D
        fl_idx = step.idx[:, :inp.k_max].contiguous()
        fl_ck = torch.zeros((B, T.hkv), dtype=torch.int32, device=dev)
        for l in step.layers[:10]:
            k, v = step.kv[l]
            D.dustin_gather_floor(k, v, T.hkv, T.d, fl_idx, fl_ck)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "calib_bytes": CALIB_BYTES, "attn_calls": 10,
                          "attn_source_sha256_16": attn_source_hash()}), flush=True)
        return

    # ---- warmup ----
    for _ in range(args.warmup):
        step.step()
    torch.cuda.synchronize()
    counts = step.count.cpu().tolist()

    # ---- timed steps (an event between consecutive steps gives each step's time) ----
    ev = lambda: torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    evs_step = [ev() for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    evs_step[0].record(stream)
    for i in range(args.steps):
        step.step()
        evs_step[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = evs_step[0].elapsed_time(evs_step[-1]) / args.steps
    per_step_us = [evs_step[i].elapsed_time(evs_step[i + 1]) * 1e3 for i in range(args.steps)]

    # ---- per-stage and per-launch timing (separate loops, same stream) ----
    def timed(fn, reps):
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    def timed_each(fn, reps):
        """Per-repetition times (µs): an event between consecutive repetitions."""
        es = [ev() for _ in range(reps + 1)]
        torch.cuda.synchronize()
        es[0].record(stream)
        for i in range(reps):
            fn()
            es[i + 1].record(stream)
        torch.cuda.synchronize()
        return [es[i].elapsed_time(es[i + 1]) * 1e3 for i in range(reps)]

    reps = max(10, args.steps // 2)
    t_score = timed_each(step.score, reps)
    t_select = timed_each(step.select, reps)
    us_score = float(np.mean(t_score))
    us_select = float(np.mean(t_select))
    attn_layers = step.layers
    # every attention launch bracketed by its own events on the launch stream
    durs = []
    for _ in range(reps):
        evs = [(ev(), ev()) for _ in attn_layers]
        for (a, b), l in zip(evs, attn_layers):
            a.record(stream)
            step.attn(l)
            b.record(stream)
        torch.cuda.synchronize()
        durs += [a.elapsed_time(b) * 1e3 for a, b in evs]
    us_attn_launch = float(np.mean(durs))
    t_attn_all = timed_each(lambda: [step.attn(l) for l in attn_layers], reps)
    us_attn_all = float(np.mean(t_attn_all))
    # the same calls also writing the Collect-2 logit sums of the selected tokens (every KV
    # head of every layer) as a by-product of verification
    lg2 = torch.empty((B, T.hkv, inp.k_max), dtype=torch.float32, device=dev)
    t_attn_lg = timed_each(lambda: [step.attn_logits(l, lg2) for l in attn_layers], reps)
    us_attn_lg = float(np.mean(t_attn_lg)) / len(attn_layers)
    dl = attn_layers[: max(1, min(args.dense_layers, len(attn_layers)))]
    t_dense_all = timed_each(lambda: [step.dense(l) for l in dl], 3)
    us_dense_all = float(np.mean(t_dense_all))
    us_dense_layer = us_dense_all / len(dl)
    # Vegas-style target signal on the same streams (raw logits summed over the first and
    # bonus queries, or over every query) and its pure top-k selection: not part of the step
    variants = {}
    for name, kw in (("vegas_collect2", {"logit_sum2": True}), ("vegas_all_queries", {"logit_sum_all": True})):
        vs = SparseVerifyStep(inp, layers=attn_layers[:1], **kw)
        vs.score()
        vs.select()
        us_v = timed(vs.score, reps)
        variants[name] = {"score_us": round(us_v, 2),
                          "score_gbs": round(score_bytes(B, inp.n_max, [T.d] * len(inp.target_groups), 1)
                                             / (us_v * 1e-6) / 1e9, 1),
                          "topk_select_us": round(timed(vs.select, reps), 2)}
        del vs

    # Verification workflow step 5 and the draft phase around the step (not part of it):
    # the verified block written into every layer's caches, the commit, and sparse
    # attention with a single query (the sparse draft phase of the Vegas summary) on the
    # same caches and selected set
    from sparse_kv_attention_amd import dustin as D
    g = torch.Generator(device=dev).manual_seed(1234)
    kn = torch.randn((B, nv, T.hkv, T.d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, nv, T.hkv, T.d), generator=g, device=dev).to(torch.bfloat16)
    # the block rows are rewritten with themselves, so the caches stay as generated
    ctxl = inp.ctx_len.cpu().tolist()
    for b in range(B):
        kn[b] = inp.k_cache[attn_layers[0]][b, ctxl[b]:ctxl[b] + nv]
        vn[b] = inp.v_cache[attn_layers[0]][b, ctxl[b]:ctxl[b] + nv]
    # these calls take a few µs of GPU time, less than their host-side launch cost, so they
    # are timed as replays of a captured HIP graph of 80 back-to-back calls
    def graph_timed(fn, n_calls=80, replays=10):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(n_calls):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        return timed(graph.replay, replays) / n_calls

    us_write = graph_timed(lambda: step.write_block(attn_layers[0], kn, vn))
    n_acc = torch.full((B,), w.gamma, dtype=torch.int32, device=dev)
    ctx_scratch = inp.ctx_len.clone()
    us_commit = graph_timed(lambda: step.commit(n_acc, ctx_len=ctx_scratch))
    q1 = {l: inp.q_verify[l][:, :1].contiguous() for l in attn_layers}
    o1 = torch.empty((B, 1, T.hq, T.d), dtype=torch.bfloat16, device=dev)
    l1 = torch.empty((B, T.hq, 1), dtype=torch.float32, device=dev)
    ws1 = D.workspace(D.dustin_sparse_verify_attn_workspace_size(B, T.hq, T.hkv, T.d, 1, inp.k_max), dev)

    def decode_all():
        for l in attn_layers:
            k, v = step.kv[l]
            D.dustin_sparse_verify_attn(q1[l], k, v, T.hkv, inp.ctx_len, step.idx, step.count, step.scale,
                                        o1, l1, ws1)
    us_decode = timed(decode_all, reps) / len(attn_layers)
    # the gather floor of the same lists: the attention's K and V list rows read the same
    # way with every row in flight and no arithmetic, 80 layers back to back (unpaged views)
    us_floor = None
    if not any(step.kv[l][0].page_table or step.kv[l][1].page_table for l in attn_layers):
        fl_idx = step.idx[:, :inp.k_max].contiguous()
        fl_ck = torch.zeros((B, T.hkv), dtype=torch.int32, device=dev)

        def floor_all():
            for l in attn_layers:
                k, v = step.kv[l]
                D.dustin_gather_floor(k, v, T.hkv, T.d, fl_idx, fl_ck)
        floor_all()
        us_floor = timed(floor_all, reps) / len(attn_layers)
    b_floor = B * T.hkv * inp.k_max * 2 * T.d * 2
    b_decode = attn_bytes(B, T.hq, T.hkv, T.d, 1, counts)
    rec_layers = [l for l in (attn_layers[0], 60) if l in step.kv]
    recovery = {}
    for l in rec_layers:
        r = step.recovery(l)
        torch.cuda.synchronize()
        recovery[f"layer_{l}"] = {"mean": round(float(r.mean()), 5), "min": round(float(r.min()), 5),
                                  "max": round(float(r.max()), 5)}
    # the Vegas aggregate in its literal form: the first and bonus verify queries of every
    # query head of one layer (a logit-sum call over the layer's 8 KV heads)
    vg_score = torch.zeros((B, inp.n_max), dtype=torch.float32, device=dev)
    vg_ws = step.vegas_all_heads(attn_layers[0], vg_score)
    us_vegas_all = timed(lambda: step.vegas_all_heads(attn_layers[0], vg_score, vg_ws), reps)
    b_vegas_all = score_bytes(B, inp.n_max, [T.d] * T.hkv, 1)
    # the whole step captured once as a HIP graph and replayed (same kernels, same order)
    us_step_graph = graph_timed(step.step, n_calls=1, replays=args.steps)
    us_attn_graph = graph_timed(lambda: [step.attn(l) for l in attn_layers], n_calls=1, replays=reps) / len(attn_layers)
    step_extras = {
        "vegas_all_heads_layer_score_us": round(us_vegas_all, 2),
        "vegas_all_heads_layer_score_gbs": round(b_vegas_all / (us_vegas_all * 1e-6) / 1e9, 1),
        "step_us_graph_replay": round(us_step_graph, 1),
        "attn_per_call_graph_replay_us": round(us_attn_graph, 2),
        "kv_write_block_us": round(us_write, 2),
        "kv_write_block_bytes": 2 * 2 * B * nv * T.hkv * T.d * 2,
        "kv_commit_us": round(us_commit, 2),
        "attn_with_collect2_logits_per_call_us": round(us_attn_lg, 2),
        "collect2_logits_added_per_call_us": round(us_attn_lg - us_attn_all / len(attn_layers), 2),
        "collect2_logits_bytes_per_call": B * T.hkv * sum(int(c) for c in counts) * 4,
        "sparse_decode_nv1_per_call_us": round(us_decode, 2),
        "sparse_decode_nv1_gbs": round(b_decode / (us_decode * 1e-6) / 1e9, 1),
        "attn_recovery": recovery,
    }

    # ---- bytes ----
    n_ctx = inp.n_max
    b_attn = attn_bytes(B, T.hq, T.hkv, T.d, nv, counts)
    d_streams = [w.draft.d] * len(inp.draft_groups) + [T.d] * len(inp.target_groups)
    b_score = score_bytes(B, n_ctx, d_streams, 2)
    b_select = select_bytes(B, n_ctx, inp.k_max)
    b_step = b_score + b_select + len(attn_layers) * b_attn
    b_dense = attn_bytes(B, T.hq, T.hkv, T.d, nv, [n_ctx] * B) - B * n_ctx * 4   # no index list
    gbs = b_step / (step_ms * 1e-3) / 1e9
    plan = D.dustin_attn_plan(B, T.hq, T.hkv, T.d, nv, inp.k_max, D.ATTN_LAYOUT_LIST)
    # full-cache verification over every layer (the dense step: no scoring or selection)
    us_dense_sum = us_dense_layer * len(attn_layers)

    def spread(v):
        q = np.percentile(np.asarray(v, dtype=np.float64), [10, 50, 90])
        return {"p10": round(float(q[0]), 2), "median": round(float(q[1]), 2), "p90": round(float(q[2]), 2),
                "n": len(v)}
    us_attn_call = us_attn_all / len(attn_layers)     # back-to-back calls, events around the loop
    attn_gbs = b_attn / (us_attn_call * 1e-6) / 1e9

    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q, 1% needle keys at cosine 0.5 in the SRH streams)",
        "config": {"workload": w.name, "batch": B, "ctx": n_ctx, "budget": w.budget, "gamma": w.gamma,
                   "n_sink": w.n_sink, "n_window": w.n_window, "m": w.m, "layers": len(attn_layers),
                   "hq": T.hq, "hkv": T.hkv, "head_dim": T.d,
                   "srh_streams": {"draft": len(inp.draft_groups), "target": len(inp.target_groups)}},
        "step_us": round(step_ms * 1e3, 1),
        "stages_us": {"score_both_signals": round(us_score, 2), "select": round(us_select, 2),
                      "attn_per_call": round(us_attn_call, 2), "attn_per_call_own_events": round(us_attn_launch, 2),
                      "attn_all_layers": round(us_attn_all, 1)},
        "stages_spread_us": {"step": spread(per_step_us), "score_both_signals": spread(t_score),
                             "select": spread(t_select), "attn_all_layers": spread(t_attn_all),
                             "attn_per_call_own_events": spread(durs),
                             "dense_attn_all_layers": spread([t * len(attn_layers) / len(dl) for t in t_dense_all])},
        "dense_step": {"sum_dense_attn_all_layers_us": round(us_dense_sum, 1), "layers": len(attn_layers),
                       "layers_timed": len(dl),
                       "step_speedup_sparse_vs_dense": round(us_dense_sum / (step_ms * 1e3), 3),
                       "attn_speedup_sparse_vs_dense": round(us_dense_layer / us_attn_call, 3),
                       "byte_ratio_dense_over_sparse_step": round(len(attn_layers) * b_dense / b_step, 3)},
        "bytes": {"step": b_step, "attn_per_launch": b_attn, "score": b_score, "select": b_select},
        "score_gbs": round(b_score / (us_score * 1e-6) / 1e9, 1),
        "dense_attn_per_layer_us": round(us_dense_layer, 2),
        "target_signal_variants": variants,
        "around_the_step": step_extras,
        "dense_attn_gbs": round(b_dense / (us_dense_layer * 1e-6) / 1e9, 1),
        "attn_speedup_vs_dense": round(us_dense_layer / us_attn_call, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "dustin_sparse_verify_attn, one layer: " + D.attn_kernel_names(T.d, plan),
                     "plan": plan, "algorithmic_bytes_per_call": b_attn, "call_us": round(us_attn_call, 2)},
    }
    if us_floor is not None:
        # the same list rows gathered with no arithmetic (dustin_gather_floor): the ceiling
        # for these bytes as laid out, and the call's time over it
        line["roofline"]["gather_floor"] = {"us": round(us_floor, 2), "bytes": b_floor,
                                            "gbs": round(b_floor / (us_floor * 1e-6) / 1e9, 1),
                                            "call_over_floor": round(us_attn_call / us_floor, 3)}

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, step, args.cpu_seconds, b_attn, b_score, b_select, attn_layers)
    print(json.dumps(line), flush=True)


def attention_sweep(dev, args):
    """Sparse against dense verification attention on one Qwen2.5-72B-shaped layer at batch
    64 and 32k context, for budgets 1024/2048/4096 and gamma 2/4/8 (m = budget/4; the draft
    tier's size does not change the attention's cost), plus each point's scoring and
    selection.  Two copies of the layer's caches alternate, so no call finds the previous
    call's rows in the last-level cache.  Prints one JSON line."""
    import torch

    from sparse_kv_attention_amd import workloads as W
    from sparse_kv_attention_amd.pipeline import SparseVerifyStep

    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    points = []
    for gamma in (2, 4, 8):
        base = W.sweep_point(1024, gamma, 0.25)
        w2 = W.shrink(base, target=W.ModelShape(2, 64, 8, 128), srh_target=tuple((0, h) for _, h in base.srh_target))
        inp = W.make_inputs(w2, device=dev)             # layers 0 and 1: identical shapes, different data
        T = w2.target
        for k in (1024, 2048, 4096):
            for r in (0.25, 0.5):
                wk = W.shrink(w2, budget=k, n_window=k // 8, m=int(r * k))
                inp.w = wk
                inp.budget.fill_(k)
                inp.n_window.fill_(k // 8)
                inp.m.fill_(int(r * k))
                inp.k_max = k
                step = SparseVerifyStep(inp, layers=[0, 1])
                step.score()
                step.select()
                us_score = timed(step.score, 5)
                us_select = timed(step.select, 10)
                if r != 0.25:
                    points.append({"budget": k, "gamma": gamma, "m_over_budget": r, "score_us": round(us_score, 1),
                                   "select_us": round(us_select, 1)})
                    continue
                counts = step.count.cpu().tolist()
                us_sparse = timed(lambda: (step.attn(0), step.attn(1)), 10) / 2
                us_dense = timed(lambda: (step.dense(0), step.dense(1)), 3) / 2
                b_sp = attn_bytes(w2.batch, T.hq, T.hkv, T.d, w2.n_verify, counts)
                b_de = attn_bytes(w2.batch, T.hq, T.hkv, T.d, w2.n_verify, [inp.n_max] * w2.batch) - w2.batch * inp.n_max * 4
                points.append({"budget": k, "gamma": gamma, "m_over_budget": r, "score_us": round(us_score, 1),
                               "select_us": round(us_select, 1), "sparse_attn_us": round(us_sparse, 2),
                               "sparse_attn_gbs": round(b_sp / (us_sparse * 1e-6) / 1e9, 1),
                               "dense_attn_us": round(us_dense, 2), "dense_attn_gbs": round(b_de / (us_dense * 1e-6) / 1e9, 1),
                               "attn_speedup": round(us_dense / us_sparse, 2), "byte_ratio": round(b_de / b_sp, 2)})
                print(f"# {points[-1]}", file=sys.stderr, flush=True)
                del step
        del inp
        torch.cuda.empty_cache()
    print(json.dumps({"attention_sweep": points, "batch": 64, "ctx": 32768,
                      "layer": "64 q-heads / 8 KV heads, d 128, bf16",
                      "inputs": "N(0,1) with Pareto(1.2) key-norm salience capped at 16"}), flush=True)


def estimator_sweep(dev, args):
    """The naive estimator against full-cache attention as the context grows (English Dustin
    summary, "Problem Statement": materialising attention scores over all heads and layers
    costs more than full-cache attention beyond 4k tokens; "Experimental Results": the SRH
    estimation is under 1% of full-cache latency).  Qwen2.5-72B-shaped target with the
    0.5B-shaped draft, batch 8, gamma 4, contexts 1k..64k.  Per context length, one target
    layer and one draft layer are timed and multiplied by the layer counts (80 and 24; every
    layer has the same shape and cost); the SRH scoring is the real one (both signals, all
    8 SRH streams).  Prints one JSON line."""
    import torch

    from sparse_kv_attention_amd import workloads as W
    from sparse_kv_attention_amd.pipeline import AllHeadsEstimator, SparseVerifyStep

    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    points = []
    for n in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        w = W.shrink(W.QWEN72B, n_ctx=n, budget=min(2048, n // 4), n_window=min(256, n // 32),
                     m=min(768, 3 * n // 32), needle_mode="none")
        inp = W.make_inputs(w, device=dev, target_layers=[0])
        T, Dm = w.target, w.draft
        step = SparseVerifyStep(inp, layers=[0])
        q_t = inp.q_verify[0].permute(0, 2, 1, 3).contiguous()            # [B][Hq][gamma+1][d]
        g = torch.Generator(device=dev).manual_seed(n)
        q_d = torch.randn((w.batch, Dm.hq, w.gamma, Dm.d), generator=g, device=dev).to(torch.bfloat16)
        est_t = AllHeadsEstimator(inp.k_cache[0], None, q_t, T.hkv, inp.ctx_len, 1.0 / math.sqrt(T.d))
        est_d = AllHeadsEstimator(inp.draft_k[2], None, q_d, Dm.hkv, inp.ctx_len, 1.0 / math.sqrt(Dm.d))
        reps = max(3, min(20, (1 << 17) // n))
        us_t = timed(est_t.score, reps)
        us_d = timed(est_d.score, reps)
        us_dense = timed(lambda: step.dense(0), reps)
        us_srh = timed(step.score, reps)
        naive = T.layers * us_t + Dm.layers * us_d
        dense = T.layers * us_dense
        # bytes of one layer's naive estimate: every K row of every KV head once (the
        # method's minimum), and as launched (each group of <= 16 (head, query) pairs reads
        # its KV head's rows again)
        kb_t = w.batch * n * T.hkv * T.d * 2
        kb_d = w.batch * n * Dm.hkv * Dm.d * 2
        rd_t = sum(len(g) for g, _ in est_t.calls) * w.batch * n * T.d * 2
        rd_d = sum(len(g) for g, _ in est_d.calls) * w.batch * n * Dm.d * 2
        b_dense = attn_bytes(w.batch, T.hq, T.hkv, T.d, w.n_verify, [n] * w.batch) - w.batch * n * 4
        points.append({"ctx": n, "naive_target_layer_us": round(us_t, 2), "naive_draft_layer_us": round(us_d, 2),
                       "dense_layer_us": round(us_dense, 2), "naive_all_layers_us": round(naive, 1),
                       "dense_all_layers_us": round(dense, 1), "srh_scoring_us": round(us_srh, 2),
                       "naive_over_dense": round(naive / dense, 3), "srh_over_dense": round(us_srh / dense, 5),
                       "naive_calls_per_layer": {"target": len(est_t.calls), "draft": len(est_d.calls)},
                       "naive_target_layer_bytes": kb_t, "naive_target_layer_bytes_as_launched": rd_t,
                       "naive_draft_layer_bytes": kb_d, "naive_draft_layer_bytes_as_launched": rd_d,
                       "naive_all_layers_bytes": T.layers * kb_t + Dm.layers * kb_d,
                       "dense_all_layers_bytes": T.layers * b_dense,
                       "naive_target_gbs_as_launched": round(rd_t / (us_t * 1e-6) / 1e9, 1),
                       "dense_gbs": round(b_dense / (us_dense * 1e-6) / 1e9, 1)})
        print(f"# ctx {n}: {points[-1]}", file=sys.stderr, flush=True)
        del step, est_t, est_d, inp
        torch.cuda.empty_cache()
    print(json.dumps({"estimator_sweep": points, "batch": 8, "gamma": 4,
                      "target": "80 layers x 64 q-heads / 8 KV heads, d 128",
                      "draft": "24 layers x 14 q-heads / 2 KV heads, d 64",
                      "layer_extrapolation": "one layer of each model timed, times its layer count"}), flush=True)


def _oracle_item(item):
    """One shard of the oracle sample, run in a worker process: ("score", files, meta),
    ("select", files, meta) or ("attn", files, meta).  Returns (kind, seconds of oracle
    time).  Workers never touch the GPU: every input arrives as a .npy file."""
    import numpy as np

    from oracle import oracle as O

    kind, files, meta = item
    ld = lambda k: np.load(files[k])
    if kind == "score":
        acc = np.zeros((1, meta["n_max"]))
        args = [(ld(f"K{i}"), ld(f"Q{i}"), meta["scale"][i]) for i in range(meta["n_groups"])]
        ctx = ld("ctx")
        t = time.perf_counter()
        for K, Q, sc in args:
            O.score_stream(K, Q, ctx, meta["n_max"], sc, O.PROB_SUM, acc)
        return kind, time.perf_counter() - t
    if kind == "select":
        a = {k: ld(k) for k in ("ctx", "sd", "st", "budget", "n_sink", "n_window", "m")}
        t = time.perf_counter()
        O.select(a["ctx"], a["sd"], a["st"], a["budget"], a["n_sink"], a["n_window"], a["m"], meta["k_max"])
        return kind, time.perf_counter() - t
    Q, K, V, idx, cnt, ctx = (ld(k) for k in ("Q", "K", "V", "idx", "cnt", "ctx"))
    t = time.perf_counter()
    O.verify_attn(Q, K, V, ctx, idx, cnt, meta["scale"], meta["hkv"])
    return kind, time.perf_counter() - t


def _worker_ready(_):
    from oracle import oracle as O
    O.lib()
    return os.getpid()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, step, budget_s, b_attn, b_score, b_select, layers):
    """The oracle (plain C, fp64, single-threaded per process) on a bounded sample of the
    same workload, sharded over the host's cores: every sequence's SRH scoring (both
    signals) and selection, and the sparse attention of every sequence on as many layers
    as the CPU-time budget allows (each (sequence, layer) an independent shard).  Shards
    run in a pool of worker processes, one per core of the host's share (at most 16); the
    figure is the sample's algorithmic bytes over the pool's wall time.  The same shards'
    summed per-shard oracle times give the one-core figure beside it.  Attention shards get
    the selected K/V rows and the new block compacted in list order with the list
    renumbered 0..count-1: the oracle computes exactly the same sums over the same rows."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np
    import torch

    u16 = lambda t: t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    w = inp.w
    B, nv = w.batch, w.n_verify
    n = inp.n_max
    ctx = inp.ctx_len.cpu().numpy().astype(np.int32)
    cnt = step.count.cpu().numpy().astype(np.int32)
    idx = step.idx.cpu().numpy()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    P = max(1, min(16, cores))
    # per-shard oracle seconds measured earlier on this workload: about 0.55 s of scoring per
    # sequence and 0.09 s per (sequence, layer) of attention; the layer count fills the
    # budget (10-30 s of single-core oracle time)
    n_layers = max(1, min(len(layers), int(budget_s / (0.09 * B))))
    shm = "/dev/shm" if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > (4 << 30) else None
    tmp = tempfile.mkdtemp(prefix="oracle_sample_", dir=shm)
    items, nbytes = [], 0.0
    try:
        def save(name, arr):
            path = os.path.join(tmp, name + ".npy")
            np.save(path, np.ascontiguousarray(arr))
            return path

        sd = step.score_draft.double().cpu().numpy()
        st = step.score_target.double().cpu().numpy()
        for b in range(B):
            files, scales, gi = {}, [], 0
            for groups, q, caches, d in ((inp.draft_groups, inp.q_srh_draft, inp.draft_k, w.draft.d),
                                         (inp.target_groups, inp.q_srh_target, inp.k_cache, w.target.d)):
                qo = 0
                for g in groups:
                    files[f"K{gi}"] = save(f"s{b}_K{gi}", u16(caches[g.layer][b:b + 1, :n, g.kv_head]))
                    files[f"Q{gi}"] = save(f"s{b}_Q{gi}", u16(q[b:b + 1, qo:qo + len(g.qheads)]))
                    scales.append(1.0 / math.sqrt(d))
                    qo += len(g.qheads)
                    gi += 1
            files["ctx"] = save(f"s{b}_ctx", ctx[b:b + 1])
            items.append(("score", files, {"n_max": n, "scale": scales, "n_groups": gi}))
            sel = {"ctx": ctx[b:b + 1], "sd": sd[b:b + 1], "st": st[b:b + 1]}
            for k in ("budget", "n_sink", "n_window", "m"):
                sel[k] = getattr(inp, k).cpu().numpy()[b:b + 1].astype(np.int32)
            items.append(("select", {k: save(f"l{b}_{k}", v) for k, v in sel.items()}, {"k_max": inp.k_max}))
            nbytes += (b_score + b_select) / B
        for l in layers[:n_layers]:
            for b in range(B):
                c = int(cnt[b])
                rows = torch.cat([step.idx[b, :c].long(),
                                  torch.arange(int(ctx[b]), int(ctx[b]) + nv, device=step.idx.device)])
                files = {"K": save(f"a{l}_{b}_K", u16(inp.k_cache[l][b].index_select(0, rows)[None])),
                         "V": save(f"a{l}_{b}_V", u16(inp.v_cache[l][b].index_select(0, rows)[None])),
                         "Q": save(f"a{l}_{b}_Q", u16(inp.q_verify[l][b:b + 1])),
                         "idx": save(f"a{l}_{b}_idx", np.arange(c, dtype=np.int32)[None]),
                         "cnt": save(f"a{l}_{b}_cnt", np.array([c], dtype=np.int32)),
                         "ctx": save(f"a{l}_{b}_ctx", np.array([c], dtype=np.int32))}
                items.append(("attn", files, {"scale": 1.0 / math.sqrt(w.target.d), "hkv": w.target.hkv}))
                nbytes += b_attn / B
        # the longest shards first, so the pool's tail is short
        items.sort(key=lambda it: {"score": 0, "attn": 1, "select": 2}[it[0]])
        ctx_mp = mp.get_context("spawn")
        with ctx_mp.Pool(P) as pool:
            pool.map(_worker_ready, range(P))          # interpreters and the oracle loaded
            t0 = time.perf_counter()
            res = pool.map(_oracle_item, items, chunksize=1)
            wall = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    cpu_s = sum(r[1] for r in res)
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": P, "kind": "oracle",
            "sample": f"SRH scoring (both signals) and selection of all {B} sequences, sparse attention of all "
                      f"{B} sequences on {n_layers} of {len(layers)} layers: {len(items)} independent shards in "
                      f"a pool of {P} processes; {cpu_s:.1f} s of oracle time, {wall:.2f} s wall",
            "cpu_model": cpu_model(), "host_cpus_visible": cores,
            "single_core_gbs": round(nbytes / cpu_s / 1e9, 4), "wall_s": round(wall, 3),
            "oracle_cpu_s": round(cpu_s, 2), "sample_bytes": int(nbytes)}


if __name__ == "__main__":
    main()
