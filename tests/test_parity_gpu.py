"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Bars: scores within 1e-5 relative (+1e-10 absolute floor; for logit sums the relative
term is taken against the sum of |logits|), selection bit-exact when the oracle selects
on the GPU's own fp32 scores, attention output max-abs 2e-2 and LSE 1e-3.
"""
import math
import os

import numpy as np
import pytest
import torch

from _harness import (SCORE_ATOL, SCORE_RTOL, check_attn, check_scores, logit_abs_sum, oracle_attn,
                      oracle_scores, oracle_select_on, rows, say, u16)
from oracle import oracle as O
from sparse_kv_attention_amd import workloads as W
from sparse_kv_attention_amd.workloads import ModelShape, Workload

pytestmark = pytest.mark.gpu


def step_for(inp, layers, logit_sum2=False, logit_sum_all=False):
    from sparse_kv_attention_amd.pipeline import SparseVerifyStep
    return SparseVerifyStep(inp, layers=layers, logit_sum2=logit_sum2, logit_sum_all=logit_sum_all)


def check_pipeline(inp, attn_layers, dense_layers, b_attn, b_score=None, logit_sum2=False, b_dense=None,
                   logit_sum_all=False):
    w = inp.w
    B = w.batch
    b_score = list(range(B)) if b_score is None else b_score
    step = step_for(inp, attn_layers, logit_sum2, logit_sum_all)
    logit_sum2 = logit_sum2 or logit_sum_all
    say(f"[{w.name}] scoring")
    step.score()
    torch.cuda.synchronize()
    sd = step.score_draft.cpu().numpy()
    st = step.score_target.cpu().numpy()
    if logit_sum2:
        mode = O.LOGIT_SUM_ALL if logit_sum_all else O.LOGIT_SUM2
        ora = oracle_scores(inp, "target", mode, b_score)
        check_scores(st[b_score], ora, "target logit-sum scores",
                     cond=logit_abs_sum(inp, "target", b_score, all_queries=logit_sum_all))
    else:
        if step.has_draft:
            check_scores(sd[b_score], oracle_scores(inp, "draft", O.PROB_SUM, b_score), "draft scores")
        check_scores(st[b_score], oracle_scores(inp, "target", O.PROB_SUM, b_score), "target scores")
    say(f"[{w.name}] selection")
    step.select()
    torch.cuda.synchronize()
    allb = list(range(B))
    idx_o, cnt_o = oracle_select_on(inp, sd.astype(np.float64) if step.has_draft else None,
                                    st.astype(np.float64), allb, pure_topk=logit_sum2)
    idx_g = step.idx.cpu().numpy()
    cnt_g = step.count.cpu().numpy()
    assert np.array_equal(cnt_g, cnt_o), (cnt_g, cnt_o)
    assert np.array_equal(idx_g[:, :inp.k_max], idx_o), "selected positions differ from the oracle's"
    say(f"  selection bit-exact over {B} sequences (counts {cnt_g.min()}..{cnt_g.max()})")
    for l in attn_layers:
        say(f"[{w.name}] sparse attention layer {l}")
        step.attn(l)
        torch.cuda.synchronize()
        check_attn(step.out, step.lse, oracle_attn(inp, l, idx_g, cnt_g, b_attn), b_attn, f"sparse layer {l}")
    for l in dense_layers:
        say(f"[{w.name}] dense attention layer {l}")
        bd = b_attn if b_dense is None else b_dense
        step.dense(l)
        torch.cuda.synchronize()
        check_attn(step.out, step.lse, oracle_attn(inp, l, None, None, bd, dense=True), bd, f"dense layer {l}")
    return step


def small(name, B, n, hq, hkv, d, gamma, budget, s, w, m, seed, dd=64, value_scale=1.0):
    return Workload(name=name, batch=B, n_ctx=n, target=ModelShape(1, hq, hkv, d),
                    draft=ModelShape(1, 2, 2, dd), gamma=gamma, budget=budget, n_sink=s, n_window=w, m=m,
                    srh_draft=((0, 0), (0, 1)), srh_target=((0, 0),), seed=seed, value_scale=value_scale)


# ----------------------------------------------------------------------------- workloads

def test_tiny_pipeline():
    inp = W.make_inputs(W.TINY, device="cuda")
    step = check_pipeline(inp, [0], [0], [0])
    # the planted needles carry the largest draft scores: the draft tier must hold them all
    sel = set(step.idx[0, :int(step.count[0])].tolist())
    assert set(inp.needles[0].tolist()) <= sel


def test_qwen7b_pipeline():
    inp = W.make_inputs(W.QWEN7B, device="cuda", target_layers=[0])
    check_pipeline(inp, [0, 20], [0], [0, 1, 2, 3])


# ----------------------------------------------------------------------------- edge cases

def test_ragged_and_empty_contexts():
    w = small("ragged_edges", 5, 700, 8, 2, 128, 3, 96, 4, 16, 24, seed=11)
    inp = W.make_inputs(w, device="cuda")
    inp.ctx_len = torch.tensor([0, 1, 50, 97, 700], dtype=torch.int32, device="cuda")
    step = check_pipeline(inp, [0], [0], [0, 1, 2, 3, 4])
    assert step.count.cpu().tolist() == [0, 1, 50, 96, 96]


def test_full_budget_matches_dense_bitwise():
    w = small("full_budget", 2, 300, 8, 2, 128, 4, 300, 4, 16, 40, seed=12)
    inp = W.make_inputs(w, device="cuda")
    step = check_pipeline(inp, [0], [0], [0, 1])
    step.attn(0)
    o_s, l_s = step.out.clone(), step.lse.clone()
    step.dense(0)
    assert torch.equal(o_s, step.out) and torch.equal(l_s, step.lse)


def test_single_verify_query():
    w = small("gamma0", 3, 513, 16, 4, 128, 0, 64, 2, 8, 10, seed=13)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [0], [0, 1, 2])


def test_widest_verify_block():
    # 16 verify queries (the most accepted): the whole 16-row new-token step, causal inside
    # it; G = 4 gives 64 query rows (four 16-row tiles) at head dim 128, and the head-dim-64
    # draft streams score 15 lookahead queries
    w = small("nv16", 2, 600, 8, 2, 128, 15, 128, 4, 16, 40, seed=16)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [0], [0, 1])


def test_scoring_three_tiles_per_workgroup():
    # 8 sequences x 4 SRH groups per signal = 32 streams, so the softmax-mode logit grid has
    # 16 workgroups per stream; 12288 tokens = 48 tiles of 256, i.e. three per workgroup:
    # the two-tiles-in-flight loop ends on a half-used pair
    w = Workload(name="odd_tiles", batch=8, n_ctx=12288, target=ModelShape(1, 16, 4, 128),
                 draft=ModelShape(1, 8, 4, 64), gamma=4, budget=512, n_sink=16, n_window=64, m=192,
                 srh_draft=((0, 0), (0, 2), (0, 4), (0, 6)), srh_target=((0, 0), (0, 4), (0, 8), (0, 12)),
                 seed=17)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [], [0, 5], b_score=[0, 3, 7])


def test_query_groups_split():
    # G = 16 query heads per KV head x 8 verify queries = 128 rows: two query groups
    w = small("qgroups", 2, 400, 32, 2, 128, 7, 100, 4, 8, 20, seed=14)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [0], [0, 1])


def test_head_dim_64_and_odd_group():
    w = small("d64", 2, 1000, 14, 2, 64, 4, 200, 4, 32, 50, seed=15)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [0], [0, 1])


def test_split_plans_agree_and_repeat_bitwise():
    w = small("splits", 2, 3000, 16, 2, 128, 4, 1024, 16, 64, 300, seed=16)
    inp = W.make_inputs(w, device="cuda")
    step = check_pipeline(inp, [0], [], [0, 1])
    idx, cnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    ref = oracle_attn(inp, 0, idx, cnt, [0, 1])
    refd = oracle_attn(inp, 0, None, None, [0, 1], dense=True)
    old = os.environ.get("DUSTIN_ATTN_TARGET_WGS")
    try:
        for tw in ("1", "7", "100000"):
            os.environ["DUSTIN_ATTN_TARGET_WGS"] = tw
            step2 = step_for(inp, [0])
            step2.idx.copy_(step.idx)
            step2.count.copy_(step.count)
            outs = []
            for _ in range(3):
                step2.attn(0)
                outs.append((step2.out.clone(), step2.lse.clone()))
            torch.cuda.synchronize()
            for o, l in outs[1:]:
                assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1]), "not deterministic"
            check_attn(outs[0][0], outs[0][1], ref, [0, 1], f"sparse, target wgs {tw}")
            step2.dense(0)
            torch.cuda.synchronize()
            check_attn(step2.out, step2.lse, refd, [0, 1], f"dense, target wgs {tw}")
    finally:
        if old is None:
            os.environ.pop("DUSTIN_ATTN_TARGET_WGS", None)
        else:
            os.environ["DUSTIN_ATTN_TARGET_WGS"] = old


def test_out_of_range_device_values_are_clamped():
    """Garbage positions and counts cannot make a kernel leave its buffers: the kernel
    clamps them, and the result is the oracle's on the clamped values."""
    w = small("clamp", 2, 200, 8, 2, 128, 2, 32, 2, 4, 6, seed=17)
    inp = W.make_inputs(w, device="cuda")
    step = step_for(inp, [0])
    k_max = inp.k_max
    idx = torch.randint(0, 200, (2, k_max), dtype=torch.int32)
    idx[0, 3] = -7
    idx[1, 5] = 10 ** 9
    cnt = torch.tensor([k_max + 50, 10], dtype=torch.int32)
    step.idx.copy_(idx)
    step.count.copy_(cnt)
    step.attn(0)
    torch.cuda.synchronize()
    N = inp.ctx_len.cpu().numpy()
    idx_c = np.clip(idx.numpy(), 0, N[:, None] - 1).astype(np.int32)
    cnt_c = np.minimum(cnt.numpy(), k_max).astype(np.int32)
    check_attn(step.out, step.lse, oracle_attn(inp, 0, idx_c, cnt_c, [0, 1]), [0, 1], "clamped")


def test_logit_sum2_pure_topk():
    w = small("logit2", 3, 2000, 16, 4, 128, 4, 125, 0, 0, 0, seed=18)
    w = W.shrink(w, srh_target=((0, 0), (0, 1), (0, 4), (0, 8)))
    inp = W.make_inputs(w, device="cuda")
    check_pipeline(inp, [0], [], [0, 1, 2], logit_sum2=True)


def test_logit_sum_all_pure_topk():
    """The full Vegas aggregate over every query: one group of 4 query heads x 9 queries
    (36 pairs, three 16-pair MFMA tiles) and one of 9 pairs, ragged tail of 2000 tokens."""
    w = small("logitall", 3, 2000, 16, 4, 128, 8, 125, 0, 0, 0, seed=19)
    w = W.shrink(w, srh_target=((0, 0), (0, 1), (0, 2), (0, 3), (0, 4)))
    inp = W.make_inputs(w, device="cuda")
    check_pipeline(inp, [0], [], [0, 2], logit_sum_all=True)


def _paged_copy(x: torch.Tensor, page_size: int, seed: int):
    """x [B][n][Hkv][d] into pages [B*npg][page_size][Hkv][d] under a random page table."""
    B, n, H, d = x.shape
    npg = (n + page_size - 1) // page_size
    gen = torch.Generator().manual_seed(seed)
    pt = torch.randperm(B * npg, generator=gen).to(torch.int32).view(B, npg).to(x.device)
    padded = torch.zeros((B, npg * page_size, H, d), dtype=x.dtype, device=x.device)
    padded[:, :n] = x
    pages = torch.zeros((B * npg, page_size, H, d), dtype=x.dtype, device=x.device)
    pages[pt.reshape(-1).long()] = padded.view(B * npg, page_size, H, d)
    return pages, pt


def test_k_and_v_at_different_row_offsets():
    """K and V views whose rows sit at different offsets (V stored head-major; then K and V
    paged under different page tables): the kernel resolves K and V rows separately."""
    from sparse_kv_attention_amd import dustin as D
    w = small("kv_layouts", 3, 1500, 16, 2, 128, 4, 400, 4, 32, 100, seed=19)
    inp = W.make_inputs(w, device="cuda")
    step = check_pipeline(inp, [0], [], [0, 1, 2])
    bs = [0, 1, 2]
    idx, cnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    ref = oracle_attn(inp, 0, idx, cnt, bs)
    refd = oracle_attn(inp, 0, None, None, bs, dense=True)
    K, V = inp.k_cache[0], inp.v_cache[0]
    v_head_major = torch.empty((V.shape[0], V.shape[2], V.shape[1], V.shape[3]), dtype=V.dtype,
                               device=V.device).permute(0, 2, 1, 3)
    v_head_major.copy_(V)
    kp, ptk = _paged_copy(K, 16, 1)
    vp, ptv = _paged_copy(V, 16, 2)
    for name, kv in (("V head-major", (D.kv_view(K), D.kv_view(v_head_major))),
                     ("K and V paged, different page tables", (D.kv_view(kp, ptk), D.kv_view(vp, ptv)))):
        step.kv[0] = kv
        step.attn(0)
        torch.cuda.synchronize()
        check_attn(step.out, step.lse, ref, bs, f"sparse, {name}")
        step.dense(0)
        torch.cuda.synchronize()
        check_attn(step.out, step.lse, refd, bs, f"dense, {name}")


def _with_env(name, value, fn):
    old = os.environ.get(name)
    try:
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = value
        return fn()
    finally:
        if old is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = old


def test_fused_split_merge_matches_merge_kernel_bitwise():
    """The splits combined inside the attention kernel by the last workgroup to finish equal
    the separate merge kernel's result bit for bit (same weights, same order), for
    contiguous and paged caches, sparse and dense, under two split plans; repeated calls
    on one workspace leave its arrival counters ready for the next call."""
    from sparse_kv_attention_amd import dustin as D
    w = small("fused", 3, 2500, 16, 2, 128, 4, 900, 4, 32, 100, seed=23)
    inp = W.make_inputs(w, device="cuda")
    step = check_pipeline(inp, [0], [], [0, 2])
    bs = [0, 1, 2]
    idx, cnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    ref = oracle_attn(inp, 0, idx, cnt, bs)
    refd = oracle_attn(inp, 0, None, None, bs, dense=True)
    K, V = inp.k_cache[0], inp.v_cache[0]
    kp, ptk = _paged_copy(K, 16, 3)
    vp, ptv = _paged_copy(V, 16, 4)
    layouts = (("contiguous", (D.kv_view(K), D.kv_view(V))),
               ("paged, two page tables", (D.kv_view(kp, ptk), D.kv_view(vp, ptv))))

    def run(kv, dense):
        def go():
            s2 = step_for(inp, [0])
            s2.idx.copy_(step.idx)
            s2.count.copy_(step.count)
            s2.kv[0] = kv
            res = []
            for _ in range(3):
                s2.dense(0) if dense else s2.attn(0)
                res.append((s2.out.clone(), s2.lse.clone()))
            torch.cuda.synchronize()
            return res
        return go

    for tw in (None, "7"):
        for name, kv in layouts:
            for dense in (False, True):
                what = f"{'dense' if dense else 'sparse'}, {name}, target wgs {tw or 'default'}"
                say(f"  fused merge vs merge kernel: {what}")
                two = _with_env("DUSTIN_ATTN_TARGET_WGS", tw,
                                lambda: _with_env("DUSTIN_ATTN_FUSED_MERGE", "0", run(kv, dense)))
                fused = _with_env("DUSTIN_ATTN_TARGET_WGS", tw,
                                  lambda: _with_env("DUSTIN_ATTN_FUSED_MERGE", "1", run(kv, dense)))
                for o, l in fused + two[1:]:
                    assert torch.equal(o, two[0][0]) and torch.equal(l, two[0][1]), what
                check_attn(fused[0][0], fused[0][1], refd if dense else ref, bs, what)


def _collect2_reference(inp, layer, idx, cnt, bsel):
    """Oracle LOGIT_SUM2 over each KV head's query heads at the listed positions, and the
    sum of |logits| of the same terms (the conditioning of the sum)."""
    w = inp.w
    T = w.target
    G = T.hq // T.hkv
    nv = w.n_verify
    scale = 1.0 / math.sqrt(T.d)
    ctx = inp.ctx_len.cpu().numpy()
    ref = {}
    for i, b in enumerate(bsel):
        K = rows(inp, inp.k_cache[layer], b, inp.n_max).cpu()                 # [n_max][Hkv][d]
        for g in range(T.hkv):
            Q = inp.q_verify[layer][b:b + 1, :, g * G:(g + 1) * G].permute(0, 2, 1, 3).contiguous().cpu()
            acc = O.score_stream(u16(K[None, :, g]), u16(Q), ctx[b:b + 1], inp.n_max, scale, O.LOGIT_SUM2)
            js = sorted({0, nv - 1})
            cond = (K[:, g].double() @ Q[0][:, js].double().reshape(-1, T.d).T).abs().sum(1).numpy() * scale
            c = int(cnt[b])
            ref[(b, g)] = (acc[0][idx[b, :c]], cond[idx[b, :c]])
    return ref


@pytest.mark.parametrize("case", ["qwen7b", "paged_two_tables", "single_query", "d64_odd_group"])
def test_collect2_logits_emitted_by_verification(case):
    """The verification kernel's Collect-2 by-product: per selected token, the scaled
    pre-softmax logits of verify queries 0 and n_verify-1 summed over the KV head's query
    heads, against the oracle's LOGIT_SUM2 at the listed positions (1e-5 of the sum of
    |logits|); the attention output is unchanged bit for bit by the emission."""
    from sparse_kv_attention_amd import dustin as D
    if case == "qwen7b":
        w = W.shrink(W.QWEN7B, target=ModelShape(2, 28, 4, 128), srh_target=((0, 0), (1, 0)))
    elif case == "single_query":
        w = small("c2_nv1", 2, 900, 16, 2, 128, 0, 200, 4, 16, 40, seed=41)
    elif case == "d64_odd_group":
        w = small("c2_d64", 3, 1200, 14, 2, 64, 6, 300, 4, 32, 60, seed=42)
    else:
        w = small("c2_paged", 3, 1500, 16, 2, 128, 4, 400, 4, 32, 100, seed=43)
    inp = W.make_inputs(w, device="cuda")
    step = step_for(inp, [0])
    step.score()
    step.select()
    if case == "paged_two_tables":
        K, V = inp.k_cache[0], inp.v_cache[0]
        kp, ptk = _paged_copy(K, 16, 5)
        vp, ptv = _paged_copy(V, 16, 6)
        step.kv[0] = (D.kv_view(kp, ptk), D.kv_view(vp, ptv))
    B = w.batch
    lg = torch.full((B, w.target.hkv, inp.k_max), float("nan"), dtype=torch.float32, device="cuda")
    step.attn(0)
    torch.cuda.synchronize()
    out0, lse0 = step.out.clone(), step.lse.clone()
    step.attn_logits(0, lg)
    torch.cuda.synchronize()
    assert torch.equal(step.out, out0) and torch.equal(step.lse, lse0), "the emission changed the attention"
    idx, cnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    bs = list(range(B))
    ref = _collect2_reference(inp, 0, idx, cnt, bs)
    got = lg.cpu().numpy()
    worst = 0.0
    for (b, g), (r, cond) in ref.items():
        c = int(cnt[b])
        e = np.abs(got[b, g, :c].astype(np.float64) - r)
        tol = SCORE_RTOL * cond + SCORE_ATOL
        assert np.all(e <= tol), (case, b, g, float(np.max(e / tol)))
        assert np.all(np.isnan(got[b, g, c:])), "entries past the count were written"
        worst = max(worst, float(np.max(e / tol)) if c else 0.0)
    say(f"  collect-2 logits ({case}): max err/tol = {worst:.3g} over {int(cnt.sum())} tokens x {w.target.hkv} heads")


def test_step_replayed_as_hip_graph_matches_eager():
    """The whole step (both scoring calls, selection, two attention layers) captured once as
    a HIP graph: every replay, with eager work and synchronisations in between, gives
    bitwise the eager results (no call records a memset or allocates)."""
    inp = W.make_inputs(W.QWEN7B, device="cuda", target_layers=[0, 1])
    step = step_for(inp, [0, 1])
    outs = lambda: [t.clone() for t in (step.score_draft, step.score_target, step.idx, step.count, step.out,
                                        step.lse)]
    step.step()
    torch.cuda.synchronize()
    ref = outs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.step()
    for r in range(3):
        for t in (step.score_draft, step.score_target, step.out, step.lse):
            t.zero_()                         # eager work between the replays
        step.idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), ref):
            assert torch.equal(a, b), f"replay {r} differs from the eager step"
    say("  three graph replays equal the eager step bitwise")


def test_scores_repeat_bitwise():
    """The waves of a scoring workgroup claim tiles dynamically, but each workgroup folds
    its tiles' statistics in tile order: repeated calls give bitwise the same scores."""
    w = W.shrink(W.QWEN7B, batch=3, n_ctx=5000, ragged_lo=1000)
    inp = W.make_inputs(w, device="cuda", target_layers=[0])
    step = step_for(inp, [0])
    first = None
    for r in range(4):
        step.score_draft.zero_()
        step.score_target.zero_()
        step.score()
        torch.cuda.synchronize()
        got = (step.score_draft.clone(), step.score_target.clone())
        if first is None:
            first = got
            check_scores(got[1].cpu().numpy(), oracle_scores(inp, "target", O.PROB_SUM, [0, 1, 2]), "target scores")
        else:
            assert torch.equal(got[0], first[0]) and torch.equal(got[1], first[1]), f"call {r} differs"
    say("  four scoring calls bitwise equal")


def test_both_signals_in_one_call_match_separate_calls():
    """dustin_srh_score_signals (one logit launch for the draft and target streams of
    different head dims, one finalize) against one dustin_srh_score call per signal and
    against the oracle, on a paged ragged workload and with the target in logit-sum mode."""
    from sparse_kv_attention_amd import dustin as D
    for name, w, kw in (("7B ragged", W.shrink(W.QWEN7B, batch=3, n_ctx=5000, ragged_lo=1000), {}),
                        ("paged", W.shrink(W.RAGGED_PAGED, batch=2, n_ctx=3000, ragged_lo=700,
                                           target=ModelShape(1, 64, 8, 128),
                                           srh_target=((0, 0), (0, 8))), {}),
                        ("collect-2 target", W.shrink(W.QWEN7B, batch=2, n_ctx=3000), {"logit_sum2": True})):
        inp = W.make_inputs(w, device="cuda", target_layers=[0] if name != "paged" else None)
        step = step_for(inp, [0], **kw)
        bs = list(range(w.batch))
        step.score()
        torch.cuda.synchronize()
        fused = (step.score_draft.clone(), step.score_target.clone())
        step.score_draft.zero_()
        step.score_target.zero_()
        step.score_separately()
        torch.cuda.synchronize()
        sep = (step.score_draft.clone(), step.score_target.clone())
        if kw:
            cond = logit_abs_sum(inp, "target", bs)
            check_scores(fused[1].cpu().numpy(), oracle_scores(inp, "target", O.LOGIT_SUM2, bs),
                         f"{name}: target, one call", cond=cond)
            check_scores(sep[1].cpu().numpy(), oracle_scores(inp, "target", O.LOGIT_SUM2, bs),
                         f"{name}: target, own call", cond=cond)
            continue
        for i, sig in enumerate(("draft", "target")):
            ora = oracle_scores(inp, sig, O.PROB_SUM, bs)
            check_scores(fused[i].cpu().numpy(), ora, f"{name}: {sig}, one call")
            check_scores(sep[i].cpu().numpy(), ora, f"{name}: {sig}, own call")


def test_five_query_tiles():
    """72 query rows per KV head (G = 8, gamma = 8) fill five 16-row tiles in one workgroup:
    at head dim 128 the waves exchange their accumulators in two phases, at head dim 64 in
    one; 144 rows (G = 16) run as two query groups of five tiles."""
    for name, w in (("qt5_d128", small("qt5_d128", 2, 1100, 16, 2, 128, 8, 256, 4, 32, 64, seed=22)),
                    ("qt5_d64", small("qt5_d64", 2, 1100, 16, 2, 64, 8, 256, 4, 32, 64, seed=23)),
                    ("qt5x2_d128", small("qt5x2_d128", 2, 900, 32, 2, 128, 8, 200, 4, 16, 40, seed=24))):
        say(f"[{name}]")
        check_pipeline(W.make_inputs(w, device="cuda"), [0], [0], [0, 1])


def test_selection_stops_early_on_a_whole_digit_bin():
    """Planted scores make the radix search stop before its last pass because every key of
    the chosen digit bin belongs to the top set: after the first pass (draft tier of
    sequence 0), after the second (sequence 1), after the third in both tiers (sequence 2);
    all-equal scores (sequence 3) run every pass and take ties by position.  The target
    tier after an early draft stop must see clean histograms.  Bit-exact against the
    oracle on the same fp32 scores, 32k context (32 keys per thread), budget 512."""
    from sparse_kv_attention_amd import dustin as D
    B, n_max, k_max = 4, 32768, 512
    ctx = np.array([32768, 30000, 32768, 20000], dtype=np.int32)
    s, wdw, m = 4, 64, 256
    r = k_max - s - wdw - m                      # 188 target picks
    gen = np.random.default_rng(31)
    sd = gen.uniform(1e-6, 1e-3, (B, n_max)).astype(np.float32)
    st = gen.uniform(1e-6, 1e-3, (B, n_max)).astype(np.float32)
    u = lambda bits: np.asarray(bits, dtype=np.uint32).view(np.float32)
    pos = lambda b, n: gen.choice(np.arange(s, ctx[b] - wdw), n, replace=False)
    # sequence 0: the m draft keys alone above 1.0 (one top-byte bin)
    sd[0, pos(0, m)] = u(0x3F800000 + 4096 * np.arange(m))
    # sequence 1: m draft keys 0.75 + i*2^-16 share two bytes; 5 keys at 0.5 share the first
    p1 = pos(1, m + 5)
    sd[1, p1[:m]] = u(0x3F400000 + 256 * np.arange(m))
    sd[1, p1[m:]] = u(0x3F000000 + np.arange(5))
    # sequence 2: in both tiers the picks share three bytes, 3 keys share only two (the
    # target keys at positions the draft tier does not take)
    p2 = pos(2, m + r + 6)
    for sc, pp, n in ((sd, p2[:m + 3], m), (st, p2[m + 3:], r)):
        sc[2, pp[:n]] = u(0x3F400400 + np.arange(n))
        sc[2, pp[n:]] = u(0x3F400000 + np.arange(3))
    sd[3] = 0.0
    st[3] = 0.0
    dev = "cuda"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    full = lambda v: torch.full((B,), v, dtype=torch.int32, device=dev)
    idx = torch.full((B, k_max), -5, dtype=torch.int32, device=dev)
    cnt = torch.zeros((B,), dtype=torch.int32, device=dev)
    ws = D.workspace(D.dustin_select_workspace_size(B, n_max), dev)
    for rep in range(2):
        D.dustin_select(t(ctx), t(sd), t(st), full(k_max), full(s), full(wdw), full(m), idx, cnt, ws)
        torch.cuda.synchronize()
        want_idx, want_cnt = O.select(ctx, sd, st, [k_max] * B, [s] * B, [wdw] * B, [m] * B, k_max)
        assert np.array_equal(cnt.cpu().numpy(), want_cnt)
        got = idx.cpu().numpy()
        for b in range(B):
            assert np.array_equal(got[b], want_idx[b]), f"sequence {b} call {rep}"
    say("  early stops after passes 1, 2, 3 and the all-ties case bit-exact")


def test_selection_two_workgroups_match_one():
    """With a workspace, a sequence whose two tiers are both non-empty (|D| + |T| <= 4096)
    runs them on two workgroups, the second to finish combining them; without one, one
    workgroup runs both in turn.  Both must give the oracle's set bit for bit: ragged
    contexts at 32 and 64 keys per thread, nine sequences (a second, partial group of
    eight), ties (quantised scores) in the tiers and in the combined candidates, candidate
    lists of up to 2 and up to 4 per thread, a sequence above the 4096 cap, one with
    m = 0, one with the budget at least the context, one whose draft tier fills the
    budget, and a workspace that starts with random bytes."""
    from sparse_kv_attention_amd import dustin as D
    B, n_max, k_max = 9, 40000, 5000
    ctx = np.array([32768, 40000, 30001, 12000, 500, 20000, 32768, 40000, 39999], dtype=np.int32)
    budget = np.array([2048, 2048, 1777, 2900, 600, 1024, 2048, 4800, 4000], dtype=np.int32)
    sink = np.array([16, 16, 3, 16, 4, 16, 16, 16, 16], dtype=np.int32)
    window = np.array([256, 256, 40, 256, 8, 128, 256, 256, 100], dtype=np.int32)
    m = np.array([768, 768, 1000, 768, 100, 0, 2000, 768, 1500], dtype=np.int32)
    gen = np.random.default_rng(77)
    sd = gen.uniform(0, 1e-3, (B, n_max)).astype(np.float32)
    st = gen.uniform(0, 1e-3, (B, n_max)).astype(np.float32)
    sd[2] = np.round(sd[2] * 3000) / 3000
    st[2] = np.round(st[2] * 3000) / 3000
    st[8] = np.round(st[8] * 5e5) / 5e5          # ties among the combined candidates
    want_idx, want_cnt = O.select(ctx, sd, st, budget, sink, window, m, k_max)
    dev = "cuda"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ws = D.workspace(D.dustin_select_workspace_size(B, n_max), dev)
    ws.copy_(torch.from_numpy(gen.integers(0, 256, ws.numel(), dtype=np.uint8)).to(dev))
    got = {}
    for name, w in (("two workgroups", ws), ("one workgroup", None), ("two workgroups again", ws)):
        idx = torch.full((B, k_max), -5, dtype=torch.int32, device=dev)
        cnt = torch.zeros((B,), dtype=torch.int32, device=dev)
        D.dustin_select(t(ctx), t(sd), t(st), t(budget), t(sink), t(window), t(m), idx, cnt, w)
        torch.cuda.synchronize()
        assert np.array_equal(cnt.cpu().numpy(), want_cnt), name
        got[name] = idx.cpu().numpy()
        for b in range(B):
            assert np.array_equal(got[name][b], want_idx[b]), f"{name}: sequence {b}"
    say("  two-workgroup and one-workgroup selection identical to the oracle")


def test_selection_at_64k_positions():
    """The widest selection variant (64 keys per thread) at its size limit, through the C
    ABI with and without a workspace, against the oracle: a sequence whose two tiers sum to
    exactly the 4096-candidate cap (two workgroups), one just above it (one workgroup), a
    budget above the LDS staging area (the ordered set written without staging), and
    quantised scores (ties) in the combined candidates."""
    from sparse_kv_attention_amd import dustin as D
    B, n_max, k_max = 4, 65536, 17000
    ctx = np.array([65536, 65536, 65535, 40000], dtype=np.int32)
    budget = np.array([4368, 4369, 17000, 3000], dtype=np.int32)   # r + m = 4096, 4097, ...
    sink = np.array([16, 16, 16, 7], dtype=np.int32)
    window = np.array([256, 256, 512, 100], dtype=np.int32)
    m = np.array([1500, 1500, 6000, 2000], dtype=np.int32)
    gen = np.random.default_rng(88)
    sd = gen.uniform(0, 1e-4, (B, n_max)).astype(np.float32)
    st = gen.uniform(0, 1e-4, (B, n_max)).astype(np.float32)
    st[0] = np.round(st[0] * 2e5) / 2e5
    want_idx, want_cnt = O.select(ctx, sd, st, budget, sink, window, m, k_max)
    dev = "cuda"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ws = D.workspace(D.dustin_select_workspace_size(B, n_max), dev)
    for name, w in (("two workgroups", ws), ("one workgroup", None)):
        idx = torch.full((B, k_max), -5, dtype=torch.int32, device=dev)
        cnt = torch.zeros((B,), dtype=torch.int32, device=dev)
        D.dustin_select(t(ctx), t(sd), t(st), t(budget), t(sink), t(window), t(m), idx, cnt, w)
        torch.cuda.synchronize()
        assert np.array_equal(cnt.cpu().numpy(), want_cnt), name
        got = idx.cpu().numpy()
        for b in range(B):
            assert np.array_equal(got[b], want_idx[b]), f"{name}: sequence {b}"
    say("  64k-position selection identical to the oracle on both paths")


def test_context_above_32k():
    """Contexts of 30k..50k tokens (ragged): 64 keys per selection thread (the widest
    selection variant), scoring over 50k-token rows, a 4096-token budget over two splits
    and more; every stage against the oracle."""
    w = W.shrink(small("long_ctx", 3, 50000, 8, 2, 128, 4, 4096, 4, 64, 1024, seed=25), ragged_lo=30000)
    inp = W.make_inputs(w, device="cuda")
    assert inp.n_max > 32768
    check_pipeline(inp, [0], [], [0, 1, 2])


def test_selection_parameter_edges():
    """Per-sequence parameters at their edges, through the C ABI against the oracle:
    empty and 1-token contexts, budgets of 0 and above k_max, sinks alone exceeding the
    budget, sinks + window exceeding it, m above what is left and m = 0, on scores with
    many ties (quantised), -0/+0 and negative values; 5000 positions (5 keys per thread,
    the scalar-load path at a length that is not a multiple of 4)."""
    from sparse_kv_attention_amd import dustin as D
    B, n_max, k_max = 10, 4999, 700
    ctx = np.array([0, 1, 4999, 3000, 2500, 4000, 700, 701, 4999, 1234], dtype=np.int32)
    budget = np.array([5, 5, 0, 10000, 64, 300, 700, 700, 512, 200], dtype=np.int32)
    sink = np.array([2, 4, 3, 16, 100, 8, 0, 700, 4, 0], dtype=np.int32)
    window = np.array([1, 4, 3, 64, 10, 400, 0, 1, 32, 0], dtype=np.int32)
    m = np.array([1, 1, 5, 100, 5, 50, 350, 3, 10000, 0], dtype=np.int32)
    gen = np.random.default_rng(41)
    sd = np.round(gen.normal(0, 1, (B, n_max)) * 4) / 4           # few distinct values: ties
    st = np.round(gen.normal(0, 1, (B, n_max)) * 16) / 16
    sd[4, ::7] = -0.0
    sd[4, 1::7] = 0.0
    st[9] = 0.0
    sd, st = sd.astype(np.float32), st.astype(np.float32)
    dev = "cuda"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    idx = torch.full((B, k_max), -5, dtype=torch.int32, device=dev)
    cnt = torch.zeros((B,), dtype=torch.int32, device=dev)
    ws = D.workspace(D.dustin_select_workspace_size(B, n_max), dev)
    for draft in (sd, None):
        D.dustin_select(t(ctx), None if draft is None else t(draft), t(st), t(budget), t(sink), t(window),
                        t(m), idx, cnt, ws)
        torch.cuda.synchronize()
        want_idx, want_cnt = O.select(ctx, draft, st, budget, sink, window, m, k_max)
        assert np.array_equal(cnt.cpu().numpy(), want_cnt), (cnt.cpu().numpy(), want_cnt)
        got = idx.cpu().numpy()
        for b in range(B):
            assert np.array_equal(got[b], want_idx[b]), f"sequence {b}, draft tier {draft is not None}"
    say(f"  counts {want_cnt.tolist()} bit-exact, with and without the draft tier")


def test_one_query_head_per_kv_head():
    """Multi-head attention (G = 1): five verify rows per KV head, one query tile with
    eleven padding rows; head dim 128 and 64."""
    for name, w in (("mha_d128", small("mha_d128", 3, 900, 4, 4, 128, 4, 200, 4, 16, 40, seed=26)),
                    ("mha_d64", small("mha_d64", 2, 700, 6, 6, 64, 2, 150, 2, 8, 30, seed=27))):
        say(f"[{name}]")
        check_pipeline(W.make_inputs(w, device="cuda"), [0], [0], [0, 1])


def test_negative_and_zero_scales():
    """Any finite softmax scale: a negative one (the attention kernels move the sign into
    Q; the scoring kernels multiply it in fp64) and zero (uniform softmax: every token
    scores its pair count / N, so selection falls back to position order, and O is the
    mean of the attended V rows), scoring, selection, sparse and dense attention against
    the oracle."""
    w = small("scales", 2, 900, 8, 2, 128, 4, 200, 4, 16, 40, seed=28)
    inp = W.make_inputs(w, device="cuda")
    for sc in (-0.09, 0.0):
        say(f"[scale {sc}]")
        step = step_for(inp, [0])
        step.scale = sc
        step.scale_draft = sc
        step.score()
        torch.cuda.synchronize()
        sd = step.score_draft.cpu().numpy()
        st = step.score_target.cpu().numpy()
        check_scores(sd, oracle_scores(inp, "draft", O.PROB_SUM, [0, 1], scale=sc), "draft scores")
        check_scores(st, oracle_scores(inp, "target", O.PROB_SUM, [0, 1], scale=sc), "target scores")
        step.select()
        torch.cuda.synchronize()
        idx_o, cnt_o = oracle_select_on(inp, sd.astype(np.float64), st.astype(np.float64), [0, 1])
        idx_g, cnt_g = step.idx.cpu().numpy(), step.count.cpu().numpy()
        assert np.array_equal(cnt_g, cnt_o) and np.array_equal(idx_g[:, :inp.k_max], idx_o)
        step.attn(0)
        torch.cuda.synchronize()
        check_attn(step.out, step.lse, oracle_attn(inp, 0, idx_g, cnt_g, [0, 1], scale=sc), [0, 1], "sparse")
        step.dense(0)
        torch.cuda.synchronize()
        check_attn(step.out, step.lse, oracle_attn(inp, 0, None, None, [0, 1], dense=True, scale=sc), [0, 1],
                   "dense")


def test_single_query_signals():
    """gamma = 1: each draft group scores one (head, query) pair, the narrowest softmax
    variant; gamma = 0 with the Collect-2 signal: one verify query, which the logit sum
    counts once (first and bonus query coincide)."""
    w = small("gamma1", 2, 800, 8, 2, 128, 1, 150, 2, 8, 30, seed=29)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [], [0, 1])
    w = small("collect2_nq1", 2, 900, 8, 2, 128, 0, 120, 0, 0, 0, seed=30)
    check_pipeline(W.make_inputs(w, device="cuda"), [0], [], [0, 1], logit_sum2=True)


def floor_xor(kc: torch.Tensor, vc: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    """[B][Hkv] XOR of every 32-bit word of the K and V rows of idx (clamped to the cache):
    what dustin_gather_floor's checksum mode computes, from its definition."""
    n = kc.shape[1]
    k32 = kc.contiguous().view(torch.int16).numpy().view(np.uint32)
    v32 = vc.contiguous().view(torch.int16).numpy().view(np.uint32)
    tok = np.clip(idx, 0, n - 1)
    out = np.zeros((kc.shape[0], kc.shape[2]), dtype=np.uint32)
    for b in range(kc.shape[0]):
        out[b] = (np.bitwise_xor.reduce(k32[b, tok[b]], axis=(0, 2))
                  ^ np.bitwise_xor.reduce(v32[b, tok[b]], axis=(0, 2)))
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_gather_floor_reads_the_list_rows(d):
    """The gather-floor call reads exactly the list rows: its XOR checksum over a ragged
    list (three workgroups of 512, 512 and 276 entries) with out-of-range entries (clamped)
    matches the XOR of those rows on the host; the timing mode leaves the checksum alone."""
    from sparse_kv_attention_amd import dustin as D
    g = torch.Generator().manual_seed(41 + d)
    B, N, Hkv, k_max = 3, 2500, 3, 1300
    kc = torch.randn((B, N, Hkv, d), generator=g).to(torch.bfloat16)
    vc = torch.randn((B, N, Hkv, d), generator=g).to(torch.bfloat16)
    idx = torch.randint(-40, N + 40, (B, k_max), generator=g, dtype=torch.int32)
    kd, vd, idd = kc.cuda(), vc.cuda(), idx.cuda()
    ck = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    D.dustin_gather_floor(D.kv_view(kd), D.kv_view(vd), Hkv, d, idd, ck, mode=1)
    torch.cuda.synchronize()
    assert np.array_equal(ck.cpu().numpy().view(np.uint32), floor_xor(kc, vc, idx.numpy()))
    ck0 = torch.full((B, Hkv), 7, dtype=torch.int32, device="cuda")
    D.dustin_gather_floor(D.kv_view(kd), D.kv_view(vd), Hkv, d, idd, ck0, mode=0)
    torch.cuda.synchronize()
    assert bool((ck0 == 7).all())
