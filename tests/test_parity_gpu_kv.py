"""GPU parity of the verified block in the cache (English Dustin summary, Verification
Workflow step 5) and of the attention-recovery measurement, through the C ABI.

Bars: the block write and the commit are byte/integer work, so bit-exact against the
oracle; recovery is exp(LSE_sparse - LSE_dense) of two attention calls whose LSEs are
each within 1e-3 of the oracle's, so it is checked within exp(2e-3) - 1 relative of the
oracle's direct sum of dense probabilities over the kept set.
"""
import math

import numpy as np
import pytest
import torch

from _harness import LSE_ATOL, check_scores, rows, say, u16
from oracle import oracle as O
from sparse_kv_attention_amd import dustin as D
from sparse_kv_attention_amd import workloads as W
from sparse_kv_attention_amd.pipeline import SparseVerifyStep
from test_parity_gpu import check_pipeline, small

pytestmark = pytest.mark.gpu

REC_RTOL = math.exp(2 * LSE_ATOL) - 1.0


def logical(inp, cache, n_rows):
    return np.stack([u16(rows(inp, cache, b, n_rows)) for b in range(inp.w.batch)])


def allocated_rows(inp):
    """Rows of each sequence that its own pages hold (all rows when contiguous)."""
    if not inp.paged:
        return [inp.n_cap] * inp.w.batch
    ps = inp.w.page_size
    ctx = inp.ctx_len.cpu().numpy()
    return [(int(ctx[b]) + inp.w.n_verify + ps - 1) // ps * ps for b in range(inp.w.batch)]


def check_write(inp, n_new, ctx_override=None, seed=0):
    w = inp.w
    T = w.target
    B = w.batch
    g = torch.Generator(device="cuda").manual_seed(seed)
    kn = torch.randn((B, n_new, T.hkv, T.d), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, n_new, T.hkv, T.d), generator=g, device="cuda").to(torch.bfloat16)
    ctx = inp.ctx_len if ctx_override is None else ctx_override
    kc, vc = inp.k_cache[0], inp.v_cache[0]
    n_rows = max(allocated_rows(inp))
    k_before, v_before = logical(inp, kc, n_rows), logical(inp, vc, n_rows)
    phys_k, phys_v = kc.clone(), vc.clone()
    step = SparseVerifyStep(inp, layers=[0])
    say(f"[{w.name}] kv write block n_new={n_new} paged={inp.paged}")
    step.write_block(0, kn, vn, ctx_len=ctx)
    torch.cuda.synchronize()
    # the oracle on the clamped lengths (the view's capacity bounds where a block may go)
    cap = kc.shape[1] if not inp.paged else inp.page_table.shape[1] * w.page_size
    ctx_c = np.clip(ctx.cpu().numpy(), 0, cap - n_new).astype(np.int32)
    k_want, v_want = O.kv_write_block(u16(kn), u16(vn), ctx_c, k_before, v_before)
    k_got, v_got = logical(inp, kc, n_rows), logical(inp, vc, n_rows)
    for b, n_alloc in enumerate(allocated_rows(inp)):
        assert np.array_equal(k_got[b, :n_alloc], k_want[b, :n_alloc]), f"K rows of sequence {b}"
        assert np.array_equal(v_got[b, :n_alloc], v_want[b, :n_alloc]), f"V rows of sequence {b}"
    # no physical row outside the block changed
    changed = int((kc != phys_k).any(-1).sum() + (vc != phys_v).any(-1).sum())
    assert changed <= 2 * B * n_new * T.hkv, changed
    say(f"  bit-exact; {changed} physical head rows rewritten")


def test_write_block_contiguous_head_dim_64():
    inp = W.make_inputs(W.TINY, device="cuda")
    check_write(inp, inp.w.n_verify)


def test_write_block_contiguous_widest_block_at_capacity():
    w = small("kv_edges", 4, 400, 8, 2, 128, 15, 64, 4, 8, 16, seed=21)
    inp = W.make_inputs(w, device="cuda")
    # lengths 0, the largest that fits, and out-of-range values the kernel clamps
    ctx = torch.tensor([0, inp.n_cap - 16, -7, 1 << 30], dtype=torch.int32, device="cuda")
    check_write(inp, 16, ctx_override=ctx, seed=1)
    check_write(inp, 1, seed=2)


def test_write_block_paged():
    w = W.shrink(W.RAGGED_PAGED, batch=6, n_ctx=3000, ragged_lo=700, target=W.ModelShape(1, 64, 8, 128),
                 srh_target=((0, 0),))
    inp = W.make_inputs(w, device="cuda")
    check_write(inp, w.n_verify, seed=3)


def test_write_block_qwen72b_layer_full_size():
    inp = W.make_inputs(W.shrink(W.QWEN72B, target=W.ModelShape(1, 64, 8, 128), srh_target=((0, 0),),
                                 needle_mode="none"), device="cuda")
    check_write(inp, inp.w.n_verify, seed=4)
    del inp
    torch.cuda.empty_cache()


def test_round_trip_write_then_attend():
    # the new-token rows of the generated cache, moved out to a staging block, zeroed, and
    # written back by the library: attention must be bitwise what it was
    inp = W.make_inputs(W.shrink(W.QWEN7B, target=W.ModelShape(1, 28, 4, 128), srh_target=((0, 0),)),
                        device="cuda")
    step = SparseVerifyStep(inp, layers=[0])
    step.score()
    step.select()
    step.attn(0)
    o0, l0 = step.out.clone(), step.lse.clone()
    ctx = inp.ctx_len.cpu().tolist()
    nv = inp.w.n_verify
    kc, vc = inp.k_cache[0], inp.v_cache[0]
    kn = torch.stack([kc[b, ctx[b]:ctx[b] + nv] for b in range(inp.w.batch)]).contiguous()
    vn = torch.stack([vc[b, ctx[b]:ctx[b] + nv] for b in range(inp.w.batch)]).contiguous()
    for b in range(inp.w.batch):
        kc[b, ctx[b]:ctx[b] + nv] = 0
        vc[b, ctx[b]:ctx[b] + nv] = 0
    step.write_block(0, kn, vn)
    step.attn(0)
    torch.cuda.synchronize()
    assert torch.equal(step.out, o0) and torch.equal(step.lse, l0)


def test_commit():
    B, n_new = 37, 5
    rng = np.random.default_rng(7)
    ctx = rng.integers(0, 70000, B).astype(np.int32)
    acc = rng.integers(0, n_new, B).astype(np.int32)
    c_dev = torch.from_numpy(ctx).cuda()
    a_dev = torch.from_numpy(acc).cuda()
    D.dustin_kv_commit(a_dev, c_dev, n_new)
    torch.cuda.synchronize()
    assert np.array_equal(c_dev.cpu().numpy(), O.kv_commit(ctx, acc, n_new))
    # out-of-range acceptance counts act as their clamped values
    bad = np.array([-3, 99, 4, 0], np.int32)
    c_dev = torch.tensor([10, 10, 10, 10], dtype=torch.int32, device="cuda")
    D.dustin_kv_commit(torch.from_numpy(bad).cuda(), c_dev, n_new)
    torch.cuda.synchronize()
    assert np.array_equal(c_dev.cpu().numpy(), O.kv_commit([10] * 4, np.clip(bad, 0, n_new - 1), n_new))
    # out-of-range lengths act as their clamped values, [0, 2^30]
    lens = np.array([-5, 2 ** 31 - 1, 0, 2 ** 30], np.int32)
    c_dev = torch.from_numpy(lens).cuda()
    D.dustin_kv_commit(torch.tensor([1, 2, 3, 4], dtype=torch.int32, device="cuda"), c_dev, n_new)
    torch.cuda.synchronize()
    assert np.array_equal(c_dev.cpu().numpy(), O.kv_commit(np.clip(lens, 0, 2 ** 30), [1, 2, 3, 4], n_new))


def check_recovery(inp, layer, bsel, heads=None):
    w = inp.w
    T = w.target
    step = SparseVerifyStep(inp, layers=[layer])
    step.score()
    step.select()
    rec = step.recovery(layer)
    torch.cuda.synchronize()
    idx, cnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    ctx = inp.ctx_len.cpu().numpy()
    n_rows = int(ctx[bsel].max()) + w.n_verify
    got = rec.cpu().numpy()
    heads = list(range(T.hkv)) if heads is None else heads
    worst = 0.0
    for g in heads:                      # one KV head's query group at a time
        hs = slice(g * T.group, (g + 1) * T.group)
        K = np.stack([u16(rows(inp, inp.k_cache[layer], b, n_rows)[:, g:g + 1]) for b in bsel])
        Q = u16(inp.q_verify[layer][bsel][:, :, hs])
        ref = O.attn_recovery(Q, K, ctx[bsel], idx[bsel][:, :inp.k_max], cnt[bsel], 1.0 / math.sqrt(T.d), 1)
        err = np.abs(got[bsel][:, hs] - ref) / ref
        worst = max(worst, float(err.max()))
    say(f"  [{w.name}] recovery: mean {got[bsel].mean():.4f}, max rel err {worst:.3g} (bar {REC_RTOL:.3g})")
    assert worst <= REC_RTOL
    return got


def test_recovery_qwen7b():
    inp = W.make_inputs(W.QWEN7B, device="cuda", target_layers=[0])
    check_recovery(inp, 0, np.arange(4))


def test_recovery_full_budget_is_one():
    w = small("rec_full", 2, 300, 8, 2, 128, 4, 300, 4, 16, 40, seed=12)
    inp = W.make_inputs(w, device="cuda")
    got = check_recovery(inp, 0, np.arange(2))
    assert np.all(got == 1.0)


def test_recovery_ragged_paged():
    w = W.shrink(W.RAGGED_PAGED, batch=4, n_ctx=9000, ragged_lo=1000, target=W.ModelShape(1, 64, 8, 128),
                 srh_target=((0, 0), (0, 8)))
    inp = W.make_inputs(w, device="cuda")
    check_recovery(inp, 0, np.arange(4), heads=[0, 7])


def test_recovery_qwen72b_sampled():
    inp = W.make_inputs(W.QWEN72B, device="cuda", target_layers=[60])
    check_recovery(inp, 60, np.array([0]), heads=[0, 5])
    del inp
    torch.cuda.empty_cache()


def test_all_heads_estimator_widest_groups():
    """The naive estimator's calls: every query head of a 72B-shaped layer (groups of 3, 3
    and 2 heads x 5 queries = 15, 15, 10 pairs; calls of 16 and 8 groups) and of a draft
    layer (4 and 3 heads x 4 queries = 16, 12 pairs), each call against the oracle."""
    from sparse_kv_attention_amd.pipeline import AllHeadsEstimator
    w = W.shrink(W.QWEN72B, batch=2, n_ctx=1500, target=W.ModelShape(1, 64, 8, 128), srh_target=((0, 0),),
                 needle_mode="none")
    inp = W.make_inputs(w, device="cuda")
    ctx = inp.ctx_len.cpu().numpy()
    cases = (("target", inp.k_cache[0], inp.q_verify[0].permute(0, 2, 1, 3).contiguous(), w.target),
             ("draft", inp.draft_k[2], torch.randn((2, w.draft.hq, w.gamma, w.draft.d), device="cuda",
                                                    generator=torch.Generator(device="cuda").manual_seed(5)
                                                    ).to(torch.bfloat16), w.draft))
    for name, kc, q, shape in cases:
        est = AllHeadsEstimator(kc, None, q, shape.hkv, inp.ctx_len, 1.0 / math.sqrt(shape.d))
        est.score()
        torch.cuda.synchronize()
        say(f"[{name}] {len(est.calls)} calls, pairs per group {[nh * q.shape[2] for _, _, nh in est.calls[0][0]]}")
        for (groups, cq), got in zip(est.calls, est.scores):
            acc = np.zeros((2, est.n_max))
            h = 0
            for _, g, nh in groups:
                K = u16(kc[:, :est.n_max, g])
                O.score_stream(K, u16(cq[:, h:h + nh]), ctx, est.n_max, 1.0 / math.sqrt(shape.d), O.PROB_SUM, acc)
                h += nh
            check_scores(got.cpu().numpy(), acc, f"{name} all-heads call")


def test_all_heads_estimator_paged():
    """The estimator's widest groups on a paged, ragged cache: the page-table variant of the
    16-pair softmax kernel (one wave per SIMD at head dim 128) against the oracle."""
    from sparse_kv_attention_amd.pipeline import AllHeadsEstimator
    from sparse_kv_attention_amd.workloads import logical_rows
    w = W.shrink(W.RAGGED_PAGED, batch=3, n_ctx=3000, ragged_lo=900, target=W.ModelShape(1, 64, 8, 128),
                 srh_target=((0, 0),))
    inp = W.make_inputs(w, device="cuda")
    ctx = inp.ctx_len.cpu().numpy()
    q = inp.q_verify[0].permute(0, 2, 1, 3).contiguous()
    est = AllHeadsEstimator(inp.k_cache[0], inp.page_table, q, w.target.hkv, inp.ctx_len, 1.0 / math.sqrt(128))
    est.score()
    torch.cuda.synchronize()
    K_all = np.stack([u16(logical_rows(inp, inp.k_cache[0], b, est.n_max)) for b in range(w.batch)])
    for (groups, cq), got in zip(est.calls, est.scores):
        acc = np.zeros((w.batch, est.n_max))
        h = 0
        for _, g, nh in groups:
            O.score_stream(K_all[:, :, g], u16(cq[:, h:h + nh]), ctx, est.n_max, 1.0 / math.sqrt(128), O.PROB_SUM, acc)
            h += nh
        check_scores(got.cpu().numpy(), acc, "paged all-heads call")


@pytest.mark.parametrize("all_queries", [False, True])
def test_vegas_aggregate_over_every_head_of_a_layer(all_queries):
    """The Vegas aggregate in its literal form (German Vegas summary 2A/2B): logits of the
    first and bonus verify queries (or all of them) summed over all 64 query heads of one
    target layer, on a ragged paged cache; then pure top-k selection, bit-exact."""
    w = W.shrink(W.RAGGED_PAGED, batch=3, n_ctx=4000, ragged_lo=1200, target=W.ModelShape(1, 64, 8, 128),
                 srh_target=((0, 0),))
    inp = W.make_inputs(w, device="cuda")
    step = SparseVerifyStep(inp, layers=[0], logit_sum2=True)
    step.vegas_all_heads(0, step.score_target, all_queries=all_queries)
    step.select()
    torch.cuda.synchronize()
    ctx = inp.ctx_len.cpu().numpy()
    n = inp.n_max
    q = inp.q_verify[0].permute(0, 2, 1, 3).contiguous()
    mode = O.LOGIT_SUM_ALL if all_queries else O.LOGIT_SUM2
    acc = np.zeros((w.batch, n))
    cond = np.zeros((w.batch, n))
    G = w.target.group
    js = list(range(w.n_verify)) if all_queries else [0, w.n_verify - 1]
    for g in range(w.target.hkv):
        Kg = np.stack([u16(rows(inp, inp.k_cache[0], b, n)[:, g]) for b in range(w.batch)])
        O.score_stream(Kg, u16(q[:, g * G:(g + 1) * G]), ctx, n, 1.0 / math.sqrt(128), mode, acc)
        for b in range(w.batch):
            Kd = rows(inp, inp.k_cache[0], b, n)[:, g].double().cpu()
            Qd = q[b, g * G:(g + 1) * G][:, js].double().cpu().reshape(-1, 128)
            cond[b] += (Kd @ Qd.T).abs().sum(1).numpy() / math.sqrt(128)
    got = step.score_target.cpu().numpy()
    check_scores(got, acc, "all-heads Vegas aggregate", cond=cond)
    zeros = np.zeros(w.batch, np.int32)
    idx_o, cnt_o = O.select(ctx, None, got.astype(np.float64), inp.budget.cpu().numpy(), zeros, zeros, zeros,
                            inp.k_max)
    assert np.array_equal(step.count.cpu().numpy(), cnt_o)
    assert np.array_equal(step.idx.cpu().numpy()[:, :inp.k_max], idx_o)


def test_page_size_one():
    """Pages of one token (the page-size-1 layout of the Vegas summary's PagedAttention
    change): every row is reached through its own page-table entry.  Scoring, selection,
    sparse and dense attention against the oracle, then the verified block written through
    the one-token pages."""
    w = W.shrink(W.RAGGED_PAGED, batch=3, n_ctx=2500, ragged_lo=600, page_size=1,
                 target=W.ModelShape(1, 64, 8, 128), srh_target=((0, 0), (0, 8)))
    inp = W.make_inputs(w, device="cuda")
    assert inp.paged and w.page_size == 1
    ctx = inp.ctx_len.cpu().numpy()
    check_pipeline(inp, [0], [0], b_attn=[int(np.argmin(ctx)), int(np.argmax(ctx))], b_dense=[int(np.argmin(ctx))])
    check_write(inp, w.n_verify, seed=5)
