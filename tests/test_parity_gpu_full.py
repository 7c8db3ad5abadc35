"""GPU parity at the full workload sizes, in the launch configuration the bench times.

Scores and selection are checked for every sequence (selection bit-exact on the GPU's
own scores); attention on sampled sequences and layers, where the oracle computes each
output row one by one.
"""
import numpy as np
import pytest
import torch

from _harness import say
from sparse_kv_attention_amd import workloads as W
from test_parity_gpu import check_pipeline, floor_xor

pytestmark = pytest.mark.gpu


def test_qwen72b_b8_n32768_sampled():
    inp = W.make_inputs(W.QWEN72B, device="cuda", target_layers=[0, 79])
    step = check_pipeline(inp, [0, 79], [0], b_attn=[0, 5], b_dense=[0])
    # each sequence's 327 planted needles are strongly preferred by both signals
    sel = step.idx.cpu().numpy()
    for b in range(inp.w.batch):
        hit = np.isin(inp.needles[b].numpy(), sel[b]).mean()
        say(f"  needles kept in sequence {b}: {hit:.3f}")
        assert hit > 0.9
    # the gather floor the bench times reads exactly layer 0's rows of the selected lists
    from sparse_kv_attention_amd import dustin as D
    T = inp.w.target
    idx = step.idx[:, :inp.k_max].contiguous()
    ck = torch.zeros((inp.w.batch, T.hkv), dtype=torch.int32, device="cuda")
    D.dustin_gather_floor(D.kv_view(inp.k_cache[0]), D.kv_view(inp.v_cache[0]), T.hkv, T.d, idx, ck, mode=1)
    torch.cuda.synchronize()
    assert np.array_equal(ck.cpu().numpy().view(np.uint32),
                          floor_xor(inp.k_cache[0].cpu(), inp.v_cache[0].cpu(), idx.cpu().numpy()))
    del step, inp
    torch.cuda.empty_cache()


DENSE_POINTS = {(1024, 2, 0.25), (2048, 4, 0.5), (4096, 8, 0.5)}


@pytest.mark.parametrize("k,g,r", [(k, g, r) for k in (1024, 2048, 4096) for g in (2, 4, 8) for r in (0.25, 0.5)])
def test_sweep_b64_point(k, g, r):
    # every point of the budget x gamma x m/budget grid; dense attention at one point per
    # budget and gamma class
    inp = W.make_inputs(W.sweep_point(k, g, r), device="cuda")
    dense = (k, g, r) in DENSE_POINTS
    check_pipeline(inp, [0], [0] if dense else [], b_attn=[0, 63], b_score=[0, 31, 63], b_dense=[0])
    del inp
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def paged():
    inp = W.make_inputs(W.RAGGED_PAGED, device="cuda", target_layers=[0, 79])
    yield inp
    del inp
    torch.cuda.empty_cache()


def test_ragged_paged_hybrid(paged):
    ctx = paged.ctx_len.cpu().numpy()
    lo, hi = int(np.argmin(ctx)), int(np.argmax(ctx))
    say(f"  contexts {ctx.min()}..{ctx.max()}, budgets {paged.budget.min().item()}..{paged.budget.max().item()}")
    check_pipeline(paged, [0, 79], [0], b_attn=[lo, hi], b_dense=[lo])


def test_ragged_paged_logit_sum2_topk(paged):
    ctx = paged.ctx_len.cpu().numpy()
    check_pipeline(paged, [0], [], b_attn=[int(np.argmax(ctx))], logit_sum2=True)


def test_ragged_paged_logit_sum_all_topk(paged):
    ctx = paged.ctx_len.cpu().numpy()
    check_pipeline(paged, [79], [], b_attn=[int(np.argmin(ctx))], logit_sum_all=True)


def test_qwen72b_every_layer():
    """All 80 layers resident (each with its own caches, as the bench runs them): sparse
    attention of every layer for sequence 0, and of layers 0, 40 and 79 for every sequence,
    against the oracle, on the GPU's own selection."""
    from _harness import check_attn, oracle_attn
    from sparse_kv_attention_amd.pipeline import SparseVerifyStep
    inp = W.make_inputs(W.QWEN72B, device="cuda")
    step = SparseVerifyStep(inp)
    step.score()
    step.select()
    torch.cuda.synchronize()
    idx, cnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    for l in range(inp.w.target.layers):
        step.attn(l)
        torch.cuda.synchronize()
        bsel = list(range(inp.w.batch)) if l in (0, 40, 79) else [0]
        check_attn(step.out, step.lse, oracle_attn(inp, l, idx, cnt, bsel), bsel, f"layer {l}")
    del step, inp
    torch.cuda.empty_cache()
