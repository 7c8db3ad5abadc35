"""dustin_sparse_verify_attn_noalloc (no workspace argument: the split partials live in the
library's static scratch array) against dustin_sparse_verify_attn with a workspace: the
same kernels under the same split plan, so the results must agree bit for bit.  Two calls
in a row on the one array, the second with a smaller input, then the larger one again;
once with the split merge kernel and once with the merge fused into the attention kernel
(whose arrival counters then live in the scratch array too)."""
import os
import re

import numpy as np
import pytest
import torch

from _harness import check_attn, oracle_attn, say
from sparse_kv_attention_amd import dustin as D
from sparse_kv_attention_amd import workloads as W
from sparse_kv_attention_amd.workloads import ModelShape, Workload

pytestmark = pytest.mark.gpu

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dustin.h")


def scratch_limit():
    m = re.search(r"#define DUSTIN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def case(name, B, n, hq, hkv, d, gamma, budget, seed):
    w = Workload(name=name, batch=B, n_ctx=n, target=ModelShape(1, hq, hkv, d),
                 draft=ModelShape(1, 2, 2, 64), gamma=gamma, budget=budget, n_sink=4, n_window=32,
                 m=budget // 4, srh_draft=((0, 0), (0, 1)), srh_target=((0, 0),), seed=seed)
    inp = W.make_inputs(w, device="cuda")
    # a sorted list of distinct positions per sequence, `budget` long where the context allows
    gen = torch.Generator().manual_seed(seed)
    ctx = inp.ctx_len.cpu().tolist()
    idx = torch.full((B, budget), -1, dtype=torch.int32)
    cnt = torch.zeros(B, dtype=torch.int32)
    for b in range(B):
        k = min(budget, ctx[b])
        pos = torch.sort(torch.randperm(ctx[b], generator=gen)[:k]).values
        idx[b, :k] = pos.to(torch.int32)
        cnt[b] = k
    return inp, idx.cuda(), cnt.cuda()


def run_pair(inp, idx, cnt):
    w = inp.w
    q = inp.q_verify[0]
    kv = (D.kv_view(inp.k_cache[0]), D.kv_view(inp.v_cache[0]))
    B, nv, Hq, d = q.shape
    scale = 1.0 / d ** 0.5
    ws_bytes = D.dustin_sparse_verify_attn_workspace_size(B, Hq, w.target.hkv, d, nv, idx.shape[1])
    assert 0 < ws_bytes <= scratch_limit(), ws_bytes          # the case uses split partials
    ws = D.workspace(ws_bytes, q.device)
    out_w, lse_w = torch.empty_like(q), torch.empty((B, Hq, nv), dtype=torch.float32, device=q.device)
    out_n, lse_n = torch.full_like(q, float("nan")), torch.full((B, Hq, nv), float("nan"), device=q.device)
    D.dustin_sparse_verify_attn(q, kv[0], kv[1], w.target.hkv, inp.ctx_len, idx, cnt, scale, out_w, lse_w, ws)
    D.dustin_sparse_verify_attn_noalloc(q, kv[0], kv[1], w.target.hkv, inp.ctx_len, idx, cnt, scale, out_n, lse_n)
    return out_w, lse_w, out_n, lse_n, scale


@pytest.mark.parametrize("fused", ["0", "1"])
def test_noalloc_matches_the_workspace_entry_point(fused):
    old = os.environ.get("DUSTIN_ATTN_FUSED_MERGE")
    os.environ["DUSTIN_ATTN_FUSED_MERGE"] = fused
    try:
        big = case("noalloc_big", 3, 3000, 16, 2, 128, 4, 1100, seed=31)
        smaller = case("noalloc_small", 2, 900, 8, 2, 64, 2, 300, seed=32)
        for what, (inp, idx, cnt) in (("larger", big), ("smaller", smaller), ("larger again", big)):
            say(f"[noalloc, fused merge {fused}] {what} call: B={inp.w.batch} n={inp.w.n_ctx} "
                f"d={inp.w.target.d} k_max={idx.shape[1]}")
            out_w, lse_w, out_n, lse_n, scale = run_pair(inp, idx, cnt)
            torch.cuda.synchronize()
            assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w), what
            bs = list(range(inp.w.batch))
            ref = oracle_attn(inp, 0, idx.cpu().numpy(), cnt.cpu().numpy(), bs, scale=scale)
            check_attn(out_n, lse_n, ref, bs, f"noalloc, {what}")
    finally:
        if old is None:
            os.environ.pop("DUSTIN_ATTN_FUSED_MERGE", None)
        else:
            os.environ["DUSTIN_ATTN_FUSED_MERGE"] = old
