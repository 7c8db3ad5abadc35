"""Randomised GPU parity sweep: many small seeded shapes through the C ABI against the
oracle, covering the corners the named workloads do not: contexts of 1..64 tokens
(ragged per sequence), lists from empty to the whole context, 1..9 verify queries
(gamma 0..8), 1, 2, 7 or 8 query heads per KV head, head dims 64 and 128, contiguous and
paged caches (pages of 1, 4 or 16 tokens).  Same bars as the other parity tests:
attention output max-abs 2e-2 and LSE 1e-3, selection bit-exact, scores 1e-5 relative.
Every case prints its seed and shape before it runs."""
import math

import numpy as np
import pytest
import torch

from _harness import SCORE_ATOL, SCORE_RTOL, say
from oracle import oracle as O
from sparse_kv_attention_amd import dustin as D

pytestmark = pytest.mark.gpu

ATTN_CASES = 48
SELECT_CASES = 48
SCORE_CASES = 24


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_randn(shape, gen):
    return torch.randn(shape, generator=gen).to(torch.bfloat16)


def paged(x: torch.Tensor, page_size: int, pt: torch.Tensor):
    """x [B][cap][H][d] (cpu) -> pages [B*npg][page_size][H][d] placed by page table pt [B][npg]."""
    B, cap, H, d = x.shape
    npg = pt.shape[1]
    padded = torch.zeros((B, npg * page_size, H, d), dtype=x.dtype)
    padded[:, :cap] = x
    pages = torch.zeros((B * npg, page_size, H, d), dtype=x.dtype)
    pages[pt.reshape(-1).long()] = padded.view(B * npg, page_size, H, d)
    return pages


def attn_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 7, 8]))
    d = int(rng.choice([64, 128]))
    nv = int(rng.integers(1, 10))
    N = rng.integers(1, 65, size=B).astype(np.int32)
    N[rng.integers(0, B)] = int(rng.choice([1, 64, int(N.max())]))
    k_max = max(1, int(N.max()) + int(rng.integers(-8, 9)))
    counts = np.array([int(rng.integers(0, min(k_max, n) + 1)) for n in N], dtype=np.int32)
    if rng.random() < 0.3:
        counts = np.minimum(N, k_max).astype(np.int32)             # the whole context when it fits
    page = int(rng.choice([0, 1, 4, 16]))
    return B, Hkv, G, d, nv, N, k_max, counts, page


@pytest.mark.parametrize("seed", range(ATTN_CASES))
def test_attention_random_shapes(seed):
    B, Hkv, G, d, nv, N, k_max, counts, page = attn_case(seed)
    say(f"[sweep attn seed {seed}] B={B} Hkv={Hkv} G={G} d={d} nv={nv} N={N.tolist()} k_max={k_max} "
        f"counts={counts.tolist()} page={page}")
    gen = torch.Generator().manual_seed(1000 + seed)
    Hq = Hkv * G
    cap = int(N.max()) + nv
    K = bf16_randn((B, cap, Hkv, d), gen)
    V = bf16_randn((B, cap, Hkv, d), gen)
    Q = bf16_randn((B, nv, Hq, d), gen)
    idx = np.full((B, k_max), -1, dtype=np.int32)
    rng = np.random.default_rng(seed)
    for b in range(B):
        idx[b, :counts[b]] = np.sort(rng.choice(int(N[b]), size=int(counts[b]), replace=False))
    scale = 1.0 / math.sqrt(d)
    ora = O.verify_attn(u16(Q), u16(K), u16(V), N, idx, counts, scale, Hkv)
    orad = O.verify_attn(u16(Q), u16(K), u16(V), N, None, None, scale, Hkv)
    if page:
        # K and V under one page table, or (every other case) each under its own
        npg = (cap + page - 1) // page
        ptk = torch.randperm(B * npg, generator=gen).to(torch.int32).view(B, npg)
        ptv = ptk if seed % 2 else torch.randperm(B * npg, generator=gen).to(torch.int32).view(B, npg)
        keep = (paged(K, page, ptk).cuda(), paged(V, page, ptv).cuda(), ptk.cuda(), ptv.cuda())
        kv = (D.kv_view(keep[0], keep[2]), D.kv_view(keep[1], keep[3]))
    else:
        keep = (K.cuda(), V.cuda())
        kv = (D.kv_view(keep[0]), D.kv_view(keep[1]))
    q = Q.cuda()
    ctx = torch.from_numpy(N).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, nv), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dustin_sparse_verify_attn_workspace_size(B, Hq, Hkv, d, nv, k_max))
    D.dustin_sparse_verify_attn(q, kv[0], kv[1], Hkv, ctx, torch.from_numpy(idx).cuda(),
                                torch.from_numpy(counts).cuda(), scale, out, lse, ws)
    outd = torch.empty_like(q)
    lsed = torch.empty_like(lse)
    wsd = D.workspace(D.dense_verify_attn_workspace_size(B, Hq, Hkv, d, nv, int(N.max())))
    D.dense_verify_attn(q, kv[0], kv[1], Hkv, ctx, int(N.max()), scale, outd, lsed, wsd)
    torch.cuda.synchronize()
    for what, (o, l), (ro, rl) in (("sparse", (out, lse), ora), ("dense", (outd, lsed), orad)):
        eo = float(np.max(np.abs(o.float().cpu().numpy() - ro)))
        el = float(np.max(np.abs(l.cpu().numpy() - rl)))
        assert eo <= 2e-2 and el <= 1e-3, (seed, what, eo, el)
    del keep


@pytest.mark.parametrize("seed", range(SELECT_CASES))
def test_selection_random_parameters(seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 5))
    n_max = int(rng.choice([1, 7, 64, 300, 1000, 4096]))
    N = rng.integers(0, n_max + 1, size=B).astype(np.int32)
    k_max = int(rng.integers(0, n_max + 3))
    budget = rng.integers(-2, n_max + 3, size=B).astype(np.int32)
    sink = rng.integers(-1, 20, size=B).astype(np.int32)
    window = rng.integers(-1, 40, size=B).astype(np.int32)
    m = rng.integers(-1, 200, size=B).astype(np.int32)
    levels = int(rng.choice([3, 50, 1 << 20]))        # few levels = many ties
    sd = (rng.integers(0, levels, size=(B, n_max)) / levels).astype(np.float32)
    st = (rng.integers(0, levels, size=(B, n_max)) / levels).astype(np.float32)
    st[rng.random((B, n_max)) < 0.05] *= -1.0           # negative scores and -0
    no_draft = rng.random() < 0.25
    say(f"[sweep select seed {seed}] B={B} n_max={n_max} N={N.tolist()} k_max={k_max} budget={budget.tolist()} "
        f"levels={levels} draft={'no' if no_draft else 'yes'}")
    idx_o, cnt_o = O.select(N, None if no_draft else sd.astype(np.float64), st.astype(np.float64), budget, sink,
                            window, m, k_max)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx = torch.full((B, k_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws_b = D.dustin_select_workspace_size(B, n_max)
    D.dustin_select(cu(N), None if no_draft else cu(sd), cu(st), cu(budget), cu(sink), cu(window), cu(m), idx, cnt,
                    D.workspace(ws_b) if ws_b else None)
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), cnt_o), seed
    assert np.array_equal(idx.cpu().numpy(), idx_o), seed


@pytest.mark.parametrize("seed", range(SCORE_CASES))
def test_scoring_random_shapes(seed):
    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    n_q = int(rng.integers(1, 10))
    mode = int(rng.choice([O.PROB_SUM, O.LOGIT_SUM2, O.LOGIT_SUM_ALL]))
    n_max = int(rng.choice([1, 5, 64, 65, 700, 3000]))
    N = rng.integers(0, n_max + 1, size=B).astype(np.int32)
    n_groups = int(rng.integers(1, 4))
    cap = n_max + 2
    Hkv = 2
    per_pair = n_q if mode != O.LOGIT_SUM2 else min(2, n_q)
    max_heads = max(1, (16 if mode == O.PROB_SUM else 64) // per_pair)
    heads = [int(rng.integers(1, min(3, max_heads) + 1)) for _ in range(n_groups)]
    say(f"[sweep score seed {seed}] B={B} d={d} n_q={n_q} mode={mode} n_max={n_max} N={N.tolist()} heads={heads}")
    gen = torch.Generator().manual_seed(2000 + seed)
    Ks = [bf16_randn((B, cap, Hkv, d), gen) for _ in range(n_groups)]
    q = bf16_randn((B, sum(heads), n_q, d), gen)
    scale = 1.0 / math.sqrt(d)
    kv_heads = [int(rng.integers(0, Hkv)) for _ in range(n_groups)]
    acc = np.zeros((B, n_max))
    h0 = 0
    for K, kh, nh in zip(Ks, kv_heads, heads):
        O.score_stream(u16(K[:, :, kh]), u16(q[:, h0:h0 + nh]), N, n_max, scale, mode, acc)
        h0 += nh
    Kd = [K.cuda() for K in Ks]
    groups = [(D.kv_view(K), kh, nh) for K, kh, nh in zip(Kd, kv_heads, heads)]
    score = torch.full((B, n_max), float("nan"), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dustin_srh_score_workspace_size(B, n_max, sum(heads), n_q, mode))
    D.dustin_srh_score(torch.from_numpy(N).cuda(), groups, q.cuda(), scale, mode, score, ws)
    torch.cuda.synchronize()
    g = score.cpu().numpy().astype(np.float64)
    if mode == O.PROB_SUM:
        ref = np.abs(acc)
    else:
        # logit sums: the tolerance scales with the sum of |logits| of the summed terms
        ref = np.zeros((B, n_max))
        js = list(range(n_q)) if mode == O.LOGIT_SUM_ALL else sorted({0, n_q - 1})
        h0 = 0
        for K, kh, nh in zip(Ks, kv_heads, heads):
            Kr = K[:, :n_max, kh].double()                                  # [B][n_max][d]
            Qs = q[:, h0:h0 + nh][:, :, js].double().reshape(B, -1, d)      # [B][pairs][d]
            ref += (Kr @ Qs.transpose(1, 2)).abs().sum(2).numpy() * scale
            h0 += nh
    tol = SCORE_RTOL * ref + SCORE_ATOL
    err = np.abs(g - acc)
    assert np.all(np.isfinite(g)), seed
    assert np.all(err <= tol), (seed, float(np.max(err / tol)))
