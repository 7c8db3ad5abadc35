"""Test infrastructure: hands the exact device bits to the oracle and compares.

The oracle's inputs are host copies of the same bf16 tensors the HIP path reads
(paged caches are gathered into logical order with plain indexing); the oracle never
sees anything the HIP path computed except where a test says so (selection is run on
the GPU's own fp32 scores so both sides take the integer decision on the same values).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import oracle as O
from sparse_kv_attention_amd.workloads import Inputs, logical_rows

SCORE_RTOL, SCORE_ATOL = 1e-5, 1e-10
ATTN_ATOL, LSE_ATOL = 2e-2, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def rows(inp: Inputs, cache: torch.Tensor, b: int, n_rows: int) -> torch.Tensor:
    return logical_rows(inp, cache, b, n_rows)


def signal_spec(inp: Inputs, signal: str):
    w = inp.w
    if signal == "draft":
        return inp.draft_groups, inp.q_srh_draft, inp.draft_k, 1.0 / math.sqrt(w.draft.d)
    return inp.target_groups, inp.q_srh_target, inp.k_cache, 1.0 / math.sqrt(w.target.d)


def oracle_scores(inp: Inputs, signal: str, mode: int, bsel, scale=None):
    groups, q, caches, default_scale = signal_spec(inp, signal)
    scale = default_scale if scale is None else scale
    ctx = inp.ctx_len.cpu().numpy()[bsel]
    acc = np.zeros((len(bsel), inp.n_max), dtype=np.float64)
    qoff = 0
    for g in groups:
        nq = len(g.qheads)
        K = np.stack([u16(rows(inp, caches[g.layer], b, inp.n_max)[:, g.kv_head]) for b in bsel])
        Q = u16(q[bsel, qoff:qoff + nq])
        O.score_stream(K, Q, ctx, inp.n_max, scale, mode, acc)
        qoff += nq
    return acc


def logit_abs_sum(inp: Inputs, signal: str, bsel, all_queries=False):
    """sum over (head, query in {0, last} or every query) of |logit|: the conditioning of
    a logit sum."""
    groups, q, caches, scale = signal_spec(inp, signal)
    out = np.zeros((len(bsel), inp.n_max))
    qoff = 0
    for g in groups:
        nq = len(g.qheads)
        for i, b in enumerate(bsel):
            K = rows(inp, caches[g.layer], b, inp.n_max)[:, g.kv_head].double().cpu()
            js = list(range(q.shape[2])) if all_queries else [0, q.shape[2] - 1]
            Qs = q[b, qoff:qoff + nq][:, js].double().cpu().reshape(-1, q.shape[-1])
            out[i] += (K @ Qs.T).abs().sum(1).numpy() * scale
        qoff += nq
    return out


def check_scores(gpu: np.ndarray, ora: np.ndarray, what: str, cond=None):
    ref = np.abs(ora) if cond is None else cond
    err = np.abs(gpu.astype(np.float64) - ora)
    tol = SCORE_RTOL * ref + SCORE_ATOL
    bad = err > tol
    worst = float(np.max(err / tol))
    say(f"  {what}: max err/tol = {worst:.3g}")
    assert not bad.any(), f"{what}: {int(bad.sum())} scores outside 1e-5 rel (worst err/tol {worst:.3g})"


def oracle_select_on(inp: Inputs, sd: np.ndarray, st: np.ndarray, bsel, pure_topk=False):
    c = lambda t: t.cpu().numpy()[bsel]
    B = len(bsel)
    zeros = np.zeros(B, np.int32)
    if pure_topk:
        return O.select(c(inp.ctx_len), None, st, c(inp.budget), zeros, zeros, zeros, inp.k_max)
    return O.select(c(inp.ctx_len), sd, st, c(inp.budget), c(inp.n_sink), c(inp.n_window), c(inp.m), inp.k_max)


def oracle_attn(inp: Inputs, layer: int, idx, count, bsel, dense=False, scale=None):
    """Returns (O float64 [len(bsel)][nv][Hq][d], lse [len(bsel)][Hq][nv])."""
    ctx = inp.ctx_len.cpu().numpy()
    n_rows = int(max(ctx[b] for b in bsel)) + inp.w.n_verify
    K = np.stack([u16(rows(inp, inp.k_cache[layer], b, n_rows)) for b in bsel])
    V = np.stack([u16(rows(inp, inp.v_cache[layer], b, n_rows)) for b in bsel])
    Q = u16(inp.q_verify[layer][bsel])
    scale = 1.0 / math.sqrt(inp.w.target.d) if scale is None else scale
    if dense:
        return O.verify_attn(Q, K, V, ctx[bsel], None, None, scale, inp.w.target.hkv)
    return O.verify_attn(Q, K, V, ctx[bsel], idx[bsel], count[bsel], scale, inp.w.target.hkv)


def check_attn(out: torch.Tensor, lse: torch.Tensor, ref, bsel, what: str):
    o = out[bsel].float().cpu().numpy()
    l = lse[bsel].cpu().numpy()
    eo = float(np.max(np.abs(o - ref[0])))
    el = float(np.max(np.abs(l - ref[1])))
    say(f"  {what}: max|dO| = {eo:.3g}  max|dLSE| = {el:.3g}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    assert eo <= ATTN_ATOL, f"{what}: O max-abs {eo}"
    assert el <= LSE_ATOL, f"{what}: LSE max-abs {el}"
