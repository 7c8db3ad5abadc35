"""One sparse-verification step on device-resident inputs, driven through the C ABI.

Holds the views, workspaces and output buffers of a workload and issues the library
calls in the order of the verification workflow (English Dustin summary, "Methodology"
3, steps 2-4): score the draft SRHs, score the target SRHs, select I_verify, then
verify attention layer by layer; step 5 (the verified block in the cache) and the
attention-recovery measurement are separate methods.  Argument marshalling only; all
arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import torch

from . import dustin as D
from .workloads import Inputs


class SparseVerifyStep:
    def __init__(self, inp: Inputs, layers: Optional[Sequence[int]] = None, logit_sum2: bool = False,
                 logit_sum_all: bool = False):
        """logit_sum2 / logit_sum_all: the Vegas-style target signal (German Vegas summary
        2A/2B: raw logits summed over the first and bonus queries, or over every query)
        with pure top-k selection and no draft signal."""
        self.inp = inp
        w = inp.w
        dev = inp.ctx_len.device
        pt = inp.page_table
        self.B, self.n_max, self.k_max = w.batch, inp.n_max, inp.k_max
        self.T, self.Dm = w.target, w.draft
        self.layers = sorted(inp.k_cache) if layers is None else list(layers)
        logit_sum2 = logit_sum2 or logit_sum_all
        self.logit_sum2 = logit_sum2
        # a draft signal exists only if the draft speculated at least one token
        self.has_draft = w.gamma > 0 and not logit_sum2
        self.draft_groups = [(D.kv_view(inp.draft_k[g.layer], pt), g.kv_head, len(g.qheads))
                             for g in inp.draft_groups]
        self.target_groups = [(D.kv_view(inp.k_cache[g.layer], pt), g.kv_head, len(g.qheads))
                              for g in inp.target_groups]
        self.kv: Dict[int, tuple] = {l: (D.kv_view(inp.k_cache[l], pt), D.kv_view(inp.v_cache[l], pt))
                                     for l in inp.k_cache}
        B, n_max = self.B, self.n_max
        self.score_draft = torch.zeros((B, n_max), dtype=torch.float32, device=dev)
        self.score_target = torch.zeros((B, n_max), dtype=torch.float32, device=dev)
        nd = inp.q_srh_draft.shape[1]
        nt = inp.q_srh_target.shape[1]
        mode_t = (D.SCORE_LOGIT_SUM_ALL if logit_sum_all else
                  D.SCORE_LOGIT_SUM2 if logit_sum2 else D.SCORE_PROB_SUM)
        self.mode_t = mode_t
        self.scale_draft = 1.0 / math.sqrt(self.Dm.d)
        self.scale = 1.0 / math.sqrt(self.T.d)
        # both signals in one library call (one logit launch, one finalize)
        ws_score = D.dustin_srh_score_signals_workspace_size(B, n_max, self.signals())
        ws_score = max(ws_score, D.dustin_srh_score_workspace_size(B, n_max, nt, w.n_verify, mode_t))
        if self.has_draft:
            ws_score = max(ws_score, D.dustin_srh_score_workspace_size(B, n_max, nd, w.gamma, D.SCORE_PROB_SUM))
        self.ws_score = D.workspace(ws_score, dev)
        self.ws_select = D.workspace(D.dustin_select_workspace_size(B, n_max), dev)
        H = (B, self.T.hq, self.T.hkv, self.T.d, w.n_verify)
        ws_attn = max(D.dustin_sparse_verify_attn_workspace_size(*H, self.k_max),
                      D.dense_verify_attn_workspace_size(*H, n_max))
        self.ws_attn = D.workspace(ws_attn, dev)
        self.idx = torch.full((B, max(self.k_max, 1)), -1, dtype=torch.int32, device=dev)
        self.count = torch.zeros((B,), dtype=torch.int32, device=dev)
        if logit_sum2:
            zeros = torch.zeros((B,), dtype=torch.int32, device=dev)
            self.sel_params = (zeros, zeros, zeros)
        else:
            self.sel_params = (inp.n_sink, inp.n_window, inp.m)
        self.out = torch.empty((B, w.n_verify, self.T.hq, self.T.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, self.T.hq, w.n_verify), dtype=torch.float32, device=dev)

    # ---- the stages ----
    def signals(self):
        """(groups, q, scale, mode, score) of the draft signal (when there is one) and the
        target signal, with the current scales."""
        inp = self.inp
        sig = []
        if self.has_draft:
            sig.append((self.draft_groups, inp.q_srh_draft, self.scale_draft, D.SCORE_PROB_SUM, self.score_draft))
        sig.append((self.target_groups, inp.q_srh_target, self.scale, self.mode_t, self.score_target))
        return sig

    def score(self, stream=None):
        """Both signals in one call."""
        D.dustin_srh_score_signals(self.inp.ctx_len, self.signals(), self.ws_score, stream)

    def score_separately(self, stream=None):
        """The same scores from one call per signal."""
        inp = self.inp
        if self.has_draft:
            D.dustin_srh_score(inp.ctx_len, self.draft_groups, inp.q_srh_draft, self.scale_draft,
                               D.SCORE_PROB_SUM, self.score_draft, self.ws_score, stream)
        D.dustin_srh_score(inp.ctx_len, self.target_groups, inp.q_srh_target, self.scale,
                           self.mode_t, self.score_target, self.ws_score, stream)

    def select(self, stream=None):
        inp = self.inp
        sink, window, m = self.sel_params
        D.dustin_select(inp.ctx_len, self.score_draft if self.has_draft else None, self.score_target,
                        inp.budget, sink, window, m, self.idx, self.count, self.ws_select, stream)

    def attn(self, layer: int, out=None, lse=None, stream=None):
        k, v = self.kv[layer]
        D.dustin_sparse_verify_attn(self.inp.q_verify[layer], k, v, self.T.hkv, self.inp.ctx_len, self.idx,
                                    self.count, self.scale, self.out if out is None else out,
                                    self.lse if lse is None else lse, self.ws_attn, stream)

    def attn_logits(self, layer: int, logit_sum2, out=None, lse=None, stream=None):
        """attn() that also writes the Collect-2 logit sums of the selected tokens
        (fp32 [B][Hkv][k_max]) as a by-product of verification."""
        k, v = self.kv[layer]
        D.dustin_sparse_verify_attn_logits(self.inp.q_verify[layer], k, v, self.T.hkv, self.inp.ctx_len, self.idx,
                                           self.count, self.scale, self.out if out is None else out,
                                           self.lse if lse is None else lse, logit_sum2, self.ws_attn, stream)

    def dense(self, layer: int, out=None, lse=None, stream=None):
        k, v = self.kv[layer]
        D.dense_verify_attn(self.inp.q_verify[layer], k, v, self.T.hkv, self.inp.ctx_len, self.n_max,
                            self.scale, self.out if out is None else out, self.lse if lse is None else lse,
                            self.ws_attn, stream)

    def vegas_all_heads(self, layer: int, score, ws=None, all_queries: bool = False, stream=None):
        """The Vegas aggregate as the German Vegas summary writes it (2A: logits summed over
        every query head; 2B: the first and the bonus query only, unless all_queries): one
        logit-sum scoring call over every KV head of a target layer with all of its query
        heads, from the layer's verify queries.  Writes score [B][n_max]; returns the
        workspace it used (pass it back to reuse it)."""
        inp = self.inp
        q = inp.q_verify[layer].permute(0, 2, 1, 3).contiguous()      # [B][Hq][n_verify][d]
        k, _ = self.kv[layer]
        groups = [(k, g, self.T.group) for g in range(self.T.hkv)]
        mode = D.SCORE_LOGIT_SUM_ALL if all_queries else D.SCORE_LOGIT_SUM2
        if ws is None:
            ws = D.workspace(D.dustin_srh_score_workspace_size(self.B, self.n_max, self.T.hq, inp.w.n_verify, mode),
                             score.device)
        D.dustin_srh_score(inp.ctx_len, groups, q, self.scale, mode, score, ws, stream)
        return ws

    def recovery(self, layer: int, rec=None, stream=None):
        """Share of the dense attention mass on the kept set, per (b, h, t) [B][Hq][n_verify]:
        one sparse and one dense call on the layer, then the library's recovery kernel."""
        lse_s = torch.empty_like(self.lse)
        lse_d = torch.empty_like(self.lse)
        rec = torch.empty_like(self.lse) if rec is None else rec
        self.attn(layer, out=torch.empty_like(self.out), lse=lse_s, stream=stream)
        self.dense(layer, out=torch.empty_like(self.out), lse=lse_d, stream=stream)
        D.dustin_attn_recovery(lse_s, lse_d, rec, stream)
        return rec

    def write_block(self, layer: int, k_new, v_new, ctx_len=None, stream=None):
        """Store a block [B][n_new][Hkv][d] behind the committed context of a layer's caches."""
        k, v = self.kv[layer]
        D.dustin_kv_write_block(k_new, v_new, self.inp.ctx_len if ctx_len is None else ctx_len, k, v, stream)

    def commit(self, n_accept, ctx_len=None, stream=None):
        """Advance the context lengths (in place) over the kept rows of the verified block."""
        D.dustin_kv_commit(n_accept, self.inp.ctx_len if ctx_len is None else ctx_len, self.inp.w.n_verify, stream)

    def step(self, stream=None):
        """One whole sparse-verification step: both signals, selection, every layer."""
        self.score(stream)
        self.select(stream)
        for l in self.layers:
            self.attn(l, stream=stream)


class AllHeadsEstimator:
    """The naive importance estimator that SRHs replace: the softmax attention scores of
    every query head of a layer (English Dustin summary, "Problem Statement": naive
    estimators materialise attention scores across all heads and layers; "Methodology" 2:
    SRHs cut the estimation to a small share of that full calculation).

    For one layer's K cache and queries q [B][Hq][n_q][d] (every head), each KV head's
    query heads are cut into groups of at most 16 (head, query) pairs, the groups into
    library calls of at most 16 groups; call c writes its own score vector scores[c]
    (the estimator's map is their sum).  Argument marshalling only."""

    MAX_PAIRS, MAX_GROUPS = 16, 16

    def __init__(self, k_cache, page_table, q, Hkv: int, ctx_len, scale: float):
        B, Hq, n_q, d = q.shape
        self.q, self.ctx_len, self.scale = q, ctx_len, scale
        G = Hq // Hkv
        per = max(1, self.MAX_PAIRS // n_q)            # query heads per group
        view = D.kv_view(k_cache, page_table)
        groups = []                                     # (view, kv_head, first head, n heads)
        for g in range(Hkv):
            for h0 in range(g * G, (g + 1) * G, per):
                groups.append((view, g, h0, min(per, (g + 1) * G - h0)))
        self.calls = []                                 # (groups, q slice)
        for c0 in range(0, len(groups), self.MAX_GROUPS):
            cg = groups[c0:c0 + self.MAX_GROUPS]
            h_lo, h_hi = cg[0][2], cg[-1][2] + cg[-1][3]
            self.calls.append(([(v, g, nh) for v, g, _, nh in cg], q[:, h_lo:h_hi].contiguous()))
        n_max = int(ctx_len.max())
        self.n_max = n_max
        dev = q.device
        self.scores = [torch.zeros((B, n_max), dtype=torch.float32, device=dev) for _ in self.calls]
        ws = max(D.dustin_srh_score_workspace_size(B, n_max, cq.shape[1], n_q, D.SCORE_PROB_SUM)
                 for _, cq in self.calls)
        self.ws = D.workspace(ws, dev)

    def score(self, stream=None):
        for (groups, cq), out in zip(self.calls, self.scores):
            D.dustin_srh_score(self.ctx_len, groups, cq, self.scale, D.SCORE_PROB_SUM, out, self.ws, stream)
