"""Seeded synthetic workloads for the sparse-verification path.

This module only builds inputs: shapes, seeded random tensors, planted needle keys,
key-norm salience and paged layouts.  It holds none of the method's arithmetic (no
scoring, no selection, no attention) and imports neither the HIP binding nor the
oracle, so both sides of every parity test can be fed from it.

The five workloads follow the shapes of the Dustin summary's evaluation setting
(Qwen2.5 7B/72B targets with a 0.5B-class draft, 32k contexts, large batches; the
"Experimental Results" section of the English Dustin summary) and the Vegas summary's
aggregated-logit selection mode ("A. Aggregierte Attention-Logit-Selektion",
"B. Collect-2-Query").  The public benchmarks those pages measure on (PG-19,
LongBench) are not available; these seeded tensors stand in for them.

Layouts (all bf16 unless noted):
  contiguous cache  [B][n_cap][Hkv][d], n_cap = n_max + gamma + 1; the gamma+1 new
                    verify tokens of sequence b sit at rows ctx_len[b] .. ctx_len[b]+gamma
  paged cache       [num_pages][page_size][Hkv][d] + page_table int32 [B][max_pages]
  verify queries    [B][gamma+1][Hq][d]
  SRH queries       [B][n_qheads][n_q][d_s] per signal (draft: n_q = gamma lookahead
                    queries; target-historical: n_q = gamma+1 queries of the previous pass)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch


@dataclass(frozen=True)
class ModelShape:
    layers: int
    hq: int
    hkv: int
    d: int

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_ctx: int                      # context length (upper end of the range when ragged)
    target: ModelShape
    draft: ModelShape
    gamma: int
    budget: int                     # fixed budget, or 0 when budget_frac is used
    n_sink: int
    n_window: int                   # fixed window, or -1 when window_frac is used
    m: int                          # fixed draft-tier size, or -1 when m_frac is used
    srh_draft: Tuple[Tuple[int, int], ...]   # (draft layer, draft q-head)
    srh_target: Tuple[Tuple[int, int], ...]  # (target layer, target q-head)
    seed: int
    value_scale: float = 1.0        # Q/K/V ~ N(0, value_scale^2)
    needle_count: int = 0
    needle_mode: str = "none"       # "set3" | "cosine" | "none"
    needle_cos: float = 0.0
    needle_from_protected: bool = False   # draw needles from [s, N-w) when True
    needle_frac: float = 0.0        # fraction of tokens (used when needle_count == 0)
    salience_alpha: float = 0.0     # Pareto key-norm salience (0 = off)
    salience_cap: float = 16.0
    ragged_lo: int = 0              # >0: N_b ~ U{ragged_lo .. n_ctx}
    page_size: int = 0              # >0: paged caches with a random page table
    budget_frac_den: int = 0        # >0: budget_b = floor(N_b / den)
    window_frac_den: int = 0        # >0: w_b = floor(budget_b / den)
    m_frac: float = 0.0             # >0: m_b = floor(m_frac * budget_b)

    @property
    def n_verify(self) -> int:
        return self.gamma + 1


TINY = Workload(
    name="tiny_b1_n512",
    batch=1, n_ctx=512,
    target=ModelShape(layers=1, hq=4, hkv=2, d=64),
    draft=ModelShape(layers=1, hq=2, hkv=2, d=64),
    gamma=4, budget=128, n_sink=4, n_window=32, m=32,
    srh_draft=((0, 0), (0, 1)), srh_target=((0, 0), (0, 2)),
    seed=1, value_scale=1.0 / 8.0,
    needle_count=8, needle_mode="set3", needle_from_protected=True,
)

QWEN7B = Workload(
    name="qwen7b_b4_n4096",
    batch=4, n_ctx=4096,
    target=ModelShape(layers=28, hq=28, hkv=4, d=128),
    draft=ModelShape(layers=24, hq=14, hkv=2, d=64),
    gamma=4, budget=512, n_sink=16, n_window=64, m=160,
    srh_draft=((2, 0), (5, 0)), srh_target=((20, 0), (24, 0)),
    seed=2,
    needle_count=32, needle_mode="cosine", needle_cos=0.6, needle_from_protected=True,
)

QWEN72B = Workload(
    name="qwen72b_b8_n32768",
    batch=8, n_ctx=32768,
    target=ModelShape(layers=80, hq=64, hkv=8, d=128),
    draft=ModelShape(layers=24, hq=14, hkv=2, d=64),
    gamma=4, budget=2048, n_sink=16, n_window=256, m=768,
    srh_draft=((2, 0), (2, 7), (5, 0), (5, 7)),
    srh_target=((60, 0), (60, 8), (72, 0), (72, 8)),
    seed=3,
    needle_mode="cosine", needle_cos=0.5, needle_frac=0.01,
)


def sweep_point(budget: int, gamma: int, m_ratio: float) -> Workload:
    """One point of the single-layer large-batch sweep (B=64, 32k, 72B-shaped layer)."""
    return Workload(
        name=f"sweep_b64_n32768_k{budget}_g{gamma}_m{m_ratio:g}",
        batch=64, n_ctx=32768,
        target=ModelShape(layers=1, hq=64, hkv=8, d=128),
        draft=ModelShape(layers=24, hq=14, hkv=2, d=64),
        gamma=gamma, budget=budget, n_sink=16, n_window=budget // 8,
        m=int(m_ratio * budget),
        srh_draft=((2, 0), (2, 7), (5, 0), (5, 7)),
        srh_target=((0, 0), (0, 8), (0, 16), (0, 24)),
        seed=4,
        salience_alpha=1.2, salience_cap=16.0,
    )


SWEEP = tuple(sweep_point(k, g, r) for k in (1024, 2048, 4096) for g in (2, 4, 8) for r in (0.25, 0.5))

RAGGED_PAGED = Workload(
    name="ragged_paged_b16_n8k_64k",
    batch=16, n_ctx=65536,
    target=ModelShape(layers=80, hq=64, hkv=8, d=128),
    draft=ModelShape(layers=24, hq=14, hkv=2, d=64),
    gamma=4, budget=0, n_sink=16, n_window=-1, m=-1,
    srh_draft=((2, 0), (2, 7), (5, 0), (5, 7)),
    srh_target=((60, 0), (60, 8), (72, 0), (72, 8)),
    seed=5,
    ragged_lo=8192, page_size=16,
    budget_frac_den=16, window_frac_den=8, m_frac=0.375,
)

WORKLOADS = {w.name: w for w in (TINY, QWEN7B, QWEN72B, RAGGED_PAGED) + SWEEP}


def shrink(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


# ----------------------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------------------

@dataclass
class SrhGroup:
    """One scored K stream: a model layer's K cache, one KV head, the q-heads it serves."""
    layer: int
    kv_head: int
    qheads: List[int]


@dataclass
class Inputs:
    w: Workload
    device: torch.device
    ctx_len: torch.Tensor                 # int32 [B]
    n_max: int                            # max_b ctx_len
    n_cap: int                            # tokens addressable per sequence
    budget: torch.Tensor                  # int32 [B]
    n_sink: torch.Tensor                  # int32 [B]
    n_window: torch.Tensor                # int32 [B]
    m: torch.Tensor                       # int32 [B]
    k_max: int
    # target caches: layer -> tensor.  contiguous: [B][n_cap][Hkv][d]; paged: [P][ps][Hkv][d]
    k_cache: dict = field(default_factory=dict)
    v_cache: dict = field(default_factory=dict)
    q_verify: dict = field(default_factory=dict)      # layer -> [B][V][Hq][d]
    draft_k: dict = field(default_factory=dict)       # draft layer -> draft K cache
    page_table: Optional[torch.Tensor] = None         # int32 [B][max_pages]
    num_pages: int = 0
    draft_groups: List[SrhGroup] = field(default_factory=list)
    target_groups: List[SrhGroup] = field(default_factory=list)
    q_srh_draft: Optional[torch.Tensor] = None        # [B][n_qheads][gamma][d_draft]
    q_srh_target: Optional[torch.Tensor] = None       # [B][n_qheads][gamma+1][d]
    needles: Optional[torch.Tensor] = None            # int64 [B][n_needles] (or None)

    @property
    def paged(self) -> bool:
        return self.page_table is not None


def _groups(srh: Sequence[Tuple[int, int]], shape: ModelShape) -> List[SrhGroup]:
    out: List[SrhGroup] = []
    for layer, qh in srh:
        kv = qh // shape.group
        for g in out:
            if g.layer == layer and g.kv_head == kv:
                g.qheads.append(qh)
                break
        else:
            out.append(SrhGroup(layer=layer, kv_head=kv, qheads=[qh]))
    return out


def _randn(shape, gen, device, scale=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(torch.bfloat16)


def _planted(k: torch.Tensor, u: torch.Tensor, mode: str, cos: float) -> torch.Tensor:
    """New bf16 values for key rows `k` ([n][d]) so that they point along unit vector `u`:
    "set3" makes every row 3*u; "cosine" keeps each row's norm and sets its cosine to u."""
    k = k.float()
    if mode == "set3":
        new = (3.0 * u).expand_as(k)
    else:
        norm = k.norm(dim=-1, keepdim=True).clamp_min(1e-6)
        perp = k - (k @ u)[:, None] * u[None, :]
        perp = perp / perp.norm(dim=-1, keepdim=True).clamp_min(1e-6)
        new = norm * (cos * u[None, :] + math.sqrt(max(0.0, 1.0 - cos * cos)) * perp)
    return new.to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu", target_layers: Optional[Sequence[int]] = None,
                seed: Optional[int] = None) -> Inputs:
    """Build the seeded inputs of workload `w` on `device`.

    target_layers: which target layers get K/V caches and verify queries (default: all).
    The target SRH layers are always materialised.  Generation order is fixed so a
    (workload, seed, target_layers) triple always gives the same bits on a given device.
    """
    device = torch.device(device)
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(seed + 7919)
    B, V = w.batch, w.n_verify
    T, D = w.target, w.draft

    # ---- context lengths and per-sequence selection parameters (host RNG) ----
    if w.ragged_lo > 0:
        n = torch.randint(w.ragged_lo, w.n_ctx + 1, (B,), generator=cpu_gen)
    else:
        n = torch.full((B,), w.n_ctx, dtype=torch.int64)
    if w.budget_frac_den > 0:
        budget = n // w.budget_frac_den
    else:
        budget = torch.full((B,), w.budget, dtype=torch.int64)
    window = budget // w.window_frac_den if w.window_frac_den > 0 else torch.full((B,), w.n_window)
    m = (budget.double() * w.m_frac).floor().long() if w.m_frac > 0 else torch.full((B,), w.m)
    sink = torch.full((B,), w.n_sink, dtype=torch.int64)
    n_max = int(n.max())
    n_cap = n_max + V
    k_max = int(budget.max())

    inp = Inputs(w=w, device=device,
                 ctx_len=n.to(torch.int32).to(device), n_max=n_max, n_cap=n_cap,
                 budget=budget.to(torch.int32).to(device), n_sink=sink.to(torch.int32).to(device),
                 n_window=window.to(torch.int32).to(device), m=m.to(torch.int32).to(device),
                 k_max=k_max)
    inp.draft_groups = _groups(w.srh_draft, D)
    inp.target_groups = _groups(w.srh_target, T)

    # ---- page table: a random permutation of physical pages ----
    if w.page_size > 0:
        ps = w.page_size
        pages = [(int(n[b]) + V + ps - 1) // ps for b in range(B)]
        max_pages = (n_cap + ps - 1) // ps
        total = sum(pages)
        perm = torch.randperm(total, generator=cpu_gen).to(torch.int32)
        pt = torch.zeros((B, max_pages), dtype=torch.int32)
        o = 0
        for b in range(B):
            pt[b, :pages[b]] = perm[o:o + pages[b]]
            o += pages[b]
        inp.page_table = pt.to(device)
        inp.num_pages = total

    def cache(shape: ModelShape, with_new: bool):
        if inp.paged:
            return _randn((inp.num_pages, w.page_size, shape.hkv, shape.d), gen, device, w.value_scale)
        rows = n_cap if with_new else n_max
        return _randn((B, rows, shape.hkv, shape.d), gen, device, w.value_scale)

    # ---- SRH queries ----
    nd = sum(len(g.qheads) for g in inp.draft_groups)
    nt = sum(len(g.qheads) for g in inp.target_groups)
    inp.q_srh_draft = _randn((B, nd, w.gamma, D.d), gen, device, w.value_scale)
    inp.q_srh_target = _randn((B, nt, V, T.d), gen, device, w.value_scale)

    # ---- caches ----
    layers = list(range(T.layers)) if target_layers is None else sorted(set(target_layers))
    layers = sorted(set(layers) | {g.layer for g in inp.target_groups})
    for l in layers:
        inp.k_cache[l] = cache(T, True)
        inp.v_cache[l] = cache(T, True)
        inp.q_verify[l] = _randn((B, V, T.hq, T.d), gen, device, w.value_scale)
    for l in sorted({g.layer for g in inp.draft_groups}):
        inp.draft_k[l] = cache(D, True)

    # ---- key-norm salience (Pareto, truncated) on every key row of token i ----
    if (w.salience_alpha > 0 or w.needle_mode != "none") and inp.paged:
        raise NotImplementedError("salience and needles are generated for contiguous caches only")
    if w.salience_alpha > 0:
        u = torch.rand((B, n_cap), generator=gen, device=device).clamp_min(1e-12)
        f = u.pow(-1.0 / w.salience_alpha).clamp_max(w.salience_cap)
        for kc in list(inp.k_cache.values()) + list(inp.draft_k.values()):
            rows = kc.shape[1]
            for b in range(B):             # per sequence: no full-size fp32 temporary
                kc[b].copy_((kc[b].float() * f[b, :rows, None, None]).to(torch.bfloat16))

    # ---- planted needles in the SRH streams ----
    if w.needle_mode != "none":
        needles = []
        for b in range(B):
            nb = int(n[b])
            lo, hi = (w.n_sink, nb - int(window[b])) if w.needle_from_protected else (0, nb)
            c = w.needle_count if w.needle_count > 0 else int(math.floor(w.needle_frac * nb))
            pos = lo + torch.randperm(hi - lo, generator=cpu_gen)[:c]
            needles.append(pos.sort().values)
        inp.needles = torch.stack(needles)
        for groups, qs, caches in ((inp.draft_groups, inp.q_srh_draft, inp.draft_k),
                                   (inp.target_groups, inp.q_srh_target, inp.k_cache)):
            qoff = 0
            for g in groups:
                nq = len(g.qheads)
                for b in range(B):
                    u = qs[b, qoff:qoff + nq].float().reshape(-1, qs.shape[-1]).mean(0)
                    u = u / u.norm().clamp_min(1e-12)
                    rows = needles[b].to(device)
                    view = caches[g.layer][b, :, g.kv_head]        # [rows][d] view
                    view[rows] = _planted(view[rows], u, w.needle_mode, w.needle_cos)
                qoff += nq
    return inp


# ----------------------------------------------------------------------------------------
# helpers for tests and the bench: logical (unpaged) views of a cache
# ----------------------------------------------------------------------------------------

def logical_rows(inp: Inputs, cache: torch.Tensor, b: int, n_rows: int) -> torch.Tensor:
    """[n_rows][Hkv][d] rows 0..n_rows-1 of sequence b, gathered through the page table
    when the cache is paged (plain indexing; used to hand host copies to the oracle)."""
    if not inp.paged:
        return cache[b, :n_rows]
    ps = inp.w.page_size
    rows = torch.arange(n_rows, device=cache.device)
    pg = inp.page_table[b].long()[rows // ps]
    return cache[pg, rows % ps]
