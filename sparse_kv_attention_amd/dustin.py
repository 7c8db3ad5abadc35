"""Python binding of libdustin.so (include/dustin.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module converts torch
tensors to pointers, strides and sizes, passes torch's current HIP stream, and turns
non-zero status codes into exceptions.  It never computes a result itself and has no
fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdustin.so")

OK, ERR_INVALID_ARG, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5
SCORE_PROB_SUM, SCORE_LOGIT_SUM2, SCORE_LOGIT_SUM_ALL = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python sparse_kv_attention_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class KvView(ctypes.Structure):
    _fields_ = [
        ("base", _P),
        ("stride_batch", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("n_tokens", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("page_table", _P),
        ("stride_page", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]


class SrhGroup(ctypes.Structure):
    _fields_ = [("k", KvView), ("kv_head", ctypes.c_int32), ("n_qheads", ctypes.c_int32)]


class SrhSignal(ctypes.Structure):
    _fields_ = [("n_groups", ctypes.c_int32), ("groups", ctypes.POINTER(SrhGroup)), ("head_dim", ctypes.c_int32),
                ("q", _P), ("n_q", ctypes.c_int32), ("scale", ctypes.c_float), ("mode", ctypes.c_int32),
                ("score", _P)]


def _decl(name, args):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = _I
    return f


_lib.dustin_status_string.argtypes = [_I]
_lib.dustin_status_string.restype = ctypes.c_char_p
_score_ws = _decl("dustin_srh_score_workspace_size", [_I, _I, _I, _I, _I, ctypes.POINTER(_SZ)])
_score = _decl("dustin_srh_score", [_I, _I, _P, _I, ctypes.POINTER(SrhGroup), _I, _P, _I, _F, _I,
                                    _P, _P, _SZ, _P])
_signals_ws = _decl("dustin_srh_score_signals_workspace_size", [_I, _I, _I, ctypes.POINTER(SrhSignal),
                                                               ctypes.POINTER(_SZ)])
_signals = _decl("dustin_srh_score_signals", [_I, _I, _P, _I, ctypes.POINTER(SrhSignal), _P, _SZ, _P])
_select_ws = _decl("dustin_select_workspace_size", [_I, _I, ctypes.POINTER(_SZ)])
_select = _decl("dustin_select", [_I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _SZ, _P])
_sparse_ws = _decl("dustin_sparse_verify_attn_workspace_size", [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_SZ)])
_sparse = _decl("dustin_sparse_verify_attn", [_I, _I, _I, _I, _I, _P, ctypes.POINTER(KvView),
                                              ctypes.POINTER(KvView), _P, _P, _P, _I, _F, _P, _P, _P,
                                              _SZ, _P])
_sparse_noalloc = _decl("dustin_sparse_verify_attn_noalloc",
                         [_I, _I, _I, _I, _I, _P, ctypes.POINTER(KvView), ctypes.POINTER(KvView), _P, _P, _P,
                          _I, _F, _P, _P, _P])
_sparse_logits = _decl("dustin_sparse_verify_attn_logits",
                        [_I, _I, _I, _I, _I, _P, ctypes.POINTER(KvView), ctypes.POINTER(KvView), _P, _P, _P, _I,
                         _F, _P, _P, _P, _P, _SZ, _P])
_attn_plan = _decl("dustin_attn_plan", [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_int32)])
_dense_ws = _decl("dense_verify_attn_workspace_size", [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_SZ)])
_dense = _decl("dense_verify_attn", [_I, _I, _I, _I, _I, _P, ctypes.POINTER(KvView),
                                     ctypes.POINTER(KvView), _P, _I, _F, _P, _P, _P, _SZ, _P])
_kv_write = _decl("dustin_kv_write_block", [_I, _I, _I, _I, _P, _P, _P, ctypes.POINTER(KvView),
                                             ctypes.POINTER(KvView), _P])
_kv_commit = _decl("dustin_kv_commit", [_I, _I, _P, _P, _P])
_recovery = _decl("dustin_attn_recovery", [_I, _P, _P, _P, _P])
_floor = _decl("dustin_gather_floor", [_I, _I, _I, ctypes.POINTER(KvView), ctypes.POINTER(KvView), _P, _I, _P,
                                       _I, _P])

EXPORTED = ("dustin_status_string", "dustin_srh_score_workspace_size", "dustin_srh_score",
            "dustin_srh_score_signals_workspace_size", "dustin_srh_score_signals",
            "dustin_select_workspace_size", "dustin_select",
            "dustin_sparse_verify_attn_workspace_size", "dustin_sparse_verify_attn",
            "dustin_sparse_verify_attn_noalloc", "dustin_attn_plan", "dustin_sparse_verify_attn_logits",
            "dense_verify_attn_workspace_size", "dense_verify_attn",
            "dustin_kv_write_block", "dustin_kv_commit", "dustin_attn_recovery", "dustin_gather_floor")


class DustinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.dustin_status_string(status).decode()} ({status})")


def _check(status: int, where: str):
    if status != OK:
        raise DustinError(status, where)


def status_string(status: int) -> str:
    return _lib.dustin_status_string(status).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor")


def kv_view(cache: torch.Tensor, page_table: Optional[torch.Tensor] = None) -> KvView:
    """View of a bf16 cache: contiguous [B][n_tokens][Hkv][d], or paged
    [num_pages][page_size][Hkv][d] with page_table int32 [B][max_pages]."""
    if cache.dtype != torch.bfloat16 or cache.dim() != 4 or cache.stride(3) != 1 or not cache.is_cuda:
        raise ValueError("cache must be a 4-d bf16 device tensor with a contiguous last dim")
    v = KvView()
    v.base = cache.data_ptr()
    v.stride_token = cache.stride(1)
    v.stride_head = cache.stride(2)
    v.n_heads = cache.shape[2]
    if page_table is None:
        v.stride_batch = cache.stride(0)
        v.n_tokens = cache.shape[1]
        v.page_table = None
    else:
        _dev_i32(page_table, "page_table")
        v.stride_batch = 0
        v.n_tokens = 0
        v.page_table = page_table.data_ptr()
        v.stride_page = cache.stride(0)
        v.page_size = cache.shape[1]
        v.max_pages = page_table.shape[1]
        v.num_pages = cache.shape[0]
    return v


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A zero-filled device workspace of at least `nbytes` (16-byte aligned by torch)."""
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device or "cuda")


# ------------------------------------------------------------------------------ scoring

def dustin_srh_score_workspace_size(B: int, n_max: int, total_qheads: int, n_q: int, mode: int) -> int:
    n = _SZ(0)
    _check(_score_ws(B, n_max, total_qheads, n_q, mode, ctypes.byref(n)), "dustin_srh_score_workspace_size")
    return n.value


def dustin_srh_score(ctx_len: torch.Tensor, groups: Sequence[Tuple[KvView, int, int]], q: torch.Tensor,
                     scale: float, mode: int, score: torch.Tensor, ws: torch.Tensor, stream=None):
    """groups: (kv_view, kv_head, n_qheads) per scored stream; q bf16 [B][sum n_qheads][n_q][d];
    score fp32 [B][n_max] (written)."""
    _dev_i32(ctx_len, "ctx_len")
    B, _, n_q, d = q.shape
    n_max = score.shape[1]
    arr = (SrhGroup * len(groups))()
    for i, (view, kv_head, nqh) in enumerate(groups):
        arr[i].k = view
        arr[i].kv_head = kv_head
        arr[i].n_qheads = nqh
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or score.dtype != torch.float32 or not score.is_contiguous():
        raise ValueError("q must be contiguous bf16, score contiguous fp32")
    _check(_score(B, n_max, _ptr(ctx_len), len(groups), arr, d, _ptr(q), n_q, float(scale), mode,
                  _ptr(score), _ptr(ws), ws.numel(), _stream(stream)), "dustin_srh_score")


def _signal_array(signals, B):
    """signals: (groups, q, scale, mode, score) per signal -> (SrhSignal array, keep-alive)."""
    arr = (SrhSignal * len(signals))()
    keep = []
    for i, (groups, q, scale, mode, score) in enumerate(signals):
        g = (SrhGroup * len(groups))()
        for j, (view, kv_head, nqh) in enumerate(groups):
            g[j].k = view
            g[j].kv_head = kv_head
            g[j].n_qheads = nqh
        keep.append(g)
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or score.dtype != torch.float32 \
                or not score.is_contiguous() or q.shape[0] != B:
            raise ValueError("q must be contiguous bf16 [B][heads][n_q][d], score contiguous fp32 [B][n_max]")
        arr[i].n_groups = len(groups)
        arr[i].groups = ctypes.cast(g, ctypes.POINTER(SrhGroup))
        arr[i].head_dim = q.shape[3]
        arr[i].q = q.data_ptr()
        arr[i].n_q = q.shape[2]
        arr[i].scale = float(scale)
        arr[i].mode = int(mode)
        arr[i].score = score.data_ptr()
    return arr, keep


def dustin_srh_score_signals_workspace_size(B: int, n_max: int, signals) -> int:
    """signals: (groups, q, scale, mode, score) per signal, as dustin_srh_score_signals."""
    arr, keep = _signal_array(signals, B)
    n = _SZ(0)
    _check(_signals_ws(B, n_max, len(signals), arr, ctypes.byref(n)), "dustin_srh_score_signals_workspace_size")
    return n.value


def dustin_srh_score_signals(ctx_len: torch.Tensor, signals, ws: torch.Tensor, stream=None):
    """Both scoring signals in one call.  signals: (groups, q, scale, mode, score) per signal,
    groups as in dustin_srh_score; every score [B][n_max] is written."""
    _dev_i32(ctx_len, "ctx_len")
    B = ctx_len.shape[0]
    n_max = signals[0][4].shape[1]
    arr, keep = _signal_array(signals, B)
    _check(_signals(B, n_max, _ptr(ctx_len), len(signals), arr, _ptr(ws), ws.numel(), _stream(stream)),
           "dustin_srh_score_signals")


# ---------------------------------------------------------------------------- selection

def dustin_select_workspace_size(B: int, n_max: int) -> int:
    n = _SZ(0)
    _check(_select_ws(B, n_max, ctypes.byref(n)), "dustin_select_workspace_size")
    return n.value


def dustin_select(ctx_len, score_draft, score_target, budget, n_sink, n_window, m, idx, count,
                  ws: Optional[torch.Tensor] = None, stream=None):
    """Scores fp32 [B][n_max] (score_draft may be None); per-sequence int32 [B] parameters;
    idx int32 [B][k_max] and count int32 [B] are written."""
    for t, n in ((ctx_len, "ctx_len"), (budget, "budget"), (n_sink, "n_sink"), (n_window, "n_window"),
                 (m, "m"), (idx, "idx"), (count, "count")):
        _dev_i32(t, n)
    B, n_max = score_target.shape
    for s in (score_draft, score_target):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous() or s.shape != (B, n_max)):
            raise ValueError("scores must be contiguous fp32 [B][n_max]")
    _check(_select(B, n_max, _ptr(ctx_len), _ptr(score_draft), _ptr(score_target), _ptr(budget),
                   _ptr(n_sink), _ptr(n_window), _ptr(m), idx.shape[1], _ptr(idx), _ptr(count),
                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "dustin_select")


# ---------------------------------------------------------------------------- attention

def dustin_sparse_verify_attn_workspace_size(B, Hq, Hkv, head_dim, n_verify, k_max) -> int:
    n = _SZ(0)
    _check(_sparse_ws(B, Hq, Hkv, head_dim, n_verify, k_max, ctypes.byref(n)),
           "dustin_sparse_verify_attn_workspace_size")
    return n.value


def dense_verify_attn_workspace_size(B, Hq, Hkv, head_dim, n_verify, n_max) -> int:
    n = _SZ(0)
    _check(_dense_ws(B, Hq, Hkv, head_dim, n_verify, n_max, ctypes.byref(n)), "dense_verify_attn_workspace_size")
    return n.value


ATTN_LAYOUT_LIST, ATTN_LAYOUT_TWO_TABLES, ATTN_LAYOUT_DENSE = 0, 1, 2


def dustin_attn_plan(B, Hq, Hkv, head_dim, n_verify, n_positions, layout=ATTN_LAYOUT_LIST) -> dict:
    """The attention launch plan for these sizes: query tiles per workgroup, query groups,
    splits, workgroups and how the splits are combined ("none", "merge kernel", "fused")."""
    p = (ctypes.c_int32 * 5)()
    _check(_attn_plan(B, Hq, Hkv, head_dim, n_verify, n_positions, layout, p), "dustin_attn_plan")
    return {"qt": p[0], "qgroups": p[1], "splits": p[2], "workgroups": p[3],
            "merge": ("none", "merge kernel", "fused")[p[4]]}


def attn_kernel_names(head_dim, plan: dict) -> str:
    """The kernels one attention call launches under `plan`."""
    names = f"verify_attn_kernel<{head_dim}, {plan['qt']}>"
    if plan["merge"] == "merge kernel":
        names += f" + verify_attn_merge_kernel<{head_dim}, {plan['qt']}>"
    return names


def _attn_common(q, out, lse):
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("q and out must be contiguous bf16 [B][n_verify][Hq][d]")
    if out.shape != q.shape or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("out must match q; lse must be contiguous fp32 [B][Hq][n_verify]")
    B, nv, Hq, d = q.shape
    if tuple(lse.shape) != (B, Hq, nv):
        raise ValueError("lse must be [B][Hq][n_verify]")
    return B, nv, Hq, d


def dustin_sparse_verify_attn(q, k: KvView, v: KvView, Hkv: int, ctx_len, idx, count, scale: float,
                              out, lse, ws, stream=None):
    B, nv, Hq, d = _attn_common(q, out, lse)
    _dev_i32(ctx_len, "ctx_len"); _dev_i32(idx, "idx"); _dev_i32(count, "count")
    _check(_sparse(B, Hq, Hkv, d, nv, _ptr(q), ctypes.byref(k), ctypes.byref(v), _ptr(ctx_len), _ptr(idx),
                   _ptr(count), idx.shape[1], float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                   _stream(stream)), "dustin_sparse_verify_attn")


def dustin_sparse_verify_attn_logits(q, k: KvView, v: KvView, Hkv: int, ctx_len, idx, count, scale: float,
                                     out, lse, logit_sum2, ws, stream=None):
    """dustin_sparse_verify_attn that also writes, per selected token, the Collect-2 logit
    sum (queries 0 and n_verify-1, summed over the KV head's query heads) into
    logit_sum2 fp32 [B][Hkv][k_max]."""
    B, nv, Hq, d = _attn_common(q, out, lse)
    _dev_i32(ctx_len, "ctx_len"); _dev_i32(idx, "idx"); _dev_i32(count, "count")
    if (logit_sum2.dtype != torch.float32 or not logit_sum2.is_contiguous()
            or tuple(logit_sum2.shape) != (B, Hkv, idx.shape[1])):
        raise ValueError("logit_sum2 must be contiguous fp32 [B][Hkv][k_max]")
    _check(_sparse_logits(B, Hq, Hkv, d, nv, _ptr(q), ctypes.byref(k), ctypes.byref(v), _ptr(ctx_len), _ptr(idx),
                          _ptr(count), idx.shape[1], float(scale), _ptr(out), _ptr(lse), _ptr(logit_sum2), _ptr(ws),
                          ws.numel(), _stream(stream)), "dustin_sparse_verify_attn_logits")


def dustin_sparse_verify_attn_noalloc(q, k: KvView, v: KvView, Hkv: int, ctx_len, idx, count, scale: float,
                                      out, lse, stream=None):
    """dustin_sparse_verify_attn without a workspace: the library's static scratch array of
    the current device holds the split partials (no device memory is allocated)."""
    B, nv, Hq, d = _attn_common(q, out, lse)
    _dev_i32(ctx_len, "ctx_len"); _dev_i32(idx, "idx"); _dev_i32(count, "count")
    _check(_sparse_noalloc(B, Hq, Hkv, d, nv, _ptr(q), ctypes.byref(k), ctypes.byref(v), _ptr(ctx_len), _ptr(idx),
                           _ptr(count), idx.shape[1], float(scale), _ptr(out), _ptr(lse), _stream(stream)),
           "dustin_sparse_verify_attn_noalloc")


def dense_verify_attn(q, k: KvView, v: KvView, Hkv: int, ctx_len, n_max: int, scale: float, out, lse, ws,
                      stream=None):
    B, nv, Hq, d = _attn_common(q, out, lse)
    _dev_i32(ctx_len, "ctx_len")
    _check(_dense(B, Hq, Hkv, d, nv, _ptr(q), ctypes.byref(k), ctypes.byref(v), _ptr(ctx_len), int(n_max),
                  float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)),
           "dense_verify_attn")


# ------------------------------------------------------------------- KV block, recovery

def dustin_kv_write_block(k_new, v_new, ctx_len, k: KvView, v: KvView, stream=None):
    """k_new, v_new: contiguous bf16 [B][n_new][Hkv][d]; rows go to ctx_len[b] + j of the
    caches behind the views k and v (written)."""
    _dev_i32(ctx_len, "ctx_len")
    for t in (k_new, v_new):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4 or not t.is_cuda:
            raise ValueError("k_new and v_new must be contiguous bf16 device tensors [B][n_new][Hkv][d]")
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    B, n_new, Hkv, d = k_new.shape
    _check(_kv_write(B, Hkv, d, n_new, _ptr(k_new), _ptr(v_new), _ptr(ctx_len), ctypes.byref(k),
                     ctypes.byref(v), _stream(stream)), "dustin_kv_write_block")


def dustin_kv_commit(n_accept, ctx_len, n_new: int, stream=None):
    """ctx_len[b] += 1 + n_accept[b] (clamped as the header states), in place."""
    _dev_i32(n_accept, "n_accept"); _dev_i32(ctx_len, "ctx_len")
    if n_accept.shape != ctx_len.shape or n_accept.dim() != 1:
        raise ValueError("n_accept and ctx_len must both be [B]")
    _check(_kv_commit(ctx_len.shape[0], int(n_new), _ptr(n_accept), _ptr(ctx_len), _stream(stream)),
           "dustin_kv_commit")


def dustin_attn_recovery(lse_sparse, lse_dense, rec, stream=None):
    """rec = exp(lse_sparse - lse_dense), elementwise over same-shaped contiguous fp32 tensors."""
    for t in (lse_sparse, lse_dense, rec):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("lse_sparse, lse_dense and rec must be contiguous fp32 device tensors")
    if lse_sparse.shape != lse_dense.shape or rec.shape != lse_sparse.shape:
        raise ValueError("lse_sparse, lse_dense and rec must have the same shape")
    _check(_recovery(rec.numel(), _ptr(lse_sparse), _ptr(lse_dense), _ptr(rec), _stream(stream)),
           "dustin_attn_recovery")


def dustin_gather_floor(k: KvView, v: KvView, Hkv: int, head_dim: int, idx, checksum, mode: int = 0,
                        stream=None):
    """Reads the K and V rows of idx [B][k_max] (int32) the way the sparse attention does
    and computes nothing; checksum: uint32 [B][Hkv] (as int32) receives the XOR of the words
    read in mode 1."""
    _dev_i32(idx, "idx"); _dev_i32(checksum, "checksum")
    if idx.dim() != 2 or tuple(checksum.shape) != (idx.shape[0], Hkv):
        raise ValueError("idx must be [B][k_max] and checksum [B][Hkv]")
    _check(_floor(idx.shape[0], Hkv, head_dim, ctypes.byref(k), ctypes.byref(v), _ptr(idx), idx.shape[1],
                  _ptr(checksum), int(mode), _stream(stream)), "dustin_gather_floor")


def raw_library():
    """The loaded ctypes library (for callers that pre-build argument tuples)."""
    return _lib
