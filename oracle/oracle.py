"""ctypes wrapper of the C oracle — TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the bench's CPU-baseline leg import this module.  It
takes numpy arrays (bf16 passed as uint16 bit patterns) and returns numpy arrays; it
imports nothing from the HIP library's package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
PROB_SUM, LOGIT_SUM2, LOGIT_SUM_ALL = 0, 1, 2

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, -O2, no fused multiply-add)."""
    src = os.path.join(HERE, "oracle.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < max(
            os.path.getmtime(src), os.path.getmtime(os.path.join(HERE, "oracle.h"))):
        tmp = LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-std=c99", "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()   # no-op unless the library is missing or older than its sources
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_score_stream.argtypes = [i, i, i, P, i, P, i, i, P, ctypes.c_double, i, P]
        L.oracle_select.argtypes = [i, i, P, P, P, P, P, P, P, i, P, P]
        L.oracle_verify_attn.argtypes = [i, i, i, i, i, P, P, P, i, P, P, P, i,
                                         ctypes.c_double, P, P]
        L.oracle_attn_recovery.argtypes = [i, i, i, i, i, P, P, i, P, P, P, i, ctypes.c_double, P]
        L.oracle_kv_write_block.argtypes = [i, i, i, i, P, P, P, P, P, i]
        L.oracle_kv_commit.argtypes = [i, i, P, P]
        for f in (L.oracle_score_stream, L.oracle_select, L.oracle_verify_attn, L.oracle_attn_recovery,
                  L.oracle_kv_write_block, L.oracle_kv_commit):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def score_stream(K, Q, ctx_len, n_max, scale, mode, acc=None):
    """Add one stream's scores into acc [B][n_max] (float64).
    K: uint16 [B][n_rows][d]; Q: uint16 [B][n_heads][n_q][d]."""
    K, Q, ctx_len = _u16(K), _u16(Q), _i32(ctx_len)
    B, n_rows, d = K.shape
    _, n_heads, n_q, dq = Q.shape
    assert dq == d and Q.shape[0] == B
    if acc is None:
        acc = np.zeros((B, n_max), dtype=np.float64)
    assert acc.dtype == np.float64 and acc.flags.c_contiguous and acc.shape == (B, n_max)
    rc = lib().oracle_score_stream(B, n_rows, n_max, _p(ctx_len), d, _p(K), n_heads, n_q,
                                   _p(Q), float(scale), int(mode), _p(acc))
    if rc:
        raise ValueError(f"oracle_score_stream rc={rc}")
    return acc


def select(ctx_len, score_draft, score_target, budget, n_sink, n_window, m, k_max):
    """Returns (idx int32 [B][k_max], count int32 [B])."""
    st = np.ascontiguousarray(score_target, dtype=np.float64)
    sd = None if score_draft is None else np.ascontiguousarray(score_draft, dtype=np.float64)
    B, n_max = st.shape
    ctx_len, budget, n_sink, n_window, m = map(_i32, (ctx_len, budget, n_sink, n_window, m))
    idx = np.empty((B, k_max), dtype=np.int32)
    count = np.empty((B,), dtype=np.int32)
    rc = lib().oracle_select(B, n_max, _p(ctx_len), _p(sd), _p(st), _p(budget), _p(n_sink),
                             _p(n_window), _p(m), int(k_max), _p(idx), _p(count))
    if rc:
        raise ValueError(f"oracle_select rc={rc}")
    return idx, count


def verify_attn(Q, K, V, ctx_len, idx, count, scale, Hkv):
    """Q: uint16 [B][n_verify][Hq][d]; K, V: uint16 [B][n_cap][Hkv][d];
    idx int32 [B][k_max] or None (dense).  Returns (O float64 [B][nv][Hq][d], lse [B][Hq][nv])."""
    Q, K, V, ctx_len = _u16(Q), _u16(K), _u16(V), _i32(ctx_len)
    B, nv, Hq, d = Q.shape
    n_cap = K.shape[1]
    assert K.shape == (B, n_cap, Hkv, d) and V.shape == K.shape
    if idx is not None:
        idx, count = _i32(idx), _i32(count)
        k_max = idx.shape[1]
    else:
        k_max = 0
    O = np.empty((B, nv, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, nv), dtype=np.float64)
    rc = lib().oracle_verify_attn(B, Hq, Hkv, d, nv, _p(Q), _p(K), _p(V), n_cap, _p(ctx_len),
                                  _p(idx), _p(count), k_max, float(scale), _p(O), _p(lse))
    if rc:
        raise ValueError(f"oracle_verify_attn rc={rc}")
    return O, lse


def attn_recovery(Q, K, ctx_len, idx, count, scale, Hkv):
    """Share of the dense attention probability on I_b plus the new tokens 0..t.
    Q: uint16 [B][n_verify][Hq][d]; K: uint16 [B][n_cap][Hkv][d]; idx int32 [B][k_max].
    Returns float64 [B][Hq][n_verify]."""
    Q, K, ctx_len, idx, count = _u16(Q), _u16(K), _i32(ctx_len), _i32(idx), _i32(count)
    B, nv, Hq, d = Q.shape
    n_cap = K.shape[1]
    assert K.shape == (B, n_cap, Hkv, d)
    rec = np.empty((B, Hq, nv), dtype=np.float64)
    rc = lib().oracle_attn_recovery(B, Hq, Hkv, d, nv, _p(Q), _p(K), n_cap, _p(ctx_len), _p(idx),
                                    _p(count), idx.shape[1], float(scale), _p(rec))
    if rc:
        raise ValueError(f"oracle_attn_recovery rc={rc}")
    return rec


def kv_write_block(Knew, Vnew, ctx_len, K, V):
    """Returns copies of K, V ([B][n_cap][Hkv][d] uint16) with the block rows
    Knew/Vnew [B][n_new][Hkv][d] stored at ctx_len[b] + j."""
    Knew, Vnew, ctx_len = _u16(Knew), _u16(Vnew), _i32(ctx_len)
    K, V = _u16(K).copy(), _u16(V).copy()
    B, n_cap, Hkv, d = K.shape
    n_new = Knew.shape[1]
    assert Knew.shape == (B, n_new, Hkv, d) and Vnew.shape == Knew.shape and V.shape == K.shape
    rc = lib().oracle_kv_write_block(B, Hkv, d, n_new, _p(Knew), _p(Vnew), _p(ctx_len), _p(K), _p(V), n_cap)
    if rc:
        raise ValueError(f"oracle_kv_write_block rc={rc}")
    return K, V


def kv_commit(ctx_len, n_accept, n_new):
    """Returns the committed context lengths (int32 [B])."""
    ctx = _i32(ctx_len).copy()
    n_accept = _i32(n_accept)
    rc = lib().oracle_kv_commit(ctx.shape[0], int(n_new), _p(n_accept), _p(ctx))
    if rc:
        raise ValueError(f"oracle_kv_commit rc={rc}")
    return ctx
