"""The C-ABI library: it loads, exports every function include/dustin.h declares, and
rejects bad arguments on the host with the documented status (no GPU needed: every
case here fails validation before anything is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_kv_attention_amd import dustin as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dustin.h")
FAKE = 0x10000          # a 16-byte-aligned non-null address; never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:dustin|dense)_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 18, names
    assert set(names) == set(D.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", D.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(D.raw_library(), n)


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert D.status_string(s) and D.status_string(s) != "unknown status"


def view(**kw):
    v = D.KvView()
    v.base, v.stride_batch, v.stride_token, v.stride_head = FAKE, 4 * 1024 * 128, 1024, 128
    v.n_tokens, v.n_heads = 4096, 8
    for k, val in kw.items():
        setattr(v, k, val)
    return v


def sparse(**kw):
    a = dict(B=2, Hq=64, Hkv=8, d=128, nv=5, q=FAKE, k=view(), v=view(), ctx=FAKE, idx=FAKE, cnt=FAKE,
             k_max=256, scale=0.1, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return D._sparse(a["B"], a["Hq"], a["Hkv"], a["d"], a["nv"], a["q"], ctypes.byref(a["k"]),
                     ctypes.byref(a["v"]), a["ctx"], a["idx"], a["cnt"], a["k_max"], a["scale"], a["out"],
                     a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), D.ERR_UNSUPPORTED),
    (dict(nv=17), D.ERR_UNSUPPORTED),
    (dict(Hq=60), D.ERR_INVALID_ARG),
    (dict(Hkv=0), D.ERR_INVALID_ARG),
    (dict(nv=0), D.ERR_INVALID_ARG),
    (dict(q=None), D.ERR_INVALID_ARG),
    (dict(q=FAKE + 2), D.ERR_INVALID_ARG),
    (dict(out=None), D.ERR_INVALID_ARG),
    (dict(lse=None), D.ERR_INVALID_ARG),
    (dict(ctx=None), D.ERR_INVALID_ARG),
    (dict(idx=None), D.ERR_INVALID_ARG),
    (dict(cnt=None), D.ERR_INVALID_ARG),
    (dict(k_max=-1), D.ERR_INVALID_ARG),
    (dict(scale=float("nan")), D.ERR_INVALID_ARG),
    (dict(scale=float("inf")), D.ERR_INVALID_ARG),
    (dict(scale=float("-inf")), D.ERR_INVALID_ARG),
    (dict(k=view(base=None)), D.ERR_INVALID_ARG),
    (dict(k=view(stride_token=1001)), D.ERR_INVALID_ARG),
    (dict(v=view(n_heads=4)), D.ERR_INVALID_ARG),
    (dict(v=view(n_tokens=3)), D.ERR_INVALID_ARG),
    (dict(k=view(page_table=FAKE, page_size=12, max_pages=10, num_pages=10, stride_page=4096)), D.ERR_INVALID_ARG),
    (dict(ws=None), D.ERR_WORKSPACE),
    (dict(wsb=16), D.ERR_WORKSPACE),
])
def test_sparse_attn_rejects(kw, status):
    assert sparse(**kw) == status


def test_zero_batch_is_a_noop():
    assert sparse(B=0, q=None, out=None) == D.OK


def noalloc(**kw):
    a = dict(B=2, Hq=64, Hkv=8, d=128, nv=5, q=FAKE, k=view(), v=view(), ctx=FAKE, idx=FAKE, cnt=FAKE,
             k_max=256, scale=0.1, out=FAKE, lse=FAKE)
    a.update(kw)
    return D._sparse_noalloc(a["B"], a["Hq"], a["Hkv"], a["d"], a["nv"], a["q"], ctypes.byref(a["k"]),
                             ctypes.byref(a["v"]), a["ctx"], a["idx"], a["cnt"], a["k_max"], a["scale"],
                             a["out"], a["lse"], None)


def scratch_limit():
    m = re.search(r"#define DUSTIN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def test_noalloc_attn_rejects_on_the_host():
    """The no-allocation variant validates exactly like dustin_sparse_verify_attn, and a
    shape whose workspace would exceed the static scratch array is refused before the
    device is touched."""
    n = ctypes.c_size_t(0)
    assert D._sparse_ws(64, 64, 8, 128, 9, 4096, ctypes.byref(n)) == D.OK and n.value > scratch_limit()
    v = view(n_tokens=8192)
    assert noalloc(B=64, nv=9, k_max=4096, k=v, v=v) == D.ERR_SCRATCH
    assert D._sparse_ws(8, 64, 8, 128, 5, 2048, ctypes.byref(n)) == D.OK and 0 < n.value <= scratch_limit()
    for kw, status in [(dict(d=96), D.ERR_UNSUPPORTED), (dict(Hq=60), D.ERR_INVALID_ARG),
                       (dict(q=None), D.ERR_INVALID_ARG), (dict(q=FAKE + 2), D.ERR_INVALID_ARG),
                       (dict(idx=None), D.ERR_INVALID_ARG), (dict(cnt=None), D.ERR_INVALID_ARG),
                       (dict(k_max=-1), D.ERR_INVALID_ARG), (dict(scale=float("nan")), D.ERR_INVALID_ARG),
                       (dict(k=view(stride_token=1001)), D.ERR_INVALID_ARG), (dict(out=None), D.ERR_INVALID_ARG)]:
        assert noalloc(**kw) == status, kw
    assert noalloc(B=0, q=None, out=None) == D.OK


def test_collect2_logits_call_rejects_on_the_host():
    k = view(n_tokens=8192)
    f = lambda **kw: D._sparse_logits(kw.get("B", 2), kw.get("Hq", 64), 8, 128, kw.get("nv", 5), FAKE, ctypes.byref(k),
                                      ctypes.byref(k), FAKE, FAKE, FAKE, 256, 0.1, FAKE, FAKE, kw.get("lg", FAKE),
                                      FAKE, 1 << 30, None)
    assert f(lg=None) == D.ERR_INVALID_ARG
    assert f(lg=FAKE + 2) == D.ERR_INVALID_ARG
    assert f(nv=11) == D.ERR_UNSUPPORTED          # 8 query heads x 11 queries: two query groups
    assert f(B=0) == D.OK


def test_attn_plan_query():
    """The plan query: 8 sequences x 8 KV heads with 40 query rows (64 q-heads, 5 queries)
    and a 2048-position list: 3 query tiles, one query group, four splits over 256 workgroups
    on a 256-CU plan, combined by the merge kernel."""
    import os as _os
    old = _os.environ.pop("DUSTIN_ATTN_TARGET_WGS", None)
    _os.environ["DUSTIN_ATTN_TARGET_WGS"] = "256"
    try:
        p = D.dustin_attn_plan(8, 64, 8, 128, 5, 2048)
        assert p == {"qt": 3, "qgroups": 1, "splits": 4, "workgroups": 256, "merge": "merge kernel"}, p
        assert D.attn_kernel_names(128, p) == "verify_attn_kernel<128, 3> + verify_attn_merge_kernel<128, 3>"
        assert D.dustin_attn_plan(64, 64, 8, 128, 5, 1024)["merge"] == "none"
        with pytest.raises(D.DustinError):
            D.dustin_attn_plan(8, 64, 8, 128, 5, 2048, layout=3)
    finally:
        _os.environ.pop("DUSTIN_ATTN_TARGET_WGS", None)
        if old is not None:
            _os.environ["DUSTIN_ATTN_TARGET_WGS"] = old


def test_dense_rejects():
    k = view()
    f = lambda **kw: D._dense(kw.get("B", 2), 64, 8, kw.get("d", 128), 5, FAKE, ctypes.byref(k), ctypes.byref(k),
                              FAKE, kw.get("n_max", 4000), 0.1, FAKE, FAKE, kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert f(d=64 + 1) == D.ERR_UNSUPPORTED
    assert f(n_max=-5) == D.ERR_INVALID_ARG
    assert f(ws=None) == D.ERR_WORKSPACE


def test_workspace_queries():
    n = ctypes.c_size_t(0)
    assert D._sparse_ws(8, 64, 8, 128, 5, 2048, ctypes.byref(n)) == D.OK and n.value > 0
    assert D._dense_ws(8, 64, 8, 128, 5, 32768, ctypes.byref(n)) == D.OK and n.value > 0
    assert D._sparse_ws(8, 64, 8, 96, 5, 2048, ctypes.byref(n)) == D.ERR_UNSUPPORTED
    n.value = 7
    assert D._sparse_ws(0, 64, 8, 128, 5, 2048, ctypes.byref(n)) == D.OK and n.value == 0
    n.value = 7
    assert D._dense_ws(0, 64, 8, 128, 5, 32768, ctypes.byref(n)) == D.OK and n.value == 0
    assert D._select_ws(8, 32768, ctypes.byref(n)) == D.OK
    assert n.value == 8 * (2 * 1024 + 1) * 8    # two tiers' position masks + a counter per sequence
    assert D._score_ws(8, 32768, 4, 5, D.SCORE_PROB_SUM, ctypes.byref(n)) == D.OK
    assert n.value >= 8 * 20 * 32768 * 4
    assert D._score_ws(8, 32768, 4, 5, D.SCORE_LOGIT_SUM_ALL, ctypes.byref(n)) == D.OK
    assert n.value >= 8 * 4 * 32768 * 4         # one logit row per group (a group has >= 1 head)
    assert D._score_ws(8, 32768, 4, 5, 3, ctypes.byref(n)) == D.ERR_INVALID_ARG
    assert D._score_ws(8, 32768, 4, 5, 7, ctypes.byref(n)) == D.ERR_INVALID_ARG
    assert D._score_ws(8, 32768, 4, 0, 0, ctypes.byref(n)) == D.ERR_INVALID_ARG


def test_score_rejects():
    g = (D.SrhGroup * 2)()
    for i in range(2):
        g[i].k = view()
        g[i].kv_head = i
        g[i].n_qheads = 1
    f = lambda **kw: D._score(2, kw.get("n_max", 4096), kw.get("ctx", FAKE), kw.get("ng", 2), kw.get("g", g),
                              kw.get("d", 128), kw.get("q", FAKE), kw.get("nq", 5), kw.get("scale", 0.1),
                              kw.get("mode", 0),
                              kw.get("score", FAKE), kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert f(d=32) == D.ERR_UNSUPPORTED
    assert f(ng=17) == D.ERR_UNSUPPORTED
    assert f(nq=17) == D.ERR_UNSUPPORTED
    assert f(ng=0) == D.ERR_INVALID_ARG
    assert f(mode=5) == D.ERR_INVALID_ARG
    for bad_scale in (float("nan"), float("inf"), float("-inf")):
        assert f(scale=bad_scale) == D.ERR_INVALID_ARG
    assert f(q=None) == D.ERR_INVALID_ARG
    assert f(score=None) == D.ERR_INVALID_ARG
    assert f(score=FAKE + 4) == D.ERR_INVALID_ARG      # fp32 rows are written as 16-byte vectors
    assert f(ws=None) == D.ERR_WORKSPACE
    assert f(wsb=100) == D.ERR_WORKSPACE
    bad = (D.SrhGroup * 1)()
    bad[0].k = view()
    bad[0].kv_head = 8            # the view holds 8 heads: 0..7
    bad[0].n_qheads = 1
    assert f(ng=1, g=bad) == D.ERR_INVALID_ARG
    big = (D.SrhGroup * 1)()
    big[0].k = view()
    big[0].kv_head = 0
    big[0].n_qheads = 4           # 4 heads x 5 queries = 20 softmax pairs > 16
    assert f(ng=1, g=big) == D.ERR_UNSUPPORTED
    big[0].n_qheads = 33          # 33 heads x 2 queries = 66 logit-sum pairs > 64
    assert f(ng=1, g=big, mode=1) == D.ERR_UNSUPPORTED
    big[0].n_qheads = 13          # 13 heads x 5 queries = 65 pairs over every query > 64
    assert f(ng=1, g=big, mode=D.SCORE_LOGIT_SUM_ALL) == D.ERR_UNSUPPORTED
    assert f(mode=3) == D.ERR_INVALID_ARG


def test_select_rejects():
    f = lambda **kw: D._select(2, kw.get("n_max", 4096), FAKE, kw.get("sd", FAKE), kw.get("st", FAKE), FAKE, FAKE,
                               FAKE, FAKE, kw.get("k_max", 256), kw.get("idx", FAKE), FAKE, kw.get("ws", None),
                               kw.get("wsb", 0), None)
    need = 2 * (2 * 1024 + 1) * 8
    assert f(ws=FAKE, wsb=need - 1) == D.ERR_WORKSPACE   # a workspace, but short of the query
    assert f(ws=FAKE + 8, wsb=need) == D.ERR_WORKSPACE   # not 16-byte aligned
    assert f(st=FAKE + 4) == D.ERR_INVALID_ARG        # scores are read as 16-byte vectors
    assert f(sd=FAKE + 8) == D.ERR_INVALID_ARG
    assert f(n_max=65537) == D.ERR_UNSUPPORTED
    assert f(st=None) == D.ERR_INVALID_ARG
    assert f(idx=None) == D.ERR_INVALID_ARG
    assert f(k_max=-1) == D.ERR_INVALID_ARG


def test_kv_write_block_rejects():
    k = view()
    small = view(n_tokens=4)

    def f(B=2, Hkv=8, d=128, n_new=5, kn=FAKE, vn=FAKE, ctx=FAKE, kv=k, vv=k):
        return D._kv_write(B, Hkv, d, n_new, kn, vn, ctx, ctypes.byref(kv), ctypes.byref(vv), None)

    assert f(d=96) == D.ERR_UNSUPPORTED
    assert f(n_new=17) == D.ERR_UNSUPPORTED
    assert f(n_new=0) == D.ERR_INVALID_ARG
    assert f(Hkv=0) == D.ERR_INVALID_ARG
    assert f(B=-1) == D.ERR_INVALID_ARG
    assert f(kn=None) == D.ERR_INVALID_ARG
    assert f(vn=FAKE + 8) == D.ERR_INVALID_ARG
    assert f(ctx=None) == D.ERR_INVALID_ARG
    assert f(kv=small) == D.ERR_INVALID_ARG          # the block does not fit the view
    assert f(vv=view(n_heads=4)) == D.ERR_INVALID_ARG
    assert f(B=0, kn=None, vn=None, ctx=None) == D.OK


def test_gather_floor_rejects():
    k = view()

    def f(B=2, Hkv=8, d=128, kv=k, vv=k, idx=FAKE, k_max=2048, ck=FAKE, mode=0):
        return D._floor(B, Hkv, d, ctypes.byref(kv), ctypes.byref(vv), idx, k_max, ck, mode, None)

    assert f(d=96) == D.ERR_UNSUPPORTED
    assert f(mode=2) == D.ERR_INVALID_ARG
    assert f(Hkv=0) == D.ERR_INVALID_ARG
    assert f(B=-1) == D.ERR_INVALID_ARG
    assert f(k_max=-1) == D.ERR_INVALID_ARG
    assert f(idx=None) == D.ERR_INVALID_ARG
    assert f(ck=None) == D.ERR_INVALID_ARG
    assert f(ck=FAKE + 2) == D.ERR_INVALID_ARG
    assert f(vv=view(n_heads=4)) == D.ERR_INVALID_ARG
    assert f(kv=view(page_table=FAKE, page_size=16, max_pages=8, num_pages=8, stride_page=16 * 1024)) \
        == D.ERR_UNSUPPORTED
    assert f(B=0, idx=None, ck=None) == D.OK
    assert f(k_max=0, idx=None, ck=None) == D.OK


def test_kv_commit_and_recovery_reject():
    assert D._kv_commit(2, 0, FAKE, FAKE, None) == D.ERR_INVALID_ARG
    assert D._kv_commit(2, 17, FAKE, FAKE, None) == D.ERR_UNSUPPORTED
    assert D._kv_commit(2, 5, None, FAKE, None) == D.ERR_INVALID_ARG
    assert D._kv_commit(2, 5, FAKE, None, None) == D.ERR_INVALID_ARG
    assert D._kv_commit(0, 5, None, None, None) == D.OK
    assert D._recovery(-1, FAKE, FAKE, FAKE, None) == D.ERR_INVALID_ARG
    assert D._recovery(10, None, FAKE, FAKE, None) == D.ERR_INVALID_ARG
    assert D._recovery(10, FAKE, FAKE, None, None) == D.ERR_INVALID_ARG
    assert D._recovery(0, None, None, None, None) == D.OK
