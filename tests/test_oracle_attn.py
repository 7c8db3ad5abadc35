"""Pins of the oracle's verification attention.

English Dustin summary, Verification Workflow 3-4: the target verifies the draft block
against the selected tokens only; each verify query t also sees new tokens 0..t.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.float32).to(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def make(rng, B, n_cap, Hq, Hkv, d, nv, scale=1.0):
    Q = bf16(rng.standard_normal((B, nv, Hq, d)) * scale)
    K = bf16(rng.standard_normal((B, n_cap, Hkv, d)) * scale)
    V = bf16(rng.standard_normal((B, n_cap, Hkv, d)))
    return Q, K, V


def test_worked_example():
    for c in json.load(open(os.path.join(GOLD, "attn_worked.json")))["cases"]:
        d = c["d"]
        Q = bf16(np.array(c["q"]).reshape(1, 1, 1, d))
        K = bf16(np.array([c["k_sel"], c["k_new"]]).reshape(1, 2, 1, d))
        V = bf16(np.array([c["v_sel"], c["v_new"]]).reshape(1, 2, 1, d))
        Ov, lse = O.verify_attn(bits(Q), bits(K), bits(V), [c["ctx_len"]], np.array([[0]]),
                                np.array([1]), c["scale"], 1)
        np.testing.assert_allclose(Ov[0, 0, 0], c["expect_o"], rtol=0, atol=1e-15)
        assert abs(lse[0, 0, 0] - c["expect_lse"]) < 1e-15


@pytest.mark.parametrize("scale", [0.3, -0.3, 0.0])
def test_matches_torch_sdpa_float64(scale):
    """Any finite scale, negative and zero included; at zero every attended row has the
    same weight, so O is the plain mean of the attended V rows and LSE = ln(count)."""
    rng = np.random.default_rng(0)
    B, N, Hq, Hkv, d, nv = 2, 40, 6, 2, 16, 3
    n_cap = N + nv
    Q, K, V = make(rng, B, n_cap, Hq, Hkv, d, nv)
    ctx = np.array([40, 25])
    k_max = 12
    idx = np.full((B, k_max), -1, np.int32)
    cnt = np.array([12, 7], np.int32)
    for b in range(B):
        idx[b, :cnt[b]] = np.sort(rng.choice(ctx[b], cnt[b], replace=False))
    Ov, lse = O.verify_attn(bits(Q), bits(K), bits(V), ctx, idx, cnt, scale, Hkv)
    G = Hq // Hkv
    for b in range(B):
        rows = list(idx[b, :cnt[b]]) + [ctx[b] + j for j in range(nv)]
        mask = torch.zeros(nv, len(rows), dtype=torch.bool)
        mask[:, :cnt[b]] = True
        for t in range(nv):
            mask[t, cnt[b]:cnt[b] + t + 1] = True
        for h in range(Hq):
            q = Q[b, :, h].double()                       # [nv][d]
            k = K[b, rows, h // G].double()
            v = V[b, rows, h // G].double()
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None], k[None], v[None], attn_mask=mask[None], scale=scale)[0]
            np.testing.assert_allclose(Ov[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-13)
            lg = (q @ k.T) * scale
            lg[~mask] = -np.inf
            np.testing.assert_allclose(lse[b, h], torch.logsumexp(lg, -1).numpy(), rtol=1e-13)
            if scale == 0.0:
                for t in range(nv):
                    np.testing.assert_allclose(Ov[b, t, h], v[mask[t]].mean(0).numpy(), rtol=1e-12, atol=1e-13)
                    assert abs(lse[b, h, t] - np.log(int(mask[t].sum()))) < 1e-13


def test_full_budget_equals_dense():
    rng = np.random.default_rng(1)
    B, N, Hq, Hkv, d, nv = 1, 30, 4, 2, 8, 5
    Q, K, V = make(rng, B, N + nv, Hq, Hkv, d, nv)
    idx = np.arange(N, dtype=np.int32)[None]
    a = O.verify_attn(bits(Q), bits(K), bits(V), [N], idx, [N], 0.4, Hkv)
    b = O.verify_attn(bits(Q), bits(K), bits(V), [N], None, None, 0.4, Hkv)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_single_key_and_equal_keys():
    rng = np.random.default_rng(2)
    Q, K, V = make(rng, 1, 20, 2, 1, 8, 1)
    Ov, lse = O.verify_attn(bits(Q), bits(K), bits(V), [10], np.zeros((1, 4), np.int32),
                            [0], 0.5, 1)                       # nothing selected: new token only
    np.testing.assert_array_equal(Ov[0, 0, :], V[0, 10, 0].double().numpy()[None].repeat(2, 0))
    s = 0.5 * (Q[0, 0].double() @ K[0, 10, 0].double()).numpy()
    np.testing.assert_allclose(lse[0, :, 0], s, rtol=1e-14)
    # every key equal: output is the plain mean of the values
    K2 = bf16(np.tile(rng.standard_normal(8), (1, 20, 1, 1)))
    sel = np.array([[0, 3, 4, 9]], np.int32)
    Ov, _ = O.verify_attn(bits(Q), bits(K2), bits(V), [10], sel, [4], 0.5, 1)
    mean = V[0, [0, 3, 4, 9, 10], 0].double().mean(0).numpy()
    np.testing.assert_allclose(Ov[0, 0, 0], mean, rtol=1e-13, atol=1e-15)


def test_causal_block_invariance():
    rng = np.random.default_rng(3)
    N, nv = 25, 4
    Q, K, V = make(rng, 1, N + nv, 4, 2, 16, nv)
    sel = np.array([[1, 5, 7, 20]], np.int32)
    a = O.verify_attn(bits(Q), bits(K), bits(V), [N], sel, [4], 0.25, 2)
    K2, V2 = K.clone(), V.clone()
    K2[0, N + 2:] = bf16(rng.standard_normal((nv - 2, 2, 16)))
    V2[0, N + 2:] = bf16(rng.standard_normal((nv - 2, 2, 16)))
    b = O.verify_attn(bits(Q), bits(K2), bits(V2), [N], sel, [4], 0.25, 2)
    np.testing.assert_array_equal(a[0][0, :2], b[0][0, :2])     # queries 0,1 unchanged
    np.testing.assert_array_equal(a[1][0, :, :2], b[1][0, :, :2])
    assert not np.array_equal(a[0][0, 2:], b[0][0, 2:])


def test_split_lse_combine():
    """Attention over S1 u S2 u C from the parts: Z = Z1 + Z2 - Zc and
    O*Z = O1*Z1 + O2*Z2 - Oc*Zc, with Z = exp(LSE) and C the causal block."""
    rng = np.random.default_rng(4)
    N, nv, Hq, Hkv, d = 60, 3, 4, 2, 16
    Q, K, V = make(rng, 1, N + nv, Hq, Hkv, d, nv, 0.5)
    s1 = np.sort(rng.choice(N, 20, replace=False))
    rest = np.setdiff1d(np.arange(N), s1)
    s2 = np.sort(rng.choice(rest, 15, replace=False))
    both = np.sort(np.concatenate([s1, s2]))

    def run(sel):
        sel = np.asarray(sel, np.int32)
        return O.verify_attn(bits(Q), bits(K), bits(V), [N], sel[None], [len(sel)], 0.3, Hkv)

    o1, l1 = run(s1)
    o2, l2 = run(s2)
    oc, lc = O.verify_attn(bits(Q), bits(K), bits(V), [N], np.zeros((1, 1), np.int32), [0], 0.3, Hkv)
    ob, lb = run(both)
    z1, z2, zc = np.exp(l1), np.exp(l2), np.exp(lc)
    np.testing.assert_allclose(np.exp(lb), z1 + z2 - zc, rtol=1e-12)
    zt = lambda z: np.transpose(z, (0, 2, 1))[..., None]       # [B][Hq][nv] -> [B][nv][Hq][1]
    comb = (o1 * zt(z1) + o2 * zt(z2) - oc * zt(zc)) / zt(z1 + z2 - zc)
    np.testing.assert_allclose(ob, comb, rtol=1e-10, atol=1e-12)
