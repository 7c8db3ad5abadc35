"""Pins of the oracle's attention recovery (the share of full-cache attention probability
that the kept set carries; the English Dustin summary, "Methodology" 2, names this rate
as the objective of its offline SRH search without defining it).

The pins do not retype the oracle's sum: the library's scaled_dot_product_attention
with a 0/1 membership column as the value computes the same share; the oracle's own
attention (a separate function) gives it as exp(LSE_sparse - LSE_dense); uniform logits
give a closed form; full budget gives 1; kept set and its complement partition the mass.
"""
import numpy as np
import torch

from oracle import oracle as O


def bf16(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.float32).to(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def case(seed, B=2, N=37, Hq=6, Hkv=2, d=16, nv=4, k_max=11, counts=(11, 5), scale=0.4):
    rng = np.random.default_rng(seed)
    n_cap = N + nv
    Q = bf16(rng.standard_normal((B, nv, Hq, d)))
    K = bf16(rng.standard_normal((B, n_cap, Hkv, d)))
    ctx = np.array([N, N - 9][:B], np.int32)
    idx = np.full((B, k_max), -1, np.int32)
    cnt = np.array(counts[:B], np.int32)
    for b in range(B):
        idx[b, :cnt[b]] = np.sort(rng.choice(ctx[b], cnt[b], replace=False))
    return Q, K, ctx, idx, cnt, scale


def test_matches_sdpa_with_membership_values():
    Q, K, ctx, idx, cnt, scale = case(0)
    B, nv, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    rec = O.attn_recovery(bits(Q), bits(K), ctx, idx, cnt, scale, Hkv)
    for b in range(B):
        N = int(ctx[b])
        rows = N + nv
        member = torch.zeros(rows, 1, dtype=torch.float64)
        member[idx[b, :cnt[b]]] = 1.0
        member[N:] = 1.0                     # the new tokens are seen by both attentions
        mask = torch.zeros(nv, rows, dtype=torch.bool)
        mask[:, :N] = True
        for t in range(nv):
            mask[t, N:N + t + 1] = True
        for h in range(Hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[b, :, h].double()[None], K[b, :rows, h // G].double()[None], member[None],
                attn_mask=mask[None], scale=scale)[0, :, 0]
            np.testing.assert_allclose(rec[b, h], ref.numpy(), rtol=1e-12, atol=1e-15)


def test_equals_exp_of_lse_difference_from_oracle_attention():
    Q, K, ctx, idx, cnt, scale = case(1)
    Hkv = K.shape[2]
    V = bits(bf16(np.zeros(K.shape)))
    rec = O.attn_recovery(bits(Q), bits(K), ctx, idx, cnt, scale, Hkv)
    _, lse_s = O.verify_attn(bits(Q), bits(K), V, ctx, idx, cnt, scale, Hkv)
    _, lse_d = O.verify_attn(bits(Q), bits(K), V, ctx, None, None, scale, Hkv)
    np.testing.assert_allclose(rec, np.exp(lse_s - lse_d), rtol=1e-12)


def test_full_budget_recovers_everything():
    Q, K, ctx, _, _, scale = case(2)
    B = Q.shape[0]
    k_max = int(ctx.max())
    idx = np.full((B, k_max), -1, np.int32)
    for b in range(B):
        idx[b, :ctx[b]] = np.arange(ctx[b])
    rec = O.attn_recovery(bits(Q), bits(K), ctx, idx, ctx, scale, K.shape[2])
    np.testing.assert_allclose(rec, 1.0, rtol=0, atol=1e-14)


def test_uniform_logits_closed_form():
    # zero queries: every logit is 0, so each kept row carries 1/(N + t + 1) of the mass
    Q, K, ctx, idx, cnt, scale = case(3)
    Qz = bits(bf16(np.zeros(Q.shape)))
    rec = O.attn_recovery(Qz, bits(K), ctx, idx, cnt, scale, K.shape[2])
    for b in range(Q.shape[0]):
        for t in range(Q.shape[1]):
            want = (cnt[b] + t + 1) / (ctx[b] + t + 1)
            np.testing.assert_allclose(rec[b, :, t], want, rtol=1e-14)


def test_kept_set_and_complement_partition_the_mass():
    Q, K, ctx, idx, cnt, scale = case(4)
    B, nv = Q.shape[:2]
    Hkv = K.shape[2]
    k_max = int(ctx.max())
    comp = np.full((B, k_max), -1, np.int32)
    ccnt = np.zeros(B, np.int32)
    empty = np.full((B, 1), -1, np.int32)
    for b in range(B):
        rest = np.setdiff1d(np.arange(ctx[b]), idx[b, :cnt[b]])
        comp[b, :len(rest)] = rest
        ccnt[b] = len(rest)
    r_in = O.attn_recovery(bits(Q), bits(K), ctx, idx, cnt, scale, Hkv)
    r_out = O.attn_recovery(bits(Q), bits(K), ctx, comp, ccnt, scale, Hkv)
    r_new = O.attn_recovery(bits(Q), bits(K), ctx, empty, np.zeros(B, np.int32), scale, Hkv)
    np.testing.assert_allclose(r_in + r_out, 1.0 + r_new, rtol=1e-13)
    assert (r_new > 0).all() and (r_in >= r_new).all() and (r_in <= 1.0 + 1e-15).all()


def test_growing_the_set_never_lowers_recovery():
    Q, K, ctx, idx, cnt, scale = case(5, counts=(6, 3))
    Hkv = K.shape[2]
    rng = np.random.default_rng(9)
    big = idx.copy()
    bcnt = cnt.copy()
    for b in range(Q.shape[0]):
        extra = np.setdiff1d(np.arange(ctx[b]), idx[b, :cnt[b]])
        add = rng.choice(extra, 4, replace=False)
        rows = np.sort(np.concatenate([idx[b, :cnt[b]], add]))
        big[b, :len(rows)] = rows
        bcnt[b] = len(rows)
    r_small = O.attn_recovery(bits(Q), bits(K), ctx, idx, cnt, scale, Hkv)
    r_big = O.attn_recovery(bits(Q), bits(K), ctx, big, bcnt, scale, Hkv)
    assert (r_big >= r_small - 1e-15).all() and (r_big > r_small).any()
