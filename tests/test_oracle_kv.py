"""Pins of the oracle's KV block write and commit (English Dustin summary, Verification
Workflow step 5: accepted tokens are appended to the cache, rejected ones discarded).

The written block is checked through attention: the library's scaled_dot_product_attention
over the context rows followed by the block rows (concatenated by torch) must equal the
oracle's dense verification attention over the written cache, which reads the new tokens
at ctx_len + j.  Rows outside the block stay untouched.  The commit is checked on a
hand-derived example and through the next step's attention over the kept prefix.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def bf16(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.float32).to(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def setup(seed, B=3, n_cap=48, Hkv=2, d=16, n_new=5):
    rng = np.random.default_rng(seed)
    K = bf16(rng.standard_normal((B, n_cap, Hkv, d)))
    V = bf16(rng.standard_normal((B, n_cap, Hkv, d)))
    Kn = bf16(rng.standard_normal((B, n_new, Hkv, d)))
    Vn = bf16(rng.standard_normal((B, n_new, Hkv, d)))
    ctx = np.array([30, 0, 43][:B], np.int32)          # 43 + 5 == n_cap: the block ends the cache
    return rng, K, V, Kn, Vn, ctx


def test_written_block_is_what_attention_sees():
    rng, K, V, Kn, Vn, ctx = setup(0)
    B, n_new, Hkv, d = Kn.shape
    Hq = 4
    G = Hq // Hkv
    Kw, Vw = O.kv_write_block(bits(Kn), bits(Vn), ctx, bits(K), bits(V))
    Q = bf16(rng.standard_normal((B, n_new, Hq, d)))
    Ov, _ = O.verify_attn(bits(Q), Kw, Vw, ctx, None, None, 0.25, Hkv)
    for b in range(B):
        N = int(ctx[b])
        k = torch.cat([K[b, :N], Kn[b]]).double()        # [N + n_new][Hkv][d]
        v = torch.cat([V[b, :N], Vn[b]]).double()
        mask = torch.zeros(n_new, N + n_new, dtype=torch.bool)
        mask[:, :N] = True
        for t in range(n_new):
            mask[t, N:N + t + 1] = True
        for h in range(Hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[b, :, h].double()[None], k[None, :, h // G], v[None, :, h // G], attn_mask=mask[None],
                scale=0.25)[0]
            np.testing.assert_allclose(Ov[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_rows_outside_the_block_are_untouched():
    _, K, V, Kn, Vn, ctx = setup(1)
    n_new = Kn.shape[1]
    Kw, Vw = O.kv_write_block(bits(Kn), bits(Vn), ctx, bits(K), bits(V))
    for b in range(K.shape[0]):
        keep = np.ones(K.shape[1], bool)
        keep[ctx[b]:ctx[b] + n_new] = False
        assert np.array_equal(Kw[b, keep], bits(K)[b, keep]) and np.array_equal(Vw[b, keep], bits(V)[b, keep])


def test_block_past_the_capacity_is_rejected():
    _, K, V, Kn, Vn, _ = setup(2)
    with pytest.raises(ValueError):
        O.kv_write_block(bits(Kn), bits(Vn), np.array([30, 0, 44], np.int32), bits(K), bits(V))


def test_commit_worked_example():
    # block of 5 rows (the previous step's token + 4 drafts): 0 drafts accepted keeps 1
    # row, all 4 accepted keeps 5, 2 accepted keeps 3
    assert O.kv_commit([10, 20, 0], [0, 4, 2], 5).tolist() == [11, 25, 3]
    for bad in ([-1, 0, 0], [0, 5, 0]):
        with pytest.raises(ValueError):
            O.kv_commit([10, 20, 0], bad, 5)


def test_next_step_attends_to_the_kept_prefix_only():
    rng, K, V, Kn, Vn, ctx = setup(3)
    B, n_new, Hkv, d = Kn.shape
    ctx = np.array([30, 0, 38], np.int32)
    Kw, Vw = O.kv_write_block(bits(Kn), bits(Vn), ctx, bits(K), bits(V))
    acc = np.array([2, 0, 4], np.int32)
    new_ctx = O.kv_commit(ctx, acc, n_new)
    # the next step writes its one-row block behind the committed prefix and attends
    k1 = bf16(rng.standard_normal((B, 1, Hkv, d)))
    v1 = bf16(rng.standard_normal((B, 1, Hkv, d)))
    Kw, Vw = O.kv_write_block(bits(k1), bits(v1), new_ctx, Kw, Vw)
    q = bf16(rng.standard_normal((B, 1, Hkv, d)))
    Ov, _ = O.verify_attn(bits(q), Kw, Vw, new_ctx, None, None, 0.5, Hkv)
    for b in range(B):
        N, a = int(ctx[b]), int(acc[b])
        k = torch.cat([K[b, :N], Kn[b, :a + 1], k1[b]]).double()
        v = torch.cat([V[b, :N], Vn[b, :a + 1], v1[b]]).double()
        for h in range(Hkv):
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[b, :, h].double()[None], k[None, :, h], v[None, :, h], scale=0.5)[0]
            np.testing.assert_allclose(Ov[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-13)
