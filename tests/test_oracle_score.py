"""Pins of the oracle's SRH scoring.

English Dustin summary, Methodology 1-2: per-token importance = attention scores of the
SRH queries (softmax probabilities), aggregated over the SRH (head, query) pairs.
German Vegas summary 2A/2B: raw logits summed over heads and the first/bonus queries.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import oracle as O


def bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_stream(rng, B, n, d, nh, nq, scale=1.0):
    K = bf16(rng.standard_normal((B, n, d)) * scale)
    Q = bf16(rng.standard_normal((B, nh, nq, d)) * scale)
    return K, Q


@pytest.mark.parametrize("scale", [0.25, -0.25, 0.0])
def test_matches_torch_softmax_float64(scale):
    """Any finite scale, negative and zero included; at zero every pair's softmax is
    uniform, so each token scores (pairs) / N."""
    rng = np.random.default_rng(0)
    B, n, d, nh, nq = 2, 37, 16, 3, 4
    K, Q = rand_stream(rng, B, n, d, nh, nq)
    ctx = np.array([37, 20])
    acc = O.score_stream(bits(K), bits(Q), ctx, n, scale, O.PROB_SUM)
    if scale == 0.0:
        for b in range(B):
            np.testing.assert_allclose(acc[b, :ctx[b]], nh * nq / ctx[b], rtol=1e-13)
    for b in range(B):
        nb = ctx[b]
        lg = torch.einsum("hqd,nd->hqn", Q[b].double(), K[b, :nb].double()) * scale
        ref = torch.softmax(lg, dim=-1).sum(dim=(0, 1)).numpy()
        np.testing.assert_allclose(acc[b, :nb], ref, rtol=1e-12, atol=1e-15)
        assert np.all(acc[b, nb:] == 0)


def test_sum_equals_pair_count():
    rng = np.random.default_rng(1)
    K, Q = rand_stream(rng, 1, 300, 64, 2, 5, 3.0)
    acc = O.score_stream(bits(K), bits(Q), [300], 300, 1 / 8, O.PROB_SUM)
    assert abs(acc.sum() - 10.0) < 1e-9


def test_uniform_keys_give_uniform_scores():
    rng = np.random.default_rng(2)
    k = rng.standard_normal(32)
    K = bf16(np.tile(k, (1, 50, 1)))
    Q = bf16(rng.standard_normal((1, 2, 3, 32)))
    acc = O.score_stream(bits(K), bits(Q), [50], 64, 0.3, O.PROB_SUM)
    np.testing.assert_allclose(acc[0, :50], 6.0 / 50, rtol=1e-12)


def test_single_token_context():
    rng = np.random.default_rng(3)
    K, Q = rand_stream(rng, 1, 4, 16, 3, 2)
    acc = O.score_stream(bits(K), bits(Q), [1], 4, 0.5, O.PROB_SUM)
    assert acc[0, 0] == 6.0 and np.all(acc[0, 1:] == 0)


def test_accumulates_across_streams():
    rng = np.random.default_rng(4)
    K1, Q1 = rand_stream(rng, 1, 40, 16, 1, 4)
    K2, Q2 = rand_stream(rng, 1, 40, 32, 2, 5)
    a = O.score_stream(bits(K1), bits(Q1), [40], 40, 0.25, O.PROB_SUM)
    O.score_stream(bits(K2), bits(Q2), [40], 40, 0.125, O.PROB_SUM, acc=a)
    b1 = O.score_stream(bits(K1), bits(Q1), [40], 40, 0.25, O.PROB_SUM)
    b2 = O.score_stream(bits(K2), bits(Q2), [40], 40, 0.125, O.PROB_SUM)
    np.testing.assert_allclose(a, b1 + b2, rtol=1e-14)
    assert abs(a.sum() - 14.0) < 1e-9


def test_logit_sum2_closed_form():
    """Heads sharing one key stream: score_i = scale * (sum of the first and last query
    of every head) . k_i, a single matrix-vector product."""
    rng = np.random.default_rng(5)
    B, n, d, nh, nq = 2, 50, 32, 4, 5
    K, Q = rand_stream(rng, B, n, d, nh, nq)
    acc = O.score_stream(bits(K), bits(Q), [n, 31], n, 0.2, O.LOGIT_SUM2)
    for b, nb in ((0, n), (1, 31)):
        qsum = Q[b, :, 0].double().sum(0) + Q[b, :, nq - 1].double().sum(0)
        ref = 0.2 * (K[b, :nb].double().numpy() @ qsum.numpy())
        np.testing.assert_allclose(acc[b, :nb], ref, rtol=1e-12, atol=1e-12)
        assert np.all(acc[b, nb:] == 0)
    # one query: query 0 is counted once
    K1, Q1 = rand_stream(rng, 1, 10, 8, 1, 1)
    a1 = O.score_stream(bits(K1), bits(Q1), [10], 10, 1.0, O.LOGIT_SUM2)
    np.testing.assert_allclose(a1[0], K1[0].double().numpy() @ Q1[0, 0, 0].double().numpy(), rtol=1e-12)


def test_vegas_objective_argmax_is_topk():
    """The Vegas aggregated-logit objective (German Vegas summary 2A) is maximised over
    all size-k subsets by brute force; with the Collect-2 queries (2B) it must equal the
    oracle's pure top-k selection on the LOGIT_SUM2 score."""
    rng = np.random.default_rng(6)
    for trial in range(6):
        n, d, nh, nq, k = 12, 8, 2, 4, 5
        K, Q = rand_stream(rng, 1, n, d, nh, nq)
        scale = 0.5
        acc = O.score_stream(bits(K), bits(Q), [n], n, scale, O.LOGIT_SUM2)
        L = np.einsum("hqd,nd->hqn", Q[0].double().numpy(), K[0].double().numpy()) * scale
        best, best_set = -np.inf, None
        for T in itertools.combinations(range(n), k):
            v = sum(L[h, t, i] for t in (0, nq - 1) for h in range(nh) for i in T)
            if v > best + 1e-12:
                best, best_set = v, T
        idx, cnt = O.select([n], None, acc, [k], [0], [0], [0], k)
        assert tuple(idx[0, :cnt[0]]) == tuple(sorted(best_set))


def test_logit_sum_all_closed_form():
    """The full Vegas aggregate (German Vegas summary 2A: raw logits summed over every
    query and head) is linear in the queries: score_i = scale * (sum of all queries) . k_i,
    one matrix-vector product with the summed query."""
    rng = np.random.default_rng(7)
    B, n, d, nh, nq = 2, 40, 16, 3, 5
    K, Q = rand_stream(rng, B, n, d, nh, nq)
    acc = O.score_stream(bits(K), bits(Q), [n, 17], n, 0.3, O.LOGIT_SUM_ALL)
    for b, nb in ((0, n), (1, 17)):
        qsum = Q[b].double().reshape(-1, d).sum(0).numpy()
        ref = 0.3 * (K[b, :nb].double().numpy() @ qsum)
        np.testing.assert_allclose(acc[b, :nb], ref, rtol=1e-12, atol=1e-12)
        assert np.all(acc[b, nb:] == 0)


def test_logit_sum_all_reduces_to_collect2_for_two_queries():
    """With at most two queries the first and last query are all of them, so the full
    aggregate and the Collect-2 restriction (2B) coincide."""
    rng = np.random.default_rng(8)
    for nq in (1, 2):
        K, Q = rand_stream(rng, 2, 30, 8, 2, nq)
        a = O.score_stream(bits(K), bits(Q), [30, 11], 30, 0.7, O.LOGIT_SUM_ALL)
        b = O.score_stream(bits(K), bits(Q), [30, 11], 30, 0.7, O.LOGIT_SUM2)
        np.testing.assert_array_equal(a, b)
    # with more queries the middle ones count: the difference is their own logit sum
    K, Q = rand_stream(rng, 1, 20, 8, 2, 4)
    a = O.score_stream(bits(K), bits(Q), [20], 20, 1.0, O.LOGIT_SUM_ALL)
    b = O.score_stream(bits(K), bits(Q), [20], 20, 1.0, O.LOGIT_SUM2)
    mid = K[0].double().numpy() @ Q[0, :, 1:3].double().reshape(-1, 8).sum(0).numpy()
    np.testing.assert_allclose(a[0] - b[0], mid, rtol=1e-12, atol=1e-12)


def test_vegas_full_objective_argmax_is_topk():
    """Brute force over all size-k subsets of the objective summed over every query and
    head equals the oracle's pure top-k on the LOGIT_SUM_ALL score."""
    rng = np.random.default_rng(9)
    for trial in range(6):
        n, d, nh, nq, k = 12, 8, 2, 5, 4
        K, Q = rand_stream(rng, 1, n, d, nh, nq)
        acc = O.score_stream(bits(K), bits(Q), [n], n, 0.5, O.LOGIT_SUM_ALL)
        L = np.einsum("hqd,nd->hqn", Q[0].double().numpy(), K[0].double().numpy()) * 0.5
        best, best_set = -np.inf, None
        for T in itertools.combinations(range(n), k):
            v = sum(L[h, t, i] for t in range(nq) for h in range(nh) for i in T)
            if v > best + 1e-12:
                best, best_set = v, T
        idx, cnt = O.select([n], None, acc, [k], [0], [0], [0], k)
        assert tuple(idx[0, :cnt[0]]) == tuple(sorted(best_set))
