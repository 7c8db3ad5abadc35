"""Pins of the oracle's hybrid selection against what the pages fix.

English Dustin summary, Methodology 1: a fixed-size set I_verify; sinks and a local
window are always kept; then the top-m tokens by the draft signal; then the best
REMAINING tokens by the target signal.  Checked against brute force over all subsets,
hand-worked cases, planted one-hot scores and invariances.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def sel1(N, budget, s, w, m, draft, target, k_max=None):
    k_max = budget if k_max is None else k_max
    idx, cnt = O.select([N], None if draft is None else np.asarray([draft], float),
                        np.asarray([target], float), [budget], [s], [w], [m], k_max)
    return list(idx[0, :cnt[0]]), idx[0], int(cnt[0])


def brute(N, k, s, w, m, draft, target):
    """Exhaustive search: protected set first; then among all size-m' subsets of the
    unprotected tokens the one with the largest draft sum (ties: lexicographically
    smallest sorted position tuple); then the same over what remains with the target sum."""
    if k >= N:
        return list(range(N))
    s_ = min(s, k)
    w_ = min(w, k - s_)
    P = set(range(s_)) | set(range(N - w_, N))
    md = min(m, k - len(P))
    r = k - len(P) - md

    def best(cands, size, sc):
        top = None
        for c in itertools.combinations(sorted(cands), size):
            key = (-sum(sc[i] for i in c), c)
            if top is None or key < top:
                top = key
        return set(top[1]) if top else set()

    D = best(set(range(N)) - P, md, draft)
    T = best(set(range(N)) - P - D, r, target)
    return sorted(P | D | T)


def test_worked_examples():
    cases = json.load(open(os.path.join(GOLD, "select_worked.json")))["cases"]
    for c in cases:
        got, _, _ = sel1(c["ctx_len"], c["budget"], c["n_sink"], c["n_window"], c["m"],
                         c["draft"], c["target"], k_max=max(c["budget"], c["ctx_len"]))
        assert got == c["expect"], c["comment"]


@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_small(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 13))
    k = int(rng.integers(0, N + 3))
    s = int(rng.integers(0, 4))
    w = int(rng.integers(0, 4))
    m = int(rng.integers(0, 6))
    if seed % 2:   # integer scores: many exact ties exercise the tie rule
        draft = rng.integers(0, 4, N).astype(float)
        target = rng.integers(0, 4, N).astype(float)
    else:
        draft = rng.standard_normal(N)
        target = rng.standard_normal(N)
    got, row, cnt = sel1(N, k, s, w, m, draft, target, k_max=max(k, 1))
    assert got == brute(N, k, s, w, m, draft, target)
    assert cnt == min(k, N)
    assert all(x == -1 for x in row[cnt:])


def test_fixed_size_and_protected_always_kept():
    rng = np.random.default_rng(7)
    for _ in range(30):
        N = int(rng.integers(300, 700))
        k = int(rng.integers(50, 200))
        s, w, m = 4, 32, int(rng.integers(0, 80))
        got, _, cnt = sel1(N, k, s, w, m, rng.standard_normal(N), rng.standard_normal(N))
        assert cnt == k == len(got) == len(set(got))
        assert set(range(s)) <= set(got) and set(range(N - w, N)) <= set(got)
        assert got == sorted(got)


def test_planted_one_hot():
    N, k, s, w, m = 400, 40, 4, 8, 10
    draft = np.zeros(N)
    target = np.zeros(N)
    d_hot = [17, 33, 90, 120, 150, 200, 250, 300, 310, 350]
    t_hot = [20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 100, 101, 102, 103, 104, 105, 106, 107]
    draft[d_hot] = 1.0
    target[t_hot] = 1.0
    target[d_hot] = 5.0        # already taken by the draft tier
    got, _, _ = sel1(N, k, s, w, m, draft, target)
    r = k - s - w - m
    # the 18 target-hot tokens, then the lowest-index zero-score tokens fill the rest
    rest = [i for i in range(s, N - w) if i not in d_hot and i not in t_hot][: r - len(t_hot)]
    assert got == sorted(set(range(s)) | set(range(N - w, N)) | set(d_hot) | set(t_hot) | set(rest))


def test_budget_at_least_context_keeps_all():
    got, _, cnt = sel1(50, 64, 4, 8, 10, np.random.rand(50), np.random.rand(50))
    assert got == list(range(50)) and cnt == 50


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(3)
    N = 500
    d, t = rng.standard_normal(N), rng.standard_normal(N)
    a, _, _ = sel1(N, 100, 8, 16, 30, d, t)
    b, _, _ = sel1(N, 100, 8, 16, 30, d * 4.0, t * 0.125)
    assert a == b


def test_permutation_equivariance():
    rng = np.random.default_rng(5)
    N, s, w = 300, 4, 16
    d, t = rng.standard_normal(N), rng.standard_normal(N)
    a, _, _ = sel1(N, 60, s, w, 20, d, t)
    perm = np.arange(N)
    mid = perm[s:N - w].copy()
    rng.shuffle(mid)
    perm[s:N - w] = mid                       # permute the unprotected positions only
    dp, tp = np.empty(N), np.empty(N)
    dp[perm], tp[perm] = d, t                 # token i's scores move to position perm[i]
    b, _, _ = sel1(N, 60, s, w, 20, dp, tp)
    assert sorted(perm[a].tolist()) == b


def test_negative_zero_equals_zero():
    N = 20
    d = np.zeros(N)
    d[5] = -0.0
    d[3] = -0.0
    a, _, _ = sel1(N, 6, 1, 1, 2, d, np.zeros(N))
    assert a == [0, 1, 2, 3, 4, 19]      # all tie: lowest positions win


def test_ragged_batch():
    rng = np.random.default_rng(11)
    B, n_max, k_max = 5, 200, 64
    ctx = np.array([200, 10, 64, 63, 150])
    bud = np.array([64, 64, 64, 64, 20])
    sd = rng.standard_normal((B, n_max))
    st = rng.standard_normal((B, n_max))
    idx, cnt = O.select(ctx, sd, st, bud, [4] * B, [8] * B, [10] * B, k_max)
    for b in range(B):
        one, _, c1 = sel1(int(ctx[b]), int(bud[b]), 4, 8, 10, sd[b, :ctx[b]], st[b, :ctx[b]], k_max=k_max)
        assert list(idx[b, :cnt[b]]) == one and cnt[b] == c1 == min(ctx[b], bud[b])


def test_no_draft_signal_means_no_draft_tier():
    rng = np.random.default_rng(12)
    N, t = 100, rng.standard_normal(100)
    a, _, _ = sel1(N, 20, 2, 4, 7, None, t)
    b, _, _ = sel1(N, 20, 2, 4, 0, np.zeros(N), t)
    assert a == b
