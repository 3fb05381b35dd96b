"""Pins of the oracle's recall analysis (exact top-k, overlap, tie bucket).

The exact top-k follows the review's test of the method (rank keys by
their exact q.k, compare with the Hamming selection); it is pinned here by
brute force in exact integer arithmetic, by a hand-derived case of the
sequential double sum's rounding, and by order invariants; the tie bucket
and the overlap by hand-worked examples.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

ONE, ZERO = 0x3F80, 0x0000
P60, M60 = 0x5D80, 0xDD80  # bf16 bit patterns of 2^60 and -2^60


def bf16_of_small_ints(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of small integers (|a| <= 256 are exact in bf16)."""
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_topk_brute_force_integers(seed):
    # Integer entries: every sum is exact, so z is the integer dot product;
    # the values are small, so ties are frequent and the tie-break shows.
    rng = np.random.default_rng(seed)
    n, d = 60, 128
    qi = rng.integers(-3, 4, size=d)
    Ki = rng.integers(-2, 3, size=(n, d))
    q, K = bf16_of_small_ints(qi), bf16_of_small_ints(Ki)
    z = [int(sum(int(a) * int(b) for a, b in zip(qi, Ki[i]))) for i in range(n)]
    order = sorted(range(n), key=lambda i: (-z[i], i))
    for k in (0, 1, 5, 17, 59, 60, 75, -3):
        want = sorted(order[:max(0, min(k, n))])
        got = oracle.exact_topk(q, K, k)
        assert got.tolist() == want, (k, got, want)


def test_exact_topk_sequential_double_rounding():
    # q = all ones.  Keys 0, 1, 2 have the same real sum 1, but the
    # sequential double sum gives key 0 (2^60, then +1, then -2^60) the value
    # 0, since 2^60 + 1 rounds to 2^60; key 1 (2^60 - 2^60 + 1) and key 2
    # (just 1) give 1.  Key 3 is all zero: z = 0, tied with key 0.
    d = 128
    q = np.full(d, ONE, dtype=np.uint16)
    K = np.zeros((4, d), dtype=np.uint16)
    K[0, :3] = [P60, ONE, M60]
    K[1, :3] = [P60, M60, ONE]
    K[2, 0] = ONE
    assert oracle.exact_topk(q, K, 1).tolist() == [1]
    assert oracle.exact_topk(q, K, 2).tolist() == [1, 2]
    assert oracle.exact_topk(q, K, 3).tolist() == [0, 1, 2]  # 0 beats 3 on the index
    assert oracle.exact_topk(q, K, 4).tolist() == [0, 1, 2, 3]


def test_exact_topk_order_invariants_gaussian():
    rng = np.random.default_rng(7)
    n, d, k = 3000, 128, 47
    qf = rng.standard_normal(d).astype(np.float32)
    Kf = rng.standard_normal((n, d)).astype(np.float32)
    q = (qf.view(np.uint32) >> 16).astype(np.uint16)
    K = (Kf.view(np.uint32) >> 16).astype(np.uint16)
    e = oracle.exact_topk(q, K, k)
    assert e.size == k and np.all(np.diff(e) > 0)
    qv = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Kv = (K.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = Kv @ qv
    inside = np.zeros(n, bool)
    inside[e] = True
    # A different summation order moves z by ~1e-13 at most.
    assert z[inside].min() >= z[~inside].max() - 1e-9
    # A copy of the last key in, appended at a higher index, ties with it
    # exactly and loses on the index: the set is unchanged.  Moved to the
    # front (index 0 shifts everything by one), it wins and pushes that key out.
    last = e[np.argmin(z[e])]
    K2 = np.concatenate([K, K[last:last + 1]])
    assert oracle.exact_topk(q, K2, k).tolist() == e.tolist()
    K3 = np.concatenate([K[last:last + 1], K])
    want = sorted([0] + [int(i) + 1 for i in e if i != last])
    assert oracle.exact_topk(q, K3, k).tolist() == want


def test_overlap_hand_examples():
    assert oracle.overlap(np.array([1, 4, 9, 12]), np.array([0, 4, 9, 13])) == 2
    assert oracle.overlap(np.array([], dtype=np.int64), np.array([3])) == 0
    assert oracle.overlap(np.arange(10), np.arange(10)) == 10


def test_tie_bucket_hand_examples():
    s = np.array([5, 3, 3, 7, 3, 1])
    # sorted: 1 3 3 3 5 7
    assert oracle.tie_bucket(s, 3) == (3, 1, 3, 3)
    assert oracle.tie_bucket(s, 2) == (3, 1, 3, 2)
    assert oracle.tie_bucket(s, 1) == (1, 0, 1, 1)
    assert oracle.tie_bucket(s, 5) == (5, 4, 1, 5)
    assert oracle.tie_bucket(s, 10) == (7, 5, 1, 6)
    assert oracle.tie_bucket(s, 0) == (-1, 0, 0, 0)
    assert oracle.tie_bucket(np.array([], dtype=np.int32), 4) == (-1, 0, 0, 0)


def test_tie_bucket_matches_selection():
    # The cut of the oracle's own Hamming selection: every selected score is
    # <= T, every key under T is selected, and k_eff - below keys at T are.
    rng = np.random.default_rng(3)
    s = rng.integers(200, 260, size=5000).astype(np.int32)
    for k in (1, 77, 1000, 4999, 5000):
        T, below, at, ke = oracle.tie_bucket(s, k)
        sel = oracle.select(s, k)
        assert ke == sel.size
        assert s[sel].max() == T
        assert int((s[sel] < T).sum()) == below
        assert 0 < ke - below <= at


def test_recall_unit_perfect_when_selection_is_exact():
    rng = np.random.default_rng(11)
    n, d, G, k = 400, 128, 2, 20
    q = (rng.standard_normal((G, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    K = (rng.standard_normal((n, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    e0 = oracle.exact_topk(q[0], K, k)
    r = oracle.recall_unit(q, K, k, e0, np.zeros(n, np.int32))
    assert r["overlap"][0] == k
    assert r["exact"][0].tolist() == e0.tolist()
    assert 0 <= r["overlap"][1] <= k
    assert r["tie"] == (0, 0, n, k)
