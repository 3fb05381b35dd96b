"""Pins of the oracle of the learning-to-hash objective (the training of W_H;
HATA review, "What carries the argument" and "Assumptions & free
parameters"; labels as its circularity check restates Section 3.1.2).

What pins each part, independently of the oracle's own formulas:
  - labels: brute force in exact integer arithmetic with ties (pure Python
    ranking), hand-worked counts and values (m = ceil(n_k / 10) positives,
    20 - 19 t / (m - 1));
  - loss: closed forms -- W = 0 (every code 0: L = lambda r, gradient 0);
    saturated codes equal to the rows of a Sylvester-Hadamard matrix (hand
    values of all three terms); saturated random codes, where the relaxed
    distance must equal the Hamming distance of the sign codes computed by the
    (separately pinned) encoder and XOR/popcount scorer; a batch closed under
    negation has zero bit balance;
  - gradient: central finite differences of the double-precision loss;
  - Adam: the first and second steps in closed form.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

SIG, EPS, ETA, LAM = 0.1, 0.01, 2.0, 1.0


def bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def ints_bf16(a):
    return bf16(np.asarray(a, dtype=np.float32))  # small integers are exact in bf16


# ---------------------------------------------------------------- labels


@pytest.mark.parametrize("seed,nq,nk", [(0, 5, 23), (1, 3, 10), (2, 4, 37), (3, 2, 1)])
def test_labels_brute_force_integers(seed, nq, nk):
    rng = np.random.default_rng(seed)
    qi = rng.integers(-2, 3, size=(nq, 128))
    ki = rng.integers(-1, 2, size=(nk, 128))
    ki[nk // 2:] = ki[:nk - nk // 2]  # duplicated keys: exact ties
    got = oracle.hash_labels(ints_bf16(qi), ints_bf16(ki))
    m = -(-nk // 10)
    for j in range(nq):
        z = [sum(int(a) * int(b) for a, b in zip(qi[j], ki[i])) for i in range(nk)]
        order = sorted(range(nk), key=lambda i: (-z[i], i))
        want = [-1.0] * nk
        for t in range(m):
            want[order[t]] = 20.0 if m == 1 else 20.0 - 19.0 * t / (m - 1)
        assert got[j].tolist() == [float(np.float32(v)) for v in want], j


def test_labels_hand_counts():
    # 10 keys: one positive (label 20); 20 keys: two (20 and 1); 21 keys:
    # three (20, 10.5, 1), on keys whose q.k is simply their index.
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    for nk, want in ((10, [20.0]), (20, [20.0, 1.0]), (21, [20.0, 10.5, 1.0])):
        k = np.zeros((nk, 128))
        k[:, 0] = np.arange(nk)
        lab = oracle.hash_labels(bf16(q), bf16(k))[0]
        top = [float(lab[nk - 1 - t]) for t in range(len(want))]
        assert top == want
        assert np.all(lab[:nk - len(want)] == -1.0)


# ---------------------------------------------------------------- loss


def test_zero_weights():
    # W = 0: every relaxed code is 0, so L_sim = L_bal = 0, C = 0 and
    # L_unc = |-I|^2 = r; every term's gradient carries a factor of a code.
    rng = np.random.default_rng(5)
    q, k = bf16(rng.standard_normal((6, 128))), bf16(rng.standard_normal((30, 128)))
    lab = oracle.hash_labels(q, k)
    for r in (32, 128):
        loss, grad = oracle.hash_loss_grad(q, k, np.zeros((128, r), np.float32), lab)
        assert loss.tolist() == [LAM * r, 0.0, 0.0, float(r)]
        assert np.all(grad == 0.0)


def _sylvester(n):
    H = np.array([[1]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("n,nq", [(32, 8), (64, 16)])
def test_saturated_hadamard_codes(n, nq):
    # Vector v is the unit vector e_v and W = 2^20 Had, so y_vc = 2^20 Had[v][c]
    # and the sigmoid saturates: every code is exactly row v of the
    # Sylvester-Hadamard matrix Had (n x n, r = n).  Then
    #   C = Had^T Had / n = I, so L_unc = 0;
    #   column 0 is all +1 and every other column sums to 0: L_bal = 1;
    #   two distinct rows differ in exactly n / 2 places, so D = n / 2 for
    #   every (query, key) pair and L_sim = (n / 2) (sum of labels) / n_q.
    Had = _sylvester(n)
    X = np.zeros((n, 128))
    X[np.arange(n), np.arange(n)] = 1.0
    W = np.zeros((128, n), np.float32)
    W[:n, :] = Had * 2.0 ** 20
    q, k = bf16(X[:nq]), bf16(X[nq:])
    rng = np.random.default_rng(n)
    lab = rng.choice(np.array([-1.0, 1.0, 7.5, 20.0], np.float32), size=(nq, n - nq))
    loss, grad = oracle.hash_loss_grad(q, k, W, lab)
    l_sim = (n / 2) * float(lab.astype(np.float64).sum()) / nq
    assert loss[1] == l_sim
    assert loss[2] == 1.0
    assert loss[3] == 0.0
    assert loss[0] == EPS * l_sim + ETA * 1.0
    assert np.all(grad == 0.0)  # the slope of a saturated sigmoid is 0 in double


@pytest.mark.parametrize("r", [32, 64, 256])
def test_saturated_codes_give_hamming_distances(r):
    # With W scaled by 2^40 every |sigma y| is far past the sigmoid's range
    # (no y is 0 for these Gaussian inputs), so each relaxed code is the +-1
    # form of sign(x W): the relaxed distance D must be the Hamming distance
    # of the sign codes from the oracle's encoder and XOR/popcount scorer.
    rng = np.random.default_rng(r)
    nq, nk = 3, 17
    q, k = bf16(rng.standard_normal((nq, 128))), bf16(rng.standard_normal((nk, 128)))
    W = (rng.standard_normal((128, r)) / math.sqrt(128)).astype(np.float32)
    for j in range(nq):
        lab = np.zeros((nq, nk), np.float32)
        lab[j] = 1.0  # L_sim = (1 / n_q) sum_i D(a_j, b_i)
        loss, _ = oracle.hash_loss_grad(q, k, W * np.float32(2.0 ** 40), lab)
        ham = oracle.hamming(oracle.encode(q[j:j + 1], W), oracle.encode(k, W))
        assert loss[1] * nq == float(ham.sum())


def test_balance_zero_for_a_batch_closed_under_negation():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((10, 128))
    q = bf16(np.concatenate([x[:3], -x[:3]]))
    k = bf16(np.concatenate([x[3:], -x[3:]]))
    W = (rng.standard_normal((128, 64)) / math.sqrt(128)).astype(np.float32)
    loss, _ = oracle.hash_loss_grad(q, k, W, oracle.hash_labels(q, k))
    assert loss[2] < 1e-28


# ---------------------------------------------------------------- gradient


@pytest.mark.parametrize("r", [32, 128])
def test_gradient_matches_central_differences(r):
    # W on a grid of 2^-12, so W +- 2^-12 is exact in fp32; the loss is
    # smooth, and the central difference's error is O(h^2).
    rng = np.random.default_rng(11 + r)
    nq, nk = 12, 50
    q, k = bf16(rng.standard_normal((nq, 128))), bf16(rng.standard_normal((nk, 128)))
    lab = oracle.hash_labels(q, k)
    W = np.round(rng.standard_normal((128, r)) * 0.3 * 4096) / 4096
    W = W.astype(np.float32)
    _, grad = oracle.hash_loss_grad(q, k, W, lab)
    h = 2.0 ** -12
    coords = [(int(rng.integers(0, 128)), int(rng.integers(0, r))) for _ in range(12)]
    for (t, c) in coords:
        Wp, Wm = W.copy(), W.copy()
        Wp[t, c] += np.float32(h)
        Wm[t, c] -= np.float32(h)
        assert float(Wp[t, c]) - float(W[t, c]) == h and float(W[t, c]) - float(Wm[t, c]) == h
        lp, _ = oracle.hash_loss_grad(q, k, Wp, lab)
        lm, _ = oracle.hash_loss_grad(q, k, Wm, lab)
        fd = (lp[0] - lm[0]) / (2 * h)
        assert abs(fd - grad[t, c]) <= 1e-6 * max(1.0, abs(grad).max()), (t, c, fd, grad[t, c])
    # every term contributes: a gradient check with one weight at a time
    for eps, eta, lam in ((1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0)):
        _, g1 = oracle.hash_loss_grad(q, k, W, lab, epsilon=eps, eta=eta, lam=lam)
        t, c = coords[0]
        Wp, Wm = W.copy(), W.copy()
        Wp[t, c] += np.float32(h)
        Wm[t, c] -= np.float32(h)
        lp, _ = oracle.hash_loss_grad(q, k, Wp, lab, epsilon=eps, eta=eta, lam=lam)
        lm, _ = oracle.hash_loss_grad(q, k, Wm, lab, epsilon=eps, eta=eta, lam=lam)
        fd = (lp[0] - lm[0]) / (2 * h)
        assert abs(fd - g1[t, c]) <= 1e-6 * max(1e-3, abs(g1).max()), (eps, eta, lam)
        assert abs(g1).max() > 0


# ---------------------------------------------------------------- Adam


def test_adam_first_and_second_step():
    # From m = v = 0: m1 = 0.1 g, v1 = 0.001 g^2, bias-corrected to g and
    # g^2, so w1 = w0 - lr g / (|g| + e).  A second step with the same g has
    # the same corrected moments: w2 = w1 - lr g / (|g| + e).
    g = np.array([0.5, -2.0, 1e-3, 0.0])
    w0 = np.array([1.0, 1.0, 1.0, 1.0])
    lr, e = 0.01, 1e-8
    w1, m1, v1 = oracle.adam(w0, np.zeros(4), np.zeros(4), g, 1, lr)
    assert np.allclose(m1, 0.1 * g, rtol=1e-14, atol=0)
    assert np.allclose(v1, 0.001 * g * g, rtol=1e-14, atol=0)
    assert np.allclose(w1, w0 - lr * g / (np.abs(g) + e), rtol=0, atol=1e-15)
    w2, _, _ = oracle.adam(w1, m1, v1, g, 2, lr)
    assert np.allclose(w2, w1 - lr * g / (np.abs(g) + e), rtol=0, atol=1e-15)
