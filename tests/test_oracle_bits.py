"""Pins of the CPU oracle at every supported code length r in {32, 64, 128, 256}.

The hash-length ablation of the HATA review ("Assumptions & free
parameters": accuracy from 32 to 128 bits, r = 128 kept) makes r a
parameter: W_H is d x r, a code is r/32 words, the summed Hamming score of
a group of G heads ranges over 0 .. G r.  The pins below hold the oracle's
r-dependent arithmetic (the W_H stride, the word count, the bit position
within a word, the score range, the tie bucket at the cut) to facts that do
not come from the oracle: hand-worked codes and scores
(tests/golden/hand_worked.json), textbook signs of identity, permutation,
negated and duplicated columns, exact rational arithmetic, brute force with
Python integers, the binary-code inner-product identity (EcoFormer abstract
on the Hugging Face listing page) and hyperplane-LSH statistics (Charikar's
theta / pi, named on the same page).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))
LENGTHS = [32, 64, 128, 256]


def bf16(x):
    return synth.f64_to_bf16(np.asarray(x, dtype=np.float64))


def f64(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def u32list(hexes):
    return [int(h, 16) for h in hexes]


def bits_of(codes, r):
    """u32 [n][r/32] -> bool [n][r]: bit j from word j // 32, position j % 32."""
    codes = np.asarray(codes, dtype=np.uint32)
    out = np.zeros((codes.shape[0], r), dtype=bool)
    for j in range(r):
        out[:, j] = (codes[:, j // 32] >> np.uint32(j % 32)) & np.uint32(1)
    return out


def as_int(words):
    """A code as one Python integer: word i holds bits 32 i .. 32 i + 31."""
    return sum(int(w) << (32 * i) for i, w in enumerate(words))


def selection_columns(cols, r):
    """W [128][r] whose column j is sign_j * e_{idx_j} (cols: list of (idx, sign))."""
    W = np.zeros((128, r), dtype=np.float32)
    for j, (t, s) in enumerate(cols):
        W[t, j] = s
    return W


# ---------------------------------------------------------------- encode


@pytest.mark.parametrize("r", [32, 64, 256])
def test_encode_code_length_golden(r):
    g = GOLDEN["encode_code_lengths"]
    x = np.array([g["x_pattern"][j % 3] for j in range(128)])
    if r <= 128:
        W = selection_columns([(j, 1.0) for j in range(r)], r)
    else:
        W = selection_columns([(j, 1.0) for j in range(128)] + [(j, -1.0) for j in range(128)], r)
    codes = oracle.encode(bf16(x)[None], W)
    assert codes.shape == (1, r // 32)
    assert codes[0].tolist() == u32list(g["codes"][str(r)])


@pytest.mark.parametrize("r", LENGTHS)
def test_encode_permuted_negated_duplicated_columns(r):
    # Column j of W picks +-x_{t_j}: bit j must be the textbook sign of that
    # coordinate, wherever j sits in the code (word j // 32, bit j % 32).
    rng = np.random.default_rng(100 + r)
    x = rng.standard_normal((30, 128))
    x[:, 5::11] = 0.0  # exact zeros give bit 0 under both signs
    xb = bf16(x)
    xv = f64(xb)
    t = rng.integers(0, 128, size=r)
    s = np.where(rng.random(r) < 0.5, -1.0, 1.0)
    if r == 256:
        # the second half repeats the first half's columns, negated at odd j
        t[128:] = t[:128]
        s[128:] = np.where(np.arange(128) % 2 == 1, -s[:128], s[:128])
    W = selection_columns(list(zip(t, s)), r)
    got = bits_of(oracle.encode(xb, W), r)
    want = (xv[:, t] * s) > 0
    assert np.array_equal(got, want)
    if r == 256:
        even = np.arange(0, 128, 2)
        odd = np.arange(1, 128, 2)
        assert np.array_equal(got[:, 128 + even], got[:, even])
        nz = xv[:, t[odd]] != 0
        assert np.array_equal(got[:, 128 + odd][nz], ~got[:, odd][nz])


@pytest.mark.parametrize("r", LENGTHS)
def test_encode_matches_exact_rational_sign(r):
    # An independent evaluation of sign(sum_t x_t W_tj) in exact rational
    # arithmetic (Python fractions) for every bit of every code length.
    rng = np.random.default_rng(200 + r)
    n = 3
    xb = bf16(rng.standard_normal((n, 128)))
    W = (rng.standard_normal((128, r)) / math.sqrt(128)).astype(np.float32)
    bits = bits_of(oracle.encode(xb, W), r)
    xf = [[Fraction(float(v)) for v in row] for row in f64(xb)]
    Wf = [[Fraction(float(W[t, j])) for t in range(128)] for j in range(r)]
    for i in range(n):
        for j in range(r):
            y = sum(a * b for a, b in zip(xf[i], Wf[j]))
            assert bits[i, j] == (y > 0), (r, i, j)


@pytest.mark.parametrize("r", LENGTHS)
def test_encode_cancellation_and_summation_order(r):
    # x = (2^60, 1, -2^60, 1, 0, ...).  Bits decided by exact cancellation and
    # by the sequential double sum in ascending d (the code convention):
    #   column 0: x0 + x2 = 0 exactly -> bit 0;
    #   column 1: (2^60 + 1) rounds to 2^60, minus 2^60 gives 0 -> bit 0,
    #             although the real sum is 1;
    #   column 2: 2^60 - 2^60 = 0, then + 1 -> bit 1 (summed in descending d
    #             it would be (1 - 2^60) -> -2^60, + 2^60 = 0 -> bit 0);
    #   column r-1 (the code's highest bit): x1 = 1 -> bit 1;
    #   column r-2: 2^60 * 2^-80 - 1 < 0 -> bit 0;
    #   column r-3: x1 - x3 = 0 -> bit 0.
    x = np.zeros(128)
    x[0], x[1], x[2], x[3] = 2.0 ** 60, 1.0, -(2.0 ** 60), 1.0
    W = np.zeros((128, r), dtype=np.float32)
    W[[0, 2], 0] = 1.0
    W[[0, 1, 2], 1] = 1.0
    W[[0, 2, 3], 2] = 1.0
    W[1, r - 1] = 1.0
    W[0, r - 2], W[1, r - 2] = 2.0 ** -80, -1.0
    W[1, r - 3], W[3, r - 3] = 1.0, -1.0
    bits = bits_of(oracle.encode(bf16(x)[None], W), r)[0]
    assert np.nonzero(bits)[0].tolist() == [2, r - 1]


@pytest.mark.parametrize("r", [32, 256])
def test_encode_simhash_collision_rate(r):
    # Hyperplane LSH at other code lengths: each of the r bits of two codes
    # differs with probability theta / pi under Gaussian W_H columns.
    rng = np.random.default_rng(300 + r)
    a = rng.standard_normal(128)
    b_perp = rng.standard_normal(128)
    b_perp -= a * (a @ b_perp) / (a @ a)
    draws = 40 * 128 // r + 20
    for theta in (0.4, 1.5, 2.7):
        b = math.cos(theta) * a / np.linalg.norm(a) + math.sin(theta) * b_perp / np.linalg.norm(b_perp)
        xb = bf16(np.stack([a, b]))
        xv = f64(xb)
        th = math.acos(float(xv[0] @ xv[1] / np.linalg.norm(xv[0]) / np.linalg.norm(xv[1])))
        diff = 0
        for s in range(draws):
            W = synth.normal_f32(700 + s, synth.T_W, 0, 128 * r, 1 / math.sqrt(128)).reshape(128, r)
            c = oracle.encode(xb, W)
            diff += int(oracle.hamming(c[:1], c[1:])[0])
        rate = diff / (draws * r)
        sd = math.sqrt(th / math.pi * (1 - th / math.pi) / (draws * r))
        assert abs(rate - th / math.pi) < 5 * sd + 1e-3, (r, theta, rate, th / math.pi)


# ---------------------------------------------------------------- hamming


@pytest.mark.parametrize("r", LENGTHS)
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_hamming_bruteforce_and_identity(r, G):
    rng = np.random.default_rng(400 + r + G)
    words = r // 32
    q = rng.integers(0, 2 ** 32, size=(G, words), dtype=np.uint64).astype(np.uint32)
    k = rng.integers(0, 2 ** 32, size=(40, words), dtype=np.uint64).astype(np.uint32)
    k[0] = q[0]          # distance 0 to head 0
    k[1] = ~q[0]         # distance r to head 0
    got = oracle.hamming(q, k)
    # brute force with Python integers: popcount of the XOR of r-bit values
    ref = [sum(bin(as_int(q[h]) ^ as_int(kk)).count("1") for h in range(G)) for kk in k]
    assert got.tolist() == ref
    # binary-code inner product: Ham = (r - <s_q, s_k>) / 2 with s = 2b - 1
    sq = 2 * bits_of(q, r).astype(np.int64) - 1
    sk = 2 * bits_of(k, r).astype(np.int64) - 1
    ident = ((r - sk @ sq.T) // 2).sum(axis=1)
    assert got.tolist() == ident.tolist()
    assert got.min() >= 0 and got.max() <= G * r
    single = oracle.hamming(q[:1], k[:2])
    assert single.tolist() == [0, r]


def test_hamming_and_cut_golden_g8_r256():
    g = GOLDEN["hamming_g8_r256"]
    keys = np.array([u32list(k) for k in g["keys"]], dtype=np.uint32)
    zero_q = np.zeros((8, 8), dtype=np.uint32)
    bit_q = np.zeros((8, 8), dtype=np.uint32)
    for h in range(8):
        bit_q[h, 0] = np.uint32(1 << h)
    s0 = oracle.hamming(zero_q, keys)
    assert s0.tolist() == g["scores_zero_queries"]
    assert oracle.hamming(bit_q, keys).tolist() == g["scores_bit_h_queries"]
    for k, want in g["tie_bucket_zero_queries"].items():
        assert list(oracle.tie_bucket(s0, int(k))) == want, k
    for k, want in g["select_zero_queries"].items():
        assert oracle.select(s0, int(k)).tolist() == want, k


# ---------------------------------------------------------------- select / cut


@pytest.mark.parametrize("r", LENGTHS)
def test_select_and_cut_bruteforce_score_range(r):
    # Scores over the whole range 0 .. G r of a group of G = 8 heads (up to
    # 2049 distinct values at 256 bits), against a brute-force sort.
    rng = np.random.default_rng(500 + r)
    top = 8 * r
    for trial in range(60):
        n = int(rng.integers(0, 40))
        s = rng.integers(0, top + 1, size=n)
        if n:
            s[rng.integers(0, n, size=n // 3)] = rng.choice([0, top, top // 2])
        k = int(rng.integers(-1, 45))
        order = sorted((int(s[i]), i) for i in range(n))
        ke = max(0, min(k, n))
        assert oracle.select(s, k).tolist() == sorted(i for _, i in order[:ke])
        if ke == 0:
            assert oracle.tie_bucket(s, k) == (-1, 0, 0, 0)
        else:
            T = order[ke - 1][0]
            want = (T, int((s < T).sum()), int((s == T).sum()), ke)
            assert oracle.tie_bucket(s, k) == want


# ---------------------------------------------------------------- end to end


@pytest.mark.parametrize("r", [64, 256])
def test_planted_keys_selected_other_lengths(r):
    # The planted keys (3 x the group's query direction plus noise) sit far
    # below the random keys' mean distance G r / 2 at these code lengths too.
    spec = synth.custom("bits planted", 1, 8, 2, [6000], [94], [6])
    q, new = synth.gen_q(spec), synth.gen_new_token(spec)
    w = synth.gen_w_bits(spec, r)
    G = spec.G
    for kv in range(spec.Hkv):
        K, V = synth.unit_context(spec, 0, kv, q, new)
        res = oracle.decode_unit(q[0, kv * G:(kv + 1) * G], w[kv], K, V, spec.topk[0])
        assert res["qcodes"].shape == (G, r // 32) and res["kcodes"].shape == (6000, r // 32)
        pos = synth.planted_positions(spec, 0, kv)
        assert np.all(np.isin(pos, res["idx"])), (r, kv)
        sc = res["scores"]
        assert sc.max() <= G * r
        assert abs(sc.mean() - G * r / 2) < 0.02 * G * r
