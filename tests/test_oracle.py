"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked examples (tests/golden/hand_worked.json), textbook special cases,
exact rational arithmetic, closed forms, identities, brute force on tiny
inputs and hyperplane-LSH statistics.

Sources for what is pinned (HATA review on pith.science, arXiv 2506.02572):
  - h(x) = sign(x W_H), r = 128 ("Free parameters"); rbit/32 words per key
    (Algorithm 1 in the Figure 2 caption);
  - XOR + popcount Hamming scoring, top-k by Hamming distance, attention
    over the selected K/V ("What carries the argument"; Referee report);
  - binary-code inner product <-> Hamming equivalence (EcoFormer abstract on
    the Hugging Face listing page);
  - hyperplane LSH collision probability theta/pi (Charikar 2002, named in
    the angular-LSH abstract on the same listing page; HashEvict's binarised
    Gaussian projections).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))


def bf16(x):
    return synth.f64_to_bf16(np.asarray(x, dtype=np.float64))


def f32(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def u32list(hexes):
    return [int(h, 16) for h in hexes]


# ---------------------------------------------------------------- encode


def test_encode_identity_golden():
    g = GOLDEN["encode_identity"]
    x = np.array([g["x_pattern"][j % 3] for j in range(128)])
    codes = oracle.encode(bf16(x)[None], np.eye(128, dtype=np.float32))
    assert codes[0].tolist() == u32list(g["codes_identity"])
    codes = oracle.encode(bf16(x)[None], -np.eye(128, dtype=np.float32))
    assert codes[0].tolist() == u32list(g["codes_negated"])


def _bits(codes):
    """u32 [n][4] -> bool [n][128], bit j in word j//32 at position j%32."""
    n = codes.shape[0]
    out = np.zeros((n, 128), dtype=bool)
    for j in range(128):
        out[:, j] = (codes[:, j // 32] >> np.uint32(j % 32)) & np.uint32(1)
    return out


def test_encode_textbook_sign_and_permutation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 128))
    x[:, ::7] = 0.0  # exact zeros map to bit 0
    xb = bf16(x)
    xv = f32(xb)
    bits = _bits(oracle.encode(xb, np.eye(128, dtype=np.float32)))
    assert np.array_equal(bits, xv > 0)
    bits = _bits(oracle.encode(xb, -np.eye(128, dtype=np.float32)))
    assert np.array_equal(bits, xv < 0)
    perm = rng.permutation(128)
    P = np.zeros((128, 128), dtype=np.float32)
    P[perm, np.arange(128)] = 1.0  # column j picks coordinate perm[j]
    bits = _bits(oracle.encode(xb, P))
    assert np.array_equal(bits, xv[:, perm] > 0)
    # positive power-of-two scaling of W is exact and keeps every sign
    W = synth.normal_f32(3, 2, 0, 128 * 128, 1 / math.sqrt(128)).reshape(128, 128)
    assert np.array_equal(oracle.encode(xb, W), oracle.encode(xb, W * np.float32(4.0)))


def test_encode_matches_exact_rational_sign():
    # Exact arithmetic with Python fractions: an independent evaluation of
    # sign(sum_d x_d W_dj).
    rng = np.random.default_rng(2)
    n = 6
    xb = bf16(rng.standard_normal((n, 128)))
    W = (rng.standard_normal((128, 128)) / math.sqrt(128)).astype(np.float32)
    codes = oracle.encode(xb, W)
    bits = _bits(codes)
    xf = [[Fraction(float(v)) for v in row] for row in f32(xb)]
    Wf = [[Fraction(float(W[t, j])) for t in range(128)] for j in range(128)]
    for i in range(n):
        for j in range(128):
            y = sum(a * b for a, b in zip(xf[i], Wf[j]))
            assert bits[i, j] == (y > 0), (i, j)


def test_encode_exact_zero_sum_is_bit_zero():
    x = np.zeros(128)
    x[0], x[1] = 1.0, 1.0
    W = np.zeros((128, 128), dtype=np.float32)
    W[0, 5], W[1, 5] = 0.75, -0.75   # y_5 = 0 exactly
    W[0, 6], W[1, 6] = 0.75, -0.5    # y_6 = 0.25 > 0
    bits = _bits(oracle.encode(bf16(x)[None], W))[0]
    assert not bits[5] and bits[6] and bits.sum() == 1


def test_encode_simhash_collision_rate():
    # Hyperplane LSH: with W_H columns drawn i.i.d. Gaussian, each bit of
    # the two codes differs with probability theta / pi.
    rng = np.random.default_rng(3)
    a = rng.standard_normal(128)
    b_perp = rng.standard_normal(128)
    b_perp -= a * (a @ b_perp) / (a @ a)
    draws = 160
    for theta in (0.3, 1.2, 2.5):
        b = math.cos(theta) * a / np.linalg.norm(a) + math.sin(theta) * b_perp / np.linalg.norm(b_perp)
        xb = bf16(np.stack([a, b]))
        xv = f32(xb)
        th = math.acos(float(xv[0] @ xv[1] / np.linalg.norm(xv[0]) / np.linalg.norm(xv[1])))
        diff = 0
        for s in range(draws):
            W = synth.normal_f32(100 + s, synth.T_W, 0, 128 * 128, 1 / math.sqrt(128)).reshape(128, 128)
            c = oracle.encode(xb, W)
            diff += int(oracle.hamming(c[:1], c[1:])[0])
        rate = diff / (draws * 128)
        sd = math.sqrt(th / math.pi * (1 - th / math.pi) / (draws * 128))
        assert abs(rate - th / math.pi) < 5 * sd + 1e-3, (theta, rate, th / math.pi)


# ---------------------------------------------------------------- hamming


def test_hamming_golden():
    g = GOLDEN["hamming"]
    key = np.array([u32list(g["key"])], dtype=np.uint32)
    qs = np.array([u32list(q) for q in g["queries"]], dtype=np.uint32)
    for h in range(2):
        assert oracle.hamming(qs[h:h + 1], key)[0] == g["single"][h]
    assert oracle.hamming(qs, key)[0] == g["group_sum"]


def test_hamming_bruteforce_and_identity():
    rng = np.random.default_rng(4)
    for G in (1, 2, 4, 8):
        q = rng.integers(0, 2 ** 32, size=(G, 4), dtype=np.uint64).astype(np.uint32)
        k = rng.integers(0, 2 ** 32, size=(50, 4), dtype=np.uint64).astype(np.uint32)
        got = oracle.hamming(q, k)
        # brute force with Python integers: popcount of the XOR of 128-bit values
        def as_int(c):
            return sum(int(w) << (32 * i) for i, w in enumerate(c))
        ref = [sum(bin(as_int(q[h]) ^ as_int(kk)).count("1") for h in range(G)) for kk in k]
        assert got.tolist() == ref
        # inner product of +-1 codes: Ham = (r - <s_q, s_k>) / 2
        sq = 2 * _bits(q).astype(np.int64) - 1
        sk = 2 * _bits(k).astype(np.int64) - 1
        ident = ((128 - sk @ sq.T) // 2).sum(axis=1)
        assert got.tolist() == ident.tolist()
        assert got.min() >= 0 and got.max() <= G * 128


def test_hamming_extremes():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2 ** 32, size=(3, 4), dtype=np.uint64).astype(np.uint32)
    assert oracle.hamming(c[:1], c[:1])[0] == 0
    assert oracle.hamming(c[:1], ~c[:1])[0] == 128
    assert oracle.hamming(np.concatenate([c[:1], ~c[:1]]), c[1:]).tolist() == [128, 128]


# ---------------------------------------------------------------- select


def test_select_golden():
    g = GOLDEN["select"]
    assert oracle.select(np.array(g["scores"]), g["k"]).tolist() == g["idx"]


def test_select_bruteforce_tiny():
    rng = np.random.default_rng(6)
    for trial in range(200):
        n = int(rng.integers(0, 20))
        s = rng.integers(0, 5, size=n)
        k = int(rng.integers(-1, 25))
        ref = sorted(i for _, i in sorted((int(s[i]), i) for i in range(n))[:max(0, min(k, n))])
        assert oracle.select(s, k).tolist() == ref


def test_select_invariants():
    rng = np.random.default_rng(7)
    n = 20000
    s = rng.binomial(512, 0.5, size=n)
    for k in (1, 100, 313, 5000, n, n + 10):
        idx = oracle.select(s, k)
        k_eff = min(k, n)
        assert idx.size == k_eff and np.all(np.diff(idx) > 0)
        inside = np.zeros(n, dtype=bool)
        inside[idx] = True
        if k_eff < n:
            T = s[idx].max()
            assert T <= s[~inside].min()
            # within the cut bucket the lowest indices are taken
            tied = np.nonzero(s == T)[0]
            taken = tied[inside[tied]]
            assert np.array_equal(taken, tied[:taken.size])
    assert oracle.select(s, 0).size == 0


# ---------------------------------------------------------------- attention


def test_attention_two_key_closed_form():
    g = GOLDEN["attention_two_keys"]
    K = np.zeros((2, 128))
    K[0, 0] = 8.0
    V = np.zeros((2, 128))
    V[0, :2] = [1, 2]
    V[1, 0], V[1, 2] = -1, 4
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    out = oracle.attend(bf16(q), bf16(K), bf16(V), np.array([0, 1]))
    assert np.allclose(out[0, :3], g["out_head"], rtol=0, atol=1e-14)
    assert np.all(out[0, 3:] == 0)


def test_attention_full_selection_is_dense_sdpa():
    rng = np.random.default_rng(8)
    n, G = 300, 4
    q, K, V = bf16(rng.standard_normal((G, 128))), bf16(rng.standard_normal((n, 128))), bf16(
        rng.standard_normal((n, 128)))
    out = oracle.attend(q, K, V, np.arange(n))
    tq = torch.from_numpy(f32(q))[None, :, None, :]          # [1][G][1][d]
    tk = torch.from_numpy(f32(K))[None, None].expand(1, G, n, 128)
    tv = torch.from_numpy(f32(V))[None, None].expand(1, G, n, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_attention_single_key_and_uniform_logits():
    rng = np.random.default_rng(9)
    K, V = bf16(rng.standard_normal((10, 128))), bf16(rng.standard_normal((10, 128)))
    q = bf16(rng.standard_normal((2, 128)))
    out = oracle.attend(q, K, V, np.array([7]))
    assert np.array_equal(out, np.stack([f32(V[7])] * 2))
    zq = bf16(np.zeros((1, 128)))
    sel = np.array([1, 4, 8])
    out = oracle.attend(zq, K, V, sel)
    assert np.allclose(out[0], f32(V[sel]).mean(0), rtol=0, atol=1e-14)
    assert np.all(oracle.attend(q, K, V, np.array([], dtype=np.int64)) == 0)


# ---------------------------------------------------------------- end to end


def _unit(spec, b, kv, q, new, w):
    K, V = synth.unit_context(spec, b, kv, q, new)
    G = spec.G
    return K, V, oracle.decode_unit(q[b, kv * G:(kv + 1) * G], w[kv], K, V, spec.topk[b])


def test_planted_keys_selected_config1():
    spec = synth.config(1)
    q, new, w = synth.gen_q(spec), synth.gen_new_token(spec), synth.gen_w(spec)
    for kv in range(spec.Hkv):
        K, V, r = _unit(spec, 0, kv, q, new, w)
        pos = synth.planted_positions(spec, 0, kv)
        assert np.all(np.isin(pos, r["idx"])), kv
        assert r["idx"].size == 64
        # planted keys sit far below the random-key mean of r/2 = 64
        assert r["scores"][pos].max() < r["scores"].mean() - 3 * r["scores"].std()


def test_planted_keys_selected_gqa():
    spec = synth.custom("gqa", 1, 8, 2, [6000], [94], [6])
    q, new, w = synth.gen_q(spec), synth.gen_new_token(spec), synth.gen_w(spec)
    for kv in range(spec.Hkv):
        K, V, r = _unit(spec, 0, kv, q, new, w)
        pos = synth.planted_positions(spec, 0, kv)
        assert np.all(np.isin(pos, r["idx"]))
        # the output leans on the planted values: compare with dense attention
        dense = oracle.attend(q[0, kv * 4:(kv + 1) * 4], K, V, np.arange(K.shape[0]))
        assert np.abs(r["out"] - dense).max() < 0.25


@pytest.mark.parametrize("threads", [1, 3])
def test_threaded_ranges_match(threads):
    spec = synth.custom("thr", 1, 2, 1, [5000], [50], [3])
    q, new, w = synth.gen_q(spec), synth.gen_new_token(spec), synth.gen_w(spec)
    K, V = synth.unit_context(spec, 0, 0, q, new)
    a = oracle.encode(K, w[0], threads=threads)
    b = oracle.encode(K, w[0], threads=1)
    assert np.array_equal(a, b)
