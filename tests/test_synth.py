"""The shared input generator: published SplitMix64 outputs, counter-based
slicing, Box-Muller statistics, bf16 rounding and workload shapes."""
import math

import numpy as np

import synth


def test_splitmix64_published_vector():
    # First outputs of SplitMix64 seeded with 1234567, as published with the
    # reference implementation of the generator (Vigna, splitmix64.c).
    got = synth.sm64_stream(1234567, 5).tolist()
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_counter_based_slices_agree():
    full = synth.normal_f64(0, synth.T_K, 0, 4097)
    for a, n in [(0, 1), (1, 1), (5, 100), (4000, 97), (3, 4094)]:
        part = synth.normal_f64(0, synth.T_K, a, n)
        assert np.array_equal(full[a:a + n], part)
    u = synth.u64(7, 3, 0, 100)
    assert np.array_equal(u[40:60], synth.u64(7, 3, 40, 20))
    assert not np.array_equal(u, synth.u64(8, 3, 0, 100))


def test_normal_moments():
    z = synth.normal_f64(0, synth.T_V, 0, 1 << 20)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    assert abs((z ** 4).mean() - 3) < 0.05


def test_bf16_round_to_nearest_even():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2 ** -8, 0x3F80),            # halfway, even mantissa stays
        (1.0 + 3 * 2 ** -8, 0x3F82),        # halfway, odd mantissa rounds up
        (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),  # above halfway
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.0e38, 0x7F62),
    ]
    xs = np.array([c[0] for c in cases], dtype=np.float64)
    got = synth.f64_to_bf16(xs)
    assert [int(g) for g in got] == [c[1] for c in cases]
    back = synth.bf16_to_f32(got)
    assert back[0] == 1.0 and back[4] == -2.5


def test_config_shapes():
    c1 = synth.config(1)
    assert (c1.B, c1.Hq, c1.Hkv, c1.lengths, c1.topk, c1.planted) == (1, 8, 8, (4096,), (64,), (16,))
    c3 = synth.config(3)
    assert c3.G == 4 and c3.topk == (2048,) * 4 and c3.planted == (131,) * 4
    assert synth.config(4).planted == (524,)
    c5 = synth.config(5)
    assert c5.B == 64 and all(1024 <= n <= 65536 for n in c5.lengths)
    assert all(k == max(16, n // 64) for k, n in zip(c5.topk, c5.lengths))
    assert c5.stride == 65536


def test_planted_rows():
    spec = synth.custom("t", 1, 4, 1, [300], [8], [5])
    q = synth.gen_q(spec)
    pos = synth.planted_positions(spec, 0, 0)
    assert pos.size == 5 and len(set(pos.tolist())) == 5 and pos.max() < 299
    k = synth.gen_unit_k(spec, 0, 0, q)
    plain = synth.normal_bf16(0, synth.T_K, 0, 299 * 128).reshape(299, 128)
    other = np.setdiff1d(np.arange(299), pos)
    assert np.array_equal(k[other], plain[other])
    s = synth.bf16_to_f32(q[0]).astype(np.float64).sum(0) / 2.0
    for p in pos:
        resid = synth.bf16_to_f32(k[p]).astype(np.float64) - 3 * s
        assert abs(resid.std() - 1) < 0.3  # N(0, 1) noise plus bf16 rounding
