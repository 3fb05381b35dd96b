"""GPU parity of the recall analysis (hata_exact_topk_recall) against the oracle.

Bars, all bit-exact: each query head's exact top-k index set, the overlap
count with the Hamming selection, and the tie bucket (T, below, at, k_eff) of
each group.  The oracle side computes its own selection and scores
(oracle.decode_unit), its own exact top-k (sequential double logits, full
sort) and the counts from those; nothing expected comes from the GPU.
Small workloads are checked head by head in full; the headline configuration
on sampled units, with structural properties on every head.  Two hand-built
caches drive the exact-ranking paths: keys whose logits tie or differ only
by the double sum's rounding order, and a query and keys large enough that
every key is ranked exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import hash_top_sparse_encode_amd as hata
import oracle
import synth
from workload import GpuWorkload, bf16_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_recall(cache, q, topk, k_max, sel, sc):
    ws = hata.alloc_recall_workspace(cache)
    B, Hq = cache.batch, cache.n_q_heads
    ex = torch.full((B, Hq, max(k_max, 1)), -7, dtype=torch.int32, device=cache.codes.device)
    ex = ex[:, :, :k_max].contiguous()
    ov, tie = hata.hata_exact_topk_recall(cache, q, topk, k_max, sel, sc, ws, exact_idx_out=ex)
    torch.cuda.synchronize()
    return ov.cpu().numpy(), tie.cpu().numpy(), ex.cpu().numpy()


def check_unit(spec, wl, b, kv, ov, tie, ex):
    G = spec.G
    K, V = synth.unit_context(spec, b, kv, wl.q_host, wl.new_host)
    ref = oracle.decode_unit(wl.q_host[b, kv * G:(kv + 1) * G], wl.w_host[kv], K, V,
                             spec.topk[b], threads=16)
    k = min(spec.topk[b], wl.k_max)
    for h in range(G):
        e = oracle.exact_topk(wl.q_host[b, kv * G + h], K, k)
        ke = e.size
        hq = kv * G + h
        assert np.array_equal(ex[b, hq, :ke], e), f"exact set differs at {(b, hq)}"
        assert np.all(ex[b, hq, ke:] == -1)
        assert ov[b, hq] == oracle.overlap(ref["idx"], e), (b, hq, ov[b, hq])
    assert tuple(int(x) for x in tie[b, kv]) == oracle.tie_bucket(ref["scores"], k), (b, kv)


def check_structure(spec, wl, ov, tie, ex):
    for b in range(spec.B):
        ke = max(0, min(spec.topk[b], wl.k_max, spec.lengths[b]))
        for hq in range(spec.Hq):
            row = ex[b, hq]
            assert np.all(row[ke:] == -1)
            assert np.all(np.diff(row[:ke]) > 0)
            assert ke == 0 or (row[0] >= 0 and row[ke - 1] < spec.lengths[b])
            assert 0 <= ov[b, hq] <= ke
        for kv in range(spec.Hkv):
            T, below, at, k_eff = (int(x) for x in tie[b, kv])
            assert k_eff == ke
            if ke == 0:
                assert (T, below, at) == (-1, 0, 0)
            else:
                assert 0 <= T <= 128 * spec.G and below < ke <= below + at


def run_spec(spec, device, units=None):
    _say(f"[recall] {spec.name}: generating + prefill + decode")
    wl = GpuWorkload(spec, device, extra_ctx=2)
    out, sel, sc = wl.step(debug=True)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    _say(f"[recall] {spec.name}: analysis")
    ov, tie, ex = run_recall(wl.cache, wl.q, wl.topk, wl.k_max, sel, sc)
    check_structure(spec, wl, ov, tie, ex)
    if units is None:
        units = [(b, kv) for b in range(spec.B) for kv in range(spec.Hkv)]
    for (b, kv) in units:
        _say(f"[recall] {spec.name}: oracle unit {(b, kv)} len {spec.lengths[b]}")
        check_unit(spec, wl, b, kv, ov, tie, ex)
    ke = np.array([max(0, min(spec.topk[b], wl.k_max, spec.lengths[b])) for b in range(spec.B)])
    frac = ov.sum() / max(1, int((ke[:, None] * np.ones((1, spec.Hq))).sum()))
    _say(f"[recall] {spec.name}: overlap with the exact top-k {frac:.4f}")
    return ov, tie, ex


def test_recall_config1_all_units(gpu):
    run_spec(synth.config(1), gpu)


SMALL = [
    synth.custom("g1 len1 dense", 2, 3, 3, [1, 5000], [4, 5000], [0, 4]),
    synth.custom("g2 ragged k>len k=0", 3, 4, 2, [1030, 2049, 777], [16, 2054, 0], [2, 2, 1]),
    synth.custom("g4 ragged", 2, 8, 2, [9000, 3100], [140, 48], [9, 3]),
    synth.custom("g8", 1, 16, 2, [6000], [93], [6]),
    synth.custom("g4 tiny", 3, 4, 1, [2, 3, 64], [1, 3, 5], [1, 1, 1]),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s.name for s in SMALL])
def test_recall_small_all_units(gpu, spec):
    run_spec(spec, gpu)


def test_recall_config3_sampled(gpu):
    run_spec(synth.config(3), gpu, units=[(0, 0), (3, 7)])


def _bf16(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def hand_cache(device, rows, q_rows, lengths, topk, k_max, G=1):
    """A cache holding the given key rows (bf16 bits [B][Hkv][n][128]) and
    the analyser's other inputs built by hand: the 'selection' is the first
    k_eff positions and the scores are position mod 7, so that the expected
    counts follow from the oracle alone."""
    B, Hkv, n, _ = rows.shape
    cache = hata.HataCache(B, Hkv * G, Hkv, n, device=device)
    cache.k.copy_(bf16_dev(rows, device))
    cache.v.zero_()
    cache.seq_len.copy_(torch.tensor(lengths, dtype=torch.int32))
    q = bf16_dev(q_rows, device)
    topk_t = torch.tensor(topk, dtype=torch.int32, device=device)
    sel = np.full((B, Hkv, k_max), -1, dtype=np.int32)
    scores = np.zeros((B, Hkv, n), dtype=np.int16)
    for b in range(B):
        ke = max(0, min(topk[b], k_max, lengths[b]))
        sel[b, :, :ke] = np.arange(ke)
        scores[b, :, :lengths[b]] = np.arange(lengths[b]) % 7
    sel_t = torch.from_numpy(sel).to(device)
    sc_t = torch.from_numpy(scores).to(device)
    ov, tie, ex = run_recall(cache, q, topk_t, k_max, sel_t, sc_t)
    for b in range(B):
        L = lengths[b]
        k = min(topk[b], k_max)
        for kv in range(Hkv):
            for h in range(G):
                hq = kv * G + h
                e = oracle.exact_topk(q_rows[b, hq], rows[b, kv, :L], k)
                assert np.array_equal(ex[b, hq, :e.size], e), (b, hq)
                assert np.all(ex[b, hq, e.size:] == -1)
                assert ov[b, hq] == oracle.overlap(sel[b, kv, :e.size], e), (b, hq)
            want = oracle.tie_bucket(scores[b, kv, :L].astype(np.int32), k)
            assert tuple(int(x) for x in tie[b, kv]) == want, (b, kv)
    return ov, ex


def test_recall_ties_and_rounding_order(gpu):
    # q = all ones.  Rows 500-502 have the same real logit 1, but the
    # sequential double sum gives row 500 (2^60, 1, -2^60) the value 0 and
    # rows 501 (2^60, -2^60, 1) and 502 (1) the value 1; rows 900 and 1500
    # are copies of row 10 (equal logits: the lower index wins).  The huge
    # rows widen the error bound so that every key is ranked exactly.
    rng = np.random.default_rng(5)
    n = 2000
    rows = _bf16(rng.standard_normal((2, 1, n, 128)))
    for b in range(2):
        rows[b, 0, 500:503] = 0
        rows[b, 0, 500, :3] = [0x5D80, 0x3F80, 0xDD80]
        rows[b, 0, 501, :3] = [0x5D80, 0xDD80, 0x3F80]
        rows[b, 0, 502, 0] = 0x3F80
        rows[b, 0, 900] = rows[b, 0, 10]
        rows[b, 0, 1500] = rows[b, 0, 10]
    q = np.full((2, 1, 128), 0x3F80, dtype=np.uint16)
    hand_cache(gpu, rows, q, [n, n], [1000, 37], 1000)


def test_recall_all_exact_and_empty(gpu):
    # |q| |k| >= 2^120 (q_0 = 2^62, a few keys with k_0 = +-2^62): every key is
    # ranked on its exact double logit.  Entry 1 has an empty context and
    # entry 2 a budget of 0.
    rng = np.random.default_rng(8)
    n, G = 1500, 2
    rows = _bf16(rng.standard_normal((3, 2, n, 128)))
    rows[:, :, 100:110, 0] = 0x5E80   # 2^62
    rows[:, :, 200:210, 0] = 0xDE80   # -2^62
    rows[:, :, 300:305] = rows[:, :, 100:105]
    q = _bf16(rng.standard_normal((3, 4, 128)))
    q[:, :, 0] = 0x5E80
    hand_cache(gpu, rows, q, [n, 0, 900], [64, 10, 0], 64, G=G)


def test_recall_sparse_band_random(gpu):
    # Ordinary Gaussian rows, several estimate blocks and a ragged tail: the
    # common path where almost every key is decided by its estimate.
    rng = np.random.default_rng(12)
    n = 5000
    rows = _bf16(rng.standard_normal((2, 2, n, 128)))
    q = _bf16(rng.standard_normal((2, 8, 128)))
    hand_cache(gpu, rows, q, [n, 3333], [300, 2000], 2000, G=4)
