"""GPU parity of the other code lengths (r = 32, 64, 256; the hash-length
ablation of the HATA review's "Free parameters") against the oracle, which is
written for any r.

Bars as for 128 bits: codes, summed Hamming scores (0 .. G r) and selected
indices bit-exact, outputs within 2e-2; the recall analyser's tie bucket
and overlaps bit-exact with up to 8 x 256 + 1 score bins.  Encoder inputs
include rows built to sit inside the sign decision's error band, so the
exact double-sum path is taken.
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

OUT_TOL = 2e-2
LENGTHS = [32, 64, 256]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("n_bits", LENGTHS + [128])
def test_encode_keys_nbits(gpu, n_bits):
    rng = np.random.default_rng(n_bits)
    n, H = 1000, 3
    w = (rng.standard_normal((H, 128, n_bits)) / np.sqrt(128)).astype(np.float32)
    x = rng.standard_normal((n, H, 128)).astype(np.float32)
    # rows 0-199: two entries, x_a = W[b][j] and x_b = -W[a][j] with both W
    # entries made bf16-exact, so the real sum for bit j is exactly 0 (bit 0)
    # while the fp32 estimate is a rounding residue inside the error band
    wb = w.view(np.uint32)
    for i in range(200):
        h, j = i % H, (7 * i) % n_bits
        da = i % 128
        db = (da + 1 + i // 128) % 128
        wb[h, da, j] &= 0xFFFF0000
        wb[h, db, j] &= 0xFFFF0000
        x[i, h] = 0.0
        x[i, h, da] = w[h, db, j]
        x[i, h, db] = -w[h, da, j]
    keys = _bf16(x)
    kt = bf16_dev(keys, gpu)
    codes = hata.hata_encode_keys(kt, torch.from_numpy(w).to(gpu))
    torch.cuda.synchronize()
    got = codes.cpu().numpy().view(np.uint32)
    for h in range(H):
        want = oracle.encode(keys[:, h], w[h])
        assert np.array_equal(got[:, h], want), f"r={n_bits} head {h}: " \
            f"{int((got[:, h] != want).any(1).sum())} rows differ"


def check_unit(spec, wl, b, kv, out, sel, sc):
    G = spec.G
    L = spec.lengths[b]
    K, V = synth.unit_context(spec, b, kv, wl.q_host, wl.new_host)
    ref = oracle.decode_unit(wl.q_host[b, kv * G:(kv + 1) * G], wl.w_host[kv], K, V,
                             spec.topk[b], threads=16)
    codes = wl.cache.codes[b, kv, :L].cpu().numpy().view(np.uint32)
    assert np.array_equal(codes, ref["kcodes"]), f"codes differ at {(b, kv)}"
    scores = sc[b, kv, :L].cpu().numpy().view(np.uint16).astype(np.int32)
    assert np.array_equal(scores, ref["scores"]), f"scores differ at {(b, kv)}"
    ke = max(0, min(spec.topk[b], wl.k_max, L))
    s = sel[b, kv].cpu().numpy()
    assert np.array_equal(s[:ke], ref["idx"]), f"selection differs at {(b, kv)}"
    assert np.all(s[ke:] == -1)
    o = out[b, kv * G:(kv + 1) * G].float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ref["out"]).max()
    assert err <= OUT_TOL, f"output error {err} at {(b, kv)}"
    return ref


def run_spec(spec, device, n_bits, units=None, fused=True):
    _say(f"[bits] r={n_bits} {spec.name}: prefill + step (fused={fused})")
    wl = GpuWorkload(spec, device, extra_ctx=2, n_bits=n_bits)
    out, sel, sc = wl.step(debug=True, fused=fused)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    assert wl.cache.seq_len.cpu().tolist() == list(spec.lengths)
    if units is None:
        units = [(b, kv) for b in range(spec.B) for kv in range(spec.Hkv)]
    for (b, kv) in units:
        _say(f"[bits] r={n_bits} {spec.name}: oracle unit {(b, kv)}")
        check_unit(spec, wl, b, kv, out, sel, sc)
    return wl, sel, sc


SPECS = [
    synth.custom("g1 len1 dense", 2, 3, 3, [1, 5000], [4, 5000], [0, 4]),
    synth.custom("g2 ragged k>len k=0", 3, 4, 2, [1030, 2049, 777], [16, 2054, 0], [2, 2, 1]),
    synth.custom("g4 two spans", 2, 8, 2, [17000, 3100], [300, 48], [9, 3]),
    synth.custom("g8", 1, 16, 2, [6000], [93], [6]),
    synth.custom("g4 tiny", 3, 4, 1, [2, 3, 64], [1, 3, 5], [1, 1, 1]),
]


@pytest.mark.parametrize("n_bits", LENGTHS)
@pytest.mark.parametrize("spec", SPECS, ids=[s.name for s in SPECS])
def test_decode_step_other_lengths(gpu, spec, n_bits):
    run_spec(spec, gpu, n_bits)


@pytest.mark.parametrize("n_bits", [64, 256])
def test_two_calls_other_lengths(gpu, n_bits):
    run_spec(SPECS[2], gpu, n_bits, fused=False)


def test_config2_r256_sampled(gpu):
    run_spec(synth.config(2), gpu, 256, units=[(0, 0), (7, 7)])


@pytest.mark.parametrize("n_bits", [64, 256])
def test_long_context_other_lengths(gpu, n_bits):
    # Past 512K keys a work item spans 16384 keys and keeps its scores in
    # the workspace instead of LDS (the kernel's second form); G = 8 at 256
    # bits has 2049 score bins.
    G = 4 if n_bits == 64 else 8
    spec = synth.custom(f"long r{n_bits}", 1, 2 * G, 2, [600000], [9375], [600], seed=50 + n_bits)
    run_spec(spec, gpu, n_bits, units=[(0, 1)])


def test_recall_r256_g8(gpu):
    # 8 x 256 + 1 = 2049 score bins in the tie bucket
    spec = SPECS[3]
    wl, sel, sc = run_spec(spec, gpu, 256)
    ws = hata.alloc_recall_workspace(wl.cache)
    ex = torch.full((spec.B, spec.Hq, wl.k_max), -7, dtype=torch.int32, device=gpu)
    ov, tie = hata.hata_exact_topk_recall(wl.cache, wl.q, wl.topk, wl.k_max, sel, sc, ws,
                                          exact_idx_out=ex)
    torch.cuda.synchronize()
    ov, tie, ex = ov.cpu().numpy(), tie.cpu().numpy(), ex.cpu().numpy()
    G = spec.G
    for kv in range(spec.Hkv):
        K, V = synth.unit_context(spec, 0, kv, wl.q_host, wl.new_host)
        ref = oracle.decode_unit(wl.q_host[0, kv * G:(kv + 1) * G], wl.w_host[kv], K, V,
                                 spec.topk[0], threads=16)
        k = min(spec.topk[0], wl.k_max)
        assert tuple(int(x) for x in tie[0, kv]) == oracle.tie_bucket(ref["scores"], k)
        for h in range(G):
            e = oracle.exact_topk(wl.q_host[0, kv * G + h], K, k)
            assert np.array_equal(ex[0, kv * G + h, :e.size], e)
            assert ov[0, kv * G + h] == oracle.overlap(ref["idx"], e)


def test_full_cache_other_length(gpu):
    # a sequence whose cache is full is not appended (status flag) and
    # decodes over its existing context
    spec = synth.custom("full", 2, 4, 2, [3000, 500], [40, 20], [2, 1])
    wl = GpuWorkload(spec, gpu, extra_ctx=0, n_bits=64)
    wl.cache.seq_len.copy_(torch.tensor([3000, 499], dtype=torch.int32))
    out, sel, sc = wl.step(debug=True)
    torch.cuda.synchronize()
    assert wl.cache.status() & hata.HATA_DEV_APPEND_OVERFLOW
    assert wl.cache.seq_len.cpu().tolist() == [3000, 500]


def test_cut_at_the_top_bin_r256_g8(gpu):
    # All eight query heads of the group equal, and one key of the unit's
    # last span set to their negation: its code differs from theirs in every
    # bit, so its summed score is 8 x 256 = 2048, the top bin.  With the
    # token budget equal to the context the cut T is that bin, and the last
    # span's counts below it are those of bin 2047 of its histograms (the
    # bins nearest the end of the scan state in shared memory).
    spec = synth.custom("g8 top bin", 1, 8, 1, [9000], [9000], [0], seed=77)
    wl = GpuWorkload(spec, gpu, extra_ctx=2, n_bits=256, encode_prefill=False)
    q = wl.q_host.copy()
    q[0, :] = q[0, 0]
    wl.q_host = q
    wl.q = bf16_dev(q, gpu)
    pos = 8192 + 100
    anti = (q[0, 0] ^ 0x8000).astype(np.uint16)
    wl.cache.k[0, 0, pos] = bf16_dev(anti[None], gpu)[0]
    wl.encode_prefill()
    _say("[bits] r=256 g8 top bin: step")
    out, sel, sc = wl.step(debug=True)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    K, V = synth.unit_context(spec, 0, 0, wl.q_host, wl.new_host)
    K[pos] = anti
    ref = oracle.decode_unit(q[0], wl.w_host[0], K, V, 9000, threads=16)
    assert ref["scores"][pos] == 8 * 256 and ref["scores"].max() == 8 * 256
    codes = wl.cache.codes[0, 0, :9000].cpu().numpy().view(np.uint32)
    assert np.array_equal(codes, ref["kcodes"])
    assert np.array_equal(sc[0, 0, :9000].cpu().numpy().view(np.uint16).astype(np.int32), ref["scores"])
    assert np.array_equal(sel[0, 0].cpu().numpy()[:9000], ref["idx"])
    err = np.abs(out[0].float().cpu().numpy().astype(np.float64) - ref["out"]).max()
    assert err <= OUT_TOL
