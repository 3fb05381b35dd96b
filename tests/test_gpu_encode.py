"""GPU parity of the bulk key encoder (hata_encode_keys) against the CPU
oracle, through the C ABI: codes bit-exact.

Covers the matrix-core path (from 64 rows, 16-byte aligned rows) and the
exact kernel (fewer rows, or an unaligned base), strided multi-head layouts,
and rows built to land inside the matrix cores' error band: exact
cancellation (x[t] = x[t + 64] against W[t + 64] = -W[t], whose sequential
double sum is a rounding residue or zero), tiny and huge magnitudes, and
all-zero rows.  Inputs are seeded numpy draws.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import hash_top_sparse_encode_amd as hata
import oracle
import synth

pytestmark = pytest.mark.gpu


def _bf16(x):
    return synth.f64_to_bf16(np.asarray(x, dtype=np.float64))


def _dev_bf16(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def _encode(keys_bits, w, device, pad=0, offset=0):
    """hata_encode_keys on keys [n][H][128] stored with `pad` extra elements
    per row and the base `offset` elements into the buffer."""
    n, H, _ = keys_bits.shape
    row = H * 128 + pad
    buf = np.zeros(offset + n * row + 8, dtype=np.uint16)
    view = buf[offset:offset + n * row].reshape(n, row)[:, :H * 128].reshape(n, H, 128)
    view[...] = keys_bits
    dbuf = _dev_bf16(buf, device)
    keys = torch.as_strided(dbuf, (n, H, 128), (row, 128, 1), offset)
    codes = hata.hata_encode_keys(keys, torch.from_numpy(w).to(device))
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint32)


def _oracle_codes(keys_bits, w):
    n, H, _ = keys_bits.shape
    out = np.zeros((n, H, 4), dtype=np.uint32)
    for h in range(H):
        out[:, h] = oracle.encode(np.ascontiguousarray(keys_bits[:, h]), w[h])
    return out


def _gauss_inputs(seed, n, H, wscale=1.0 / np.sqrt(128.0)):
    rng = np.random.default_rng(seed)
    keys = _bf16(rng.standard_normal((n, H, 128)))
    w = (rng.standard_normal((H, 128, 128)) * wscale).astype(np.float32)
    return keys, w


@pytest.mark.parametrize("n,H,pad,offset", [
    (1000, 3, 8, 0),     # matrix cores, strided rows
    (64, 1, 0, 0),       # one full tile
    (130, 2, 0, 8),      # ragged last tile, aligned offset
    (30, 2, 0, 0),       # exact kernel (few rows)
    (200, 2, 0, 3),      # exact kernel (unaligned base)
    (77, 2, 5, 0),       # exact kernel (stride not a multiple of 8)
])
def test_encode_keys_matches_oracle(gpu, n, H, pad, offset):
    keys, w = _gauss_inputs(100 + n + H, n, H)
    got = _encode(keys, w, gpu, pad=pad, offset=offset)
    assert np.array_equal(got, _oracle_codes(keys, w))


def test_encode_keys_band_cases(gpu):
    rng = np.random.default_rng(7)
    n, H = 512, 2
    w = (rng.standard_normal((H, 128, 128)) / np.sqrt(128.0)).astype(np.float32)
    # columns 0..63 of head 0: W[t + 64] = -W[t] for every t < 64
    w[0, 64:, :64] = -w[0, :64, :64]
    keys = _bf16(rng.standard_normal((n, H, 128)))
    # rows 0..199: x[t + 64] = x[t] -> those 64 bits of head 0 sum to exactly 0
    keys[:200, 0, 64:] = keys[:200, 0, :64]
    # rows 200..263: tiny and huge magnitudes
    scale = np.where(np.arange(64) % 2 == 0, 2.0 ** -60, 2.0 ** 60)
    keys[200:264] = _bf16(synth.bf16_to_f32(keys[200:264]).astype(np.float64) *
                          scale[:, None, None])
    # rows 264..299: all zero (every bit 0)
    keys[264:300] = 0
    # rows 300..399: a single nonzero coordinate (products exact, one term)
    keys[300:400] = 0
    keys[300:400, :, 5] = _bf16(rng.standard_normal((100, H)))
    got = _encode(keys, w, gpu)
    ref = _oracle_codes(keys, w)
    assert np.array_equal(got, ref)
    assert np.all(ref[264:300] == 0)


@pytest.mark.parametrize("n_bits", [32, 64, 128, 256])
def test_encode_keys_scaled_columns_and_tiny_rows(gpu, n_bits):
    # W_H columns the matrix-core path rescales by powers of two: a zero
    # column, columns scaled by 2^40 and 2^-40, one element 2^30 among
    # ordinary ones, columns below fp32's normal range (2^-120 scale) and a
    # column with a single nonzero element.  Rows whose squares leave the
    # normal range (2^-70, 2^-100 scale), rows with one subnormal bf16 entry,
    # rows of zeros.  650 rows: ten full 64-row groups and a ragged one.
    rng = np.random.default_rng(300 + n_bits)
    n, H = 650, 2
    w = (rng.standard_normal((H, 128, n_bits)) / np.sqrt(128.0)).astype(np.float32)
    w[0, :, 3] = 0.0
    w[0, :, 7] *= np.float32(2.0 ** 40)
    w[0, :, 9] *= np.float32(2.0 ** -40)
    w[0, 17, 11] = np.float32(2.0 ** 30)
    w[1, :, 20:24] = (w[1, :, 20:24].astype(np.float64) * 2.0 ** -120).astype(np.float32)
    w[1, :, 30] = 0.0
    w[1, 5, 30] = np.float32(-3e-30)
    x = rng.standard_normal((n, H, 128))
    x[0:64] *= 2.0 ** -70
    x[64:100] *= 2.0 ** -100
    x[100:120] = 0.0
    x[100:120, :, 9] = 2.0 ** -130
    x[120:130] = 0.0
    keys = _bf16(x)
    got = hata.hata_encode_keys(_dev_bf16(keys, gpu), torch.from_numpy(w).to(gpu))
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    for h in range(H):
        want = oracle.encode(np.ascontiguousarray(keys[:, h]), w[h])
        assert np.array_equal(got[:, h], want), f"r={n_bits} head {h}: " \
            f"{int((got[:, h] != want).any(1).sum())} rows differ"
    assert np.all(got[120:130] == 0)


def test_append_prefill_uses_matrix_cores_and_matches(gpu):
    # A prefill append with new rows given (k_new / v_new): codes, K and V
    # rows land in the cache, lengths advance.
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T = 2, 4, 2, 150
    max_ctx = 400
    cache = hata.HataCache(B, Hq, Hkv, max_ctx, device=gpu)
    cache.k.zero_()
    cache.v.zero_()
    start = [17, 0]
    cache.seq_len.copy_(torch.tensor(start, dtype=torch.int32))
    n_new = [150, 97]
    kb = _bf16(rng.standard_normal((B, T, Hkv, 128)))
    vb = _bf16(rng.standard_normal((B, T, Hkv, 128)))
    w = (rng.standard_normal((Hkv, 128, 128)) / np.sqrt(128.0)).astype(np.float32)
    hata.hata_append(cache, _dev_bf16(kb, gpu), _dev_bf16(vb, gpu),
                     torch.tensor(n_new, dtype=torch.int32, device=gpu), T,
                     torch.from_numpy(w).to(gpu))
    torch.cuda.synchronize()
    assert cache.status() == 0
    assert cache.seq_len.cpu().tolist() == [start[b] + n_new[b] for b in range(B)]
    codes = cache.codes.cpu().numpy().view(np.uint32)
    kc = cache.k.view(torch.int16).cpu().numpy().view(np.uint16)
    vc = cache.v.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        for kv in range(Hkv):
            rows = kb[b, :n_new[b], kv]
            sl = slice(start[b], start[b] + n_new[b])
            assert np.array_equal(kc[b, kv, sl], rows)
            assert np.array_equal(vc[b, kv, sl], vb[b, :n_new[b], kv])
            assert np.array_equal(codes[b, kv, sl], oracle.encode(rows, w[kv]))
