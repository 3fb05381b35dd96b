"""Host-side checks of the C ABI (no GPU needed: only argument validation and
the workspace plan run, no kernel is launched).

  - libhata.so loads and exports every function include/hata.h declares;
  - status strings;
  - every invalid or unsupported argument returns its status code before any
    launch;
  - hata_decode_workspace_bytes follows the plan for each configuration.
"""
import ctypes
import os
import re

import pytest

import hash_top_sparse_encode_amd as hata

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hata.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hata_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(hata.EXPORTED_SYMBOLS)
    L = hata.lib()
    for n in names:
        assert hasattr(L, n), n
    nm = os.popen(f"nm -D --defined-only {hata.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), n


def test_status_strings():
    for s in range(6):
        assert hata.hata_status_string(s)
    assert "unknown" in hata.hata_status_string(99)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def cache(**kw):
    base = dict(k=FAKE, v=FAKE, codes=FAKE, seq_len=FAKE, ctrl=FAKE, batch=2, n_q_heads=8,
                n_kv_heads=2, head_dim=128, n_bits=128, max_ctx=1000)
    base.update(kw)
    return hata._CCache(**base)


def decode(c, q=FAKE, w=FAKE, topk=FAKE, k_max=16, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return hata.lib().hata_decode_attn(ctypes.byref(c), q, w, topk, k_max, out, ws, ws_bytes,
                                       None, None, None)


def test_decode_validation():
    E = hata
    assert decode(cache(head_dim=64)) == E.HATA_ERR_UNSUPPORTED
    assert decode(cache(n_bits=96)) == E.HATA_ERR_UNSUPPORTED
    assert decode(cache(n_bits=512)) == E.HATA_ERR_UNSUPPORTED
    assert decode(cache(n_q_heads=6)) == E.HATA_ERR_UNSUPPORTED        # 6 % 4? G = 3
    assert decode(cache(n_q_heads=32)) == E.HATA_ERR_UNSUPPORTED       # G = 16
    assert decode(cache(n_q_heads=7)) == E.HATA_ERR_UNSUPPORTED        # not a multiple
    assert decode(cache(batch=0)) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(max_ctx=-1)) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(max_ctx=1 << 33)) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(k=0)) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(codes=0)) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(ctrl=0)) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(k=FAKE + 2)) == E.HATA_ERR_INVALID_ARG         # misaligned
    assert decode(cache(batch=40000)) == E.HATA_ERR_UNSUPPORTED        # > 65535 units
    assert decode(cache(), q=0) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(), q=FAKE + 8) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(), out=0) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(), topk=0) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(), k_max=-1) == E.HATA_ERR_INVALID_ARG
    assert decode(cache(), ws=0) == E.HATA_ERR_WORKSPACE
    assert decode(cache(), ws=FAKE + 64) == E.HATA_ERR_WORKSPACE      # not 256-aligned
    assert decode(cache(), ws_bytes=100) == E.HATA_ERR_WORKSPACE
    assert hata.lib().hata_decode_attn(None, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1 << 40, None,
                                       None, None) == E.HATA_ERR_INVALID_ARG


def test_append_validation():
    L = hata.lib()
    c = cache()

    def app(c=c, k=FAKE, v=FAKE, n=FAKE, t=4, w=FAKE):
        return L.hata_append(ctypes.byref(c), k, v, n, t, w, None)

    assert app(k=None) == hata.HATA_ERR_INVALID_ARG      # only one of k_new / v_new
    assert app(v=None) == hata.HATA_ERR_INVALID_ARG
    assert app(n=None) == hata.HATA_ERR_INVALID_ARG
    assert app(w=None) == hata.HATA_ERR_INVALID_ARG
    assert app(t=-1) == hata.HATA_ERR_INVALID_ARG
    assert app(c=cache(head_dim=96)) == hata.HATA_ERR_UNSUPPORTED
    assert app(c=cache(seq_len=0)) == hata.HATA_ERR_INVALID_ARG
    assert app(t=0) == hata.HATA_OK                       # nothing to append: no launch


def test_encode_keys_validation():
    L = hata.lib()
    enc = L.hata_encode_keys_nbits
    assert enc(FAKE, 5, 1, 128, 128, FAKE, 96, FAKE, None) == hata.HATA_ERR_UNSUPPORTED
    assert enc(FAKE + 2, 5, 1, 128, 128, FAKE, 64, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert enc(FAKE, 5, 1, 132, 128, FAKE, 64, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert enc(FAKE, 5, 1, 128, 128, None, 256, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert enc(None, 0, 1, 128, 128, None, 32, None, None) == hata.HATA_OK
    assert L.hata_encode_keys(FAKE, -1, 1, 128, 128, FAKE, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert L.hata_encode_keys(FAKE, 5, 0, 128, 128, FAKE, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert L.hata_encode_keys(None, 5, 1, 128, 128, FAKE, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert L.hata_encode_keys(FAKE, 5, 1, 128, 128, None, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert L.hata_encode_keys(FAKE, 5, 1, 128, 128, FAKE, None, None) == hata.HATA_ERR_INVALID_ARG
    assert L.hata_encode_keys(FAKE, 5, 1, -128, 128, FAKE, FAKE, None) == hata.HATA_ERR_INVALID_ARG
    assert L.hata_encode_keys(None, 0, 1, 128, 128, None, None, None) == hata.HATA_OK


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 8, 8, 4096), (8, 32, 8, 32768), (4, 32, 8, 131072),
                                       (1, 32, 8, 1048576), (64, 32, 8, 65536)])
def test_workspace_plan(B, Hq, Hkv, N):
    c = cache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_ctx=N + 8)
    n = hata.lib().hata_decode_workspace_bytes(ctypes.byref(c), 2048)
    units = B * Hkv
    assert n >= units * (N + 8) * 2  # at least the u16 scores
    G = Hq // Hkv
    # u16 scores (2 B per key) plus cumulative histograms of each 2048-key
    # scan slot (4 B per bin, 128 G + 1 bins), plus the split partials and
    # small per-unit buffers
    assert n < units * (N + 8) * (2 + 4 * (128 * G + 1) / 2048 + 0.4) + (1 << 22)
    assert n % 256 == 0
    assert hata.lib().hata_decode_workspace_bytes(ctypes.byref(cache(head_dim=64)), 1) == 0
    assert hata.lib().hata_decode_workspace_bytes(ctypes.byref(cache(n_bits=48)), 1) == 0
    assert hata.lib().hata_decode_workspace_bytes(None, 1) == 0


@pytest.mark.parametrize("n_bits", [32, 64, 128, 256])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(4, 32, 8, 131072), (1, 8, 2, 1000), (2, 16, 2, 600000)])
def test_workspace_plan_code_lengths(n_bits, B, Hq, Hkv, N):
    # Every code length runs the same step, so the workspace is one layout:
    # per unit the launch generation, the tagged query and new-key code
    # words ((G + 1) r / 32 of them), the unit histogram (G r + 2 words), per
    # work item (spans of 8192 keys, or multiples of it past 64 items) a
    # tagged cumulative histogram (G r + 1 bins) and the softmax partials,
    # then the u16 score rows; each section 256-byte aligned.
    c = cache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_ctx=N, n_bits=n_bits)
    n = hata.lib().hata_decode_workspace_bytes(ctypes.byref(c), 2048)
    units, G = B * Hkv, Hq // Hkv
    span = -(-N // (64 * 8192)) * 8192
    C = -(-N // span)
    NB = G * n_bits + 1
    a256 = lambda x: -(-x // 256) * 256
    sections = [units * 4, units * (G + 1) * (n_bits // 32) * 8, units * (NB + 1) * 4,
                units * C * NB * 8, units * C * G * 2 * 4, units * C * G * 128 * 4,
                units * (-(-N // 64) * 64) * 2]
    assert n == sum(a256(x) for x in sections)


def recall(c, q=FAKE, topk=FAKE, k_max=16, sel=FAKE, sc=FAKE, ov=FAKE, tie=FAKE, ex=None,
           ws=FAKE, ws_bytes=1 << 40):
    return hata.lib().hata_exact_topk_recall(ctypes.byref(c), q, topk, k_max, sel, sc, ov, tie,
                                             ex, ws, ws_bytes, None)


def test_recall_validation():
    E = hata
    assert recall(cache(head_dim=64)) == E.HATA_ERR_UNSUPPORTED
    assert recall(cache(n_q_heads=32)) == E.HATA_ERR_UNSUPPORTED
    assert recall(cache(k=0)) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), q=0) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), q=FAKE + 2) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), topk=0) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), sel=0) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), sc=0) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), ov=0) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), tie=0) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), k_max=-1) == E.HATA_ERR_INVALID_ARG
    assert recall(cache(), ws=0) == E.HATA_ERR_WORKSPACE
    assert recall(cache(), ws=FAKE + 64) == E.HATA_ERR_WORKSPACE
    assert recall(cache(), ws_bytes=1000) == E.HATA_ERR_WORKSPACE


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 8, 8, 4096), (4, 32, 8, 131072), (3, 6, 3, 1000)])
def test_recall_workspace_plan(B, Hq, Hkv, N):
    c = cache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_ctx=N)
    n = hata.lib().hata_recall_workspace_bytes(ctypes.byref(c))
    # fp32 estimates (row stride rounded up to 64), band indices, exact
    # logits and flags per query head and position, per-block key norms
    lo = B * Hq * N * (4 + 4 + 8 + 1)
    assert lo <= n <= lo + B * Hq * 64 * 4 + B * Hkv * (N // 1024 + 1) * 8 + 5 * 256
    assert n % 256 == 0
    assert hata.lib().hata_recall_workspace_bytes(ctypes.byref(cache(head_dim=64))) == 0
    assert hata.lib().hata_recall_workspace_bytes(None) == 0


def static_step(c, k_new=FAKE, v_new=FAKE, q=FAKE, w=FAKE, topk=FAKE, k_max=16, out=FAKE):
    return hata.lib().hata_decode_step_static(ctypes.byref(c), k_new, v_new, q, w, topk, k_max,
                                              out, None, None, None)


def test_static_step_validation():
    # Every failure below is decided on the host before anything is enqueued
    # (and before the scratch's address is looked up).
    E = hata
    assert static_step(cache(n_bits=48)) == E.HATA_ERR_UNSUPPORTED
    assert static_step(cache(head_dim=64)) == E.HATA_ERR_UNSUPPORTED
    assert static_step(cache(k=0)) == E.HATA_ERR_INVALID_ARG
    assert static_step(cache(), k_new=0) == E.HATA_ERR_INVALID_ARG
    assert static_step(cache(), v_new=0) == E.HATA_ERR_INVALID_ARG
    assert static_step(cache(), q=FAKE + 8) == E.HATA_ERR_INVALID_ARG
    assert static_step(cache(), k_new=FAKE + 8) == E.HATA_ERR_INVALID_ARG
    assert static_step(cache(), k_max=-1) == E.HATA_ERR_INVALID_ARG
    # 64 sequences x 8 KV heads at 200K context: the span histograms alone
    # take 512 units x 25 items x 513 bins x 8 B = 52 MB > the 32 MiB scratch
    big = cache(batch=64, n_q_heads=32, n_kv_heads=8, max_ctx=200000)
    assert static_step(big) == E.HATA_ERR_SCRATCH_LIMIT
    assert static_step(cache(batch=64, n_q_heads=32, n_kv_heads=8, max_ctx=200000,
                             n_bits=32)) == E.HATA_ERR_SCRATCH_LIMIT
    assert "scratch" in hata.hata_status_string(E.HATA_ERR_SCRATCH_LIMIT)
