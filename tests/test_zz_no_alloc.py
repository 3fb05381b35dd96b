"""hata_decode_step_static -- the allocation-free decode step on the
library's static scratch -- against hata_decode_step with a workspace, through
the C ABI: outputs, selected indices, scores, codes, K/V rows and lengths
bit-identical, on two calls in a row, the second with a smaller input
(fewer sequences, shorter contexts, another group size), so the second call
runs on scratch the first left under another layout.
"""
from __future__ import annotations

import pytest
import torch

import hash_top_sparse_encode_amd as hata
import synth
from workload import GpuWorkload

pytestmark = pytest.mark.gpu


def _static_step(wl, sel, sc):
    return hata.hata_decode_step_static(wl.cache, wl.k_new, wl.v_new, wl.q, wl.w, wl.topk,
                                        wl.k_max, wl.out, sel_idx_out=sel, scores_out=sc)


def _compare(spec, gpu, n_bits=128):
    ref = GpuWorkload(spec, gpu, extra_ctx=2, n_bits=n_bits)
    got = GpuWorkload(spec, gpu, extra_ctx=2, n_bits=n_bits)
    out_r, sel_r, sc_r = ref.step(debug=True)
    sel, sc = got.debug_buffers()
    _static_step(got, sel, sc)
    torch.cuda.synchronize()
    assert ref.cache.status() == 0 and got.cache.status() == 0
    assert torch.equal(got.out.view(torch.int16), out_r.view(torch.int16))
    assert torch.equal(sel, sel_r) and torch.equal(sc, sc_r)
    assert torch.equal(got.cache.codes, ref.cache.codes)
    assert torch.equal(got.cache.k, ref.cache.k) and torch.equal(got.cache.v, ref.cache.v)
    assert torch.equal(got.cache.seq_len, ref.cache.seq_len)
    # again without debug outputs (the fast scoring path), from the prefill
    got.reset_to_prefill()
    hata.hata_decode_step_static(got.cache, got.k_new, got.v_new, got.q, got.w, got.topk,
                                 got.k_max, got.out)
    torch.cuda.synchronize()
    assert got.cache.status() == 0
    assert torch.equal(got.out.view(torch.int16), out_r.view(torch.int16))


def test_static_step_matches_workspace_step_two_calls(gpu):
    big = synth.custom("static big", 3, 32, 8, [40000, 17000, 70000], [625, 265, 1100],
                       [40, 17, 70], seed=41)
    small = synth.custom("static small", 2, 8, 4, [9000, 3100], [140, 48], [9, 3], seed=42)
    print("[no-alloc] first call: 3 x 8 units up to 70K keys", flush=True)
    _compare(big, gpu)
    print("[no-alloc] second call: 2 x 4 units, G = 2", flush=True)
    _compare(small, gpu)


def test_static_step_other_code_lengths(gpu):
    # every code length runs the same step on the static scratch: 256-bit
    # codes, then a smaller 32-bit cache on what the first call left
    big = synth.custom("static r256", 2, 32, 8, [30000, 12000], [470, 190], [30, 12], seed=43)
    small = synth.custom("static r32", 2, 8, 2, [5000, 700], [80, 11], [5, 1], seed=44)
    print("[no-alloc] r = 256: 2 x 8 units up to 30K keys", flush=True)
    _compare(big, gpu, n_bits=256)
    print("[no-alloc] r = 32: 2 x 2 units, G = 4", flush=True)
    _compare(small, gpu, n_bits=32)
