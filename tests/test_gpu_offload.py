"""The offloaded layout: K/V cache rows in pinned host memory, codes and
workspace in device memory (the HATA review's offloaded setting, "Core
claim"; its offloading variant, "If this is right").  The kernels are the
same; the selected rows and the appended ones cross the host link.

Bars: against the oracle as in the device-resident parity tests (codes,
scores, indices bit-exact; outputs within 2e-2), and bit-identical to the
same workload with the cache in device memory (outputs included), for the
fused step, the two-call route and the prefill encode that reads its rows
from host memory.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from workload import GpuWorkload

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_against_oracle(spec, wl, out, sel, sc, units):
    G = spec.G
    for (b, kv) in units:
        _say(f"[offload] {spec.name}: oracle unit {(b, kv)}")
        L = spec.lengths[b]
        K, V = synth.unit_context(spec, b, kv, wl.q_host, wl.new_host)
        ref = oracle.decode_unit(wl.q_host[b, kv * G:(kv + 1) * G], wl.w_host[kv], K, V,
                                 spec.topk[b], threads=16)
        codes = wl.cache.codes[b, kv, :L].cpu().numpy().view(np.uint32)
        assert np.array_equal(codes, ref["kcodes"])
        scores = sc[b, kv, :L].cpu().numpy().view(np.uint16).astype(np.int32)
        assert np.array_equal(scores, ref["scores"])
        ke = max(0, min(spec.topk[b], wl.k_max, L))
        assert np.array_equal(sel[b, kv, :ke].cpu().numpy(), ref["idx"])
        o = out[b, kv * G:(kv + 1) * G].float().cpu().numpy().astype(np.float64)
        assert np.abs(o - ref["out"]).max() <= OUT_TOL


def compare_layouts(spec, device, fused=True, units=None):
    _say(f"[offload] {spec.name}: host K/V, fused={fused}")
    host = GpuWorkload(spec, device, extra_ctx=2, offload=True)
    assert not host.cache.k.is_cuda and host.cache.k.is_pinned()
    ho, hs, hc = host.step(debug=True, fused=fused)
    torch.cuda.synchronize()
    assert host.cache.status() == 0
    _say(f"[offload] {spec.name}: device K/V")
    dev = GpuWorkload(spec, device, extra_ctx=2)
    do, ds, dc = dev.step(debug=True, fused=fused)
    torch.cuda.synchronize()
    assert torch.equal(ho.view(torch.int16), do.view(torch.int16))
    assert torch.equal(hs, ds) and torch.equal(hc, dc)
    assert torch.equal(host.cache.codes, dev.cache.codes)
    assert torch.equal(host.cache.seq_len, dev.cache.seq_len)
    # the appended rows landed in host memory
    assert torch.equal(host.cache.k.to(device), dev.cache.k)
    assert torch.equal(host.cache.v.to(device), dev.cache.v)
    if units is None:
        units = [(b, kv) for b in range(spec.B) for kv in range(spec.Hkv)]
    check_against_oracle(spec, host, ho, hs, hc, units)


SPECS = [
    synth.custom("off g2 ragged k>len k=0", 3, 4, 2, [1030, 2049, 777], [16, 2054, 0], [2, 2, 1]),
    synth.custom("off g4 ragged", 2, 8, 2, [9000, 3100], [140, 48], [9, 3]),
    synth.custom("off g8", 1, 16, 2, [6000], [93], [6]),
]


@pytest.mark.parametrize("spec", SPECS, ids=[s.name for s in SPECS])
def test_offload_fused_step(gpu, spec):
    compare_layouts(spec, gpu)


def test_offload_two_calls(gpu):
    compare_layouts(SPECS[1], gpu, fused=False)


def test_offload_config2_sampled(gpu):
    compare_layouts(synth.config(2), gpu, units=[(0, 0), (7, 7)])
