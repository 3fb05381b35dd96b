"""The decode step's stall path: every cross-workgroup wait of the fused
128-bit kernel is bounded, and a wait that gives up sets HATA_DEV_STALL
(include/hata.h).  The host forces the waits to give up almost at once
(HATA_DECODE_WAIT_LIMIT=0, the library's test control), so every kernel still
runs to its normal end; then the documented recovery -- a zero-filled
workspace, the status bit cleared, hata_decode_attn again -- must give
results bit-identical to an undisturbed step.
"""
from __future__ import annotations

import torch
import pytest

import hash_top_sparse_encode_amd as hata
import synth
from workload import GpuWorkload

pytestmark = pytest.mark.gpu


STALL_SPECS = [
    synth.custom("stall", 2, 8, 2, [20000, 9000], [300, 140], [20, 9], seed=13),
    # 256 units of two or three items each: more workgroups than the chip
    # holds at once, so the grid runs in the unit-by-unit order
    synth.custom("stall, grid larger than the chip", 32, 32, 8, [9000 if b % 2 else 13000 for b in range(32)],
                 [140 if b % 2 else 200 for b in range(32)], [9 if b % 2 else 13 for b in range(32)], seed=17),
]


@pytest.mark.parametrize("spec", STALL_SPECS, ids=[s.name for s in STALL_SPECS])
def test_forced_stall_sets_status_and_recovers(gpu, monkeypatch, spec):
    clean = GpuWorkload(spec, gpu, extra_ctx=2)
    out_c, sel_c, sc_c = clean.step(debug=True)
    torch.cuda.synchronize()
    assert clean.cache.status() == 0
    out_c = out_c.clone()

    wl = GpuWorkload(spec, gpu, extra_ctx=2)
    print("[stall] fused step with the waits capped at 0 re-reads", flush=True)
    monkeypatch.setenv("HATA_DECODE_WAIT_LIMIT", "0")
    wl.fused_step()
    monkeypatch.delenv("HATA_DECODE_WAIT_LIMIT")
    torch.cuda.synchronize()
    st = wl.cache.status()
    assert st & hata.HATA_DEV_STALL, f"status {st:#x}: no wait gave up"
    assert st & ~hata.HATA_DEV_STALL == 0
    # the cache itself is valid: appended rows, their codes, the lengths
    assert torch.equal(wl.cache.seq_len, clean.cache.seq_len)
    assert torch.equal(wl.cache.codes, clean.cache.codes)
    assert torch.equal(wl.cache.k, clean.cache.k) and torch.equal(wl.cache.v, clean.cache.v)

    # recovery: zero-filled workspace, status cleared, decode again
    wl.ws.zero_()
    wl.cache.ctrl[0] = 0
    sel, sc = wl.debug_buffers()
    wl.decode(sel_idx_out=sel, scores_out=sc)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    assert torch.equal(wl.out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(sel, sel_c) and torch.equal(sc, sc_c)
    # and the next steps on the recovered workspace run normally
    wl.reset_to_prefill()
    clean.reset_to_prefill()
    for _ in range(2):
        wl.fused_step()
        clean.fused_step()
        torch.cuda.synchronize()
        assert wl.cache.status() == 0 and clean.cache.status() == 0
        assert torch.equal(wl.out.view(torch.int16), clean.out.view(torch.int16))
        wl.reset_to_prefill()
        clean.reset_to_prefill()
