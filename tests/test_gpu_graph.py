"""The decode step captured in a HIP graph (the boundary allocates nothing,
never synchronises and launches only on the given stream): every replay
equals the same step run eagerly on a twin workload -- outputs, selection,
codes and lengths bit-identical -- with eager work and synchronisations
between the replays, at two code lengths (one kernel serves every length).
"""
from __future__ import annotations

import pytest
import torch

import synth
from workload import GpuWorkload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_bits", [128, 64])
def test_decode_step_graph_replays_match_eager(gpu, n_bits):
    spec = synth.custom("graph", 2, 8, 2, [9000, 3100], [140, 48], [9, 3], seed=41)
    g_wl = GpuWorkload(spec, gpu, extra_ctx=8, n_bits=n_bits)
    e_wl = GpuWorkload(spec, gpu, extra_ctx=8, n_bits=n_bits)
    sel_g, sc_g = g_wl.debug_buffers()
    sel_e, sc_e = e_wl.debug_buffers()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_wl.fused_step(sel_idx_out=sel_g, scores_out=sc_g)
    torch.cuda.synchronize()
    # capture records the launch; the cache is untouched until a replay
    assert g_wl.cache.seq_len.cpu().tolist() == [n - 1 for n in spec.lengths]
    for r in range(4):
        graph.replay()
        e_wl.fused_step(sel_idx_out=sel_e, scores_out=sc_e)
        torch.cuda.synchronize()
        assert torch.equal(g_wl.out.view(torch.int16), e_wl.out.view(torch.int16)), r
        assert torch.equal(sel_g, sel_e) and torch.equal(sc_g, sc_e), r
        assert torch.equal(g_wl.cache.seq_len, e_wl.cache.seq_len), r
        assert torch.equal(g_wl.cache.codes, e_wl.cache.codes), r
        assert g_wl.cache.status() == 0 and e_wl.cache.status() == 0
    assert g_wl.cache.seq_len.cpu().tolist() == [n + 3 for n in spec.lengths]
