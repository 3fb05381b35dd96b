"""Full-size GPU parity on every unit of the four large workloads, through the
C ABI, including the benchmarked call's own fast path.

For configurations 2-5 (Llama-3.1-8B-shaped 32K batch 8, 128K batch 4,
1M batch 1, and 64 ragged sequences of 1K-64K) every (batch, KV head) unit
is compared with the CPU oracle:
  - key codes of every cached row, the summed Hamming scores and the selected
    indices: bit-exact;
  - attention outputs: max |gpu - oracle| <= 2e-2;
then the same step is run again without the scores output -- the kernel's
fast scoring path, the one the benchmark times -- with only the selection
written: its indices must equal the oracle's on every unit and its outputs
be bit-identical to the first run; finally with no debug output at all
(exactly the benchmarked call), outputs bit-identical again.

The cut of these selections falls inside a large tied score bucket (about
760 keys share the cut score at 128K context, of which about 410 are taken;
the HATA review's Referee Report, major comment 1, on ties in Algorithm 3's
TopK): the lowest-index rule decides which of them are selected, and only an
index-exact comparison of every unit shows that the GPU takes the same ones.
"""
from __future__ import annotations

import sys
import time

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


class OracleRefs:
    """Runs the oracle on each unit's prefilled rows as the workload generates
    them (the step's appended token is the last row of the context)."""

    def __init__(self, spec):
        self.spec = spec
        self.q = synth.gen_q(spec)
        self.w = synth.gen_w(spec)
        self.new = synth.gen_new_token(spec)
        self.refs = {}
        self.t0 = time.time()

    def __call__(self, b, kv, k, v):
        spec, G = self.spec, self.spec.G
        K = np.concatenate([k, self.new[0][b, 0, kv][None]], axis=0)
        V = np.concatenate([v, self.new[1][b, 0, kv][None]], axis=0)
        r = oracle.decode_unit(self.q[b, kv * G:(kv + 1) * G], self.w[kv], K, V, spec.topk[b])
        del r["qcodes"]
        self.refs[(b, kv)] = r
        n = len(self.refs)
        if spec.B * spec.Hkv <= 64 or n % 16 == 0 or n == spec.B * spec.Hkv:
            _say(f"[fullsize] {spec.name}: oracle {n}/{spec.B * spec.Hkv} units "
                 f"({time.time() - self.t0:.0f} s)")


def _check_all_units(spec, wl, refs, out, sel, sc):
    codes = wl.cache.codes.cpu().numpy().view(np.uint32)
    sel = sel.cpu().numpy()
    sc = sc.cpu().numpy().view(np.uint16)
    outf = out.float().cpu().numpy().astype(np.float64)
    G, worst = spec.G, 0.0
    for b in range(spec.B):
        L = spec.lengths[b]
        ke = max(0, min(spec.topk[b], wl.k_max, L))
        for kv in range(spec.Hkv):
            ref = refs[(b, kv)]
            got = codes[b, kv, :L]
            assert np.array_equal(got, ref["kcodes"]), \
                f"codes differ at unit {(b, kv)}: {int((got != ref['kcodes']).any(1).sum())} rows"
            assert np.array_equal(sc[b, kv, :L].astype(np.int32), ref["scores"]), \
                f"scores differ at unit {(b, kv)}"
            assert np.array_equal(sel[b, kv, :ke], ref["idx"]), f"selection differs at unit {(b, kv)}"
            assert np.all(sel[b, kv, ke:] == -1)
            err = float(np.abs(outf[b, kv * G:(kv + 1) * G] - ref["out"]).max())
            assert err <= OUT_TOL, f"output error {err} at unit {(b, kv)}"
            worst = max(worst, err)
    return worst


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_every_unit_and_the_fast_path(gpu, cfg):
    spec = synth.config(cfg)
    _say(f"[fullsize] {spec.name}: generating, uploading and running the oracle per unit")
    refs = OracleRefs(spec)
    wl = GpuWorkload(spec, gpu, extra_ctx=2, unit_hook=refs)
    assert len(refs.refs) == spec.B * spec.Hkv

    # 1. debug outputs: codes, scores, indices, outputs on every unit
    out1, sel1, sc1 = wl.step(debug=True)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    assert wl.cache.seq_len.cpu().tolist() == list(spec.lengths)
    worst = _check_all_units(spec, wl, refs.refs, out1, sel1, sc1)
    out1 = out1.clone()
    _say(f"[fullsize] {spec.name}: every unit exact, max output error {worst:.3e}")

    # 2. the fast scoring path (no scores output), selection written
    wl.reset_to_prefill()
    sel2 = torch.full_like(sel1, -7)
    wl.fused_step(sel_idx_out=sel2)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    s2 = sel2.cpu().numpy()
    for b in range(spec.B):
        ke = max(0, min(spec.topk[b], wl.k_max, spec.lengths[b]))
        for kv in range(spec.Hkv):
            assert np.array_equal(s2[b, kv, :ke], refs.refs[(b, kv)]["idx"]), \
                f"fast-path selection differs at unit {(b, kv)}"
            assert np.all(s2[b, kv, ke:] == -1)
    assert torch.equal(wl.out.view(torch.int16), out1.view(torch.int16))

    # 3. exactly the benchmarked call: no debug output at all
    wl.reset_to_prefill()
    wl.fused_step()
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    assert torch.equal(wl.out.view(torch.int16), out1.view(torch.int16))
    assert wl.cache.seq_len.cpu().tolist() == list(spec.lengths)
    _say(f"[fullsize] {spec.name}: fast path indices exact on every unit, outputs bit-identical")
