"""GPU parity of the decode step against the CPU oracle, through the C ABI.

Bars (per unit (batch, KV head) checked):
  - key codes, query-group Hamming scores and selected indices: bit-exact;
  - attention outputs: max |gpu - oracle| <= 2e-2 (bf16 output, fp32
    accumulation; the oracle is exact double precision).
Small and fuzzed workloads are checked unit by unit in full here; the
full-size configurations, every unit of them, in test_gpu_fullsize.py.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from workload import GpuWorkload, bf16_bits

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_unit(spec, wl, b, kv):
    K, V = synth.unit_context(spec, b, kv, wl.q_host, wl.new_host)
    G = spec.G
    return oracle.decode_unit(wl.q_host[b, kv * G:(kv + 1) * G], wl.w_host[kv], K, V,
                              spec.topk[b])


def k_eff_of(spec, b, k_max):
    return max(0, min(spec.topk[b], k_max, spec.lengths[b]))


def check_unit(spec, wl, b, kv, out, sel, sc, ref=None):
    G = spec.G
    L = spec.lengths[b]
    ref = ref if ref is not None else oracle_unit(spec, wl, b, kv)
    codes = wl.cache.codes[b, kv, :L].cpu().numpy().view(np.uint32)
    assert np.array_equal(codes, ref["kcodes"]), f"codes differ at unit {(b, kv)}: " \
        f"{int((codes != ref['kcodes']).any(1).sum())} rows"
    scores = sc[b, kv, :L].cpu().numpy().view(np.uint16).astype(np.int32)
    assert np.array_equal(scores, ref["scores"]), f"scores differ at unit {(b, kv)}"
    ke = k_eff_of(spec, b, wl.k_max)
    s = sel[b, kv].cpu().numpy()
    assert np.array_equal(s[:ke], ref["idx"]), f"selection differs at unit {(b, kv)}"
    assert np.all(s[ke:] == -1)
    o = out[b, kv * G:(kv + 1) * G].float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ref["out"]).max()
    assert err <= OUT_TOL, f"output error {err} at unit {(b, kv)}"
    return err


def check_structure(spec, wl, sel):
    s = sel.cpu().numpy()
    for b in range(spec.B):
        ke = k_eff_of(spec, b, wl.k_max)
        for kv in range(spec.Hkv):
            row = s[b, kv]
            assert np.all(row[ke:] == -1)
            head = row[:ke]
            assert np.all(np.diff(head) > 0) and (ke == 0 or (head[0] >= 0 and head[-1] < spec.lengths[b]))


def run_spec(spec, device, units=None, extra_ctx=3, fused=True):
    _say(f"[parity] {spec.name}: generating + prefill")
    wl = GpuWorkload(spec, device, extra_ctx=extra_ctx)
    out, sel, sc = wl.step(debug=True, fused=fused)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    assert wl.cache.seq_len.cpu().tolist() == list(spec.lengths)
    check_structure(spec, wl, sel)
    if units is None:
        units = [(b, kv) for b in range(spec.B) for kv in range(spec.Hkv)]
    errs = []
    for (b, kv) in units:
        _say(f"[parity] {spec.name}: oracle unit {(b, kv)} len {spec.lengths[b]}")
        errs.append(check_unit(spec, wl, b, kv, out, sel, sc))
    _say(f"[parity] {spec.name}: max out err {max(errs):.3e}")
    return wl, out, sel, sc


def test_config1_all_units(gpu):
    run_spec(synth.config(1), gpu)


FUZZ = [
    synth.custom("g1 len1 dense", 2, 3, 3, [1, 5000], [4, 5000], [0, 4]),
    synth.custom("g2 ragged k>len k=0", 3, 4, 2, [1030, 2049, 777], [16, 2054, 0], [2, 2, 1]),
    synth.custom("g4 ragged", 2, 8, 2, [9000, 3100], [140, 48], [9, 3]),
    synth.custom("g8", 1, 16, 2, [6000], [93], [6]),
    synth.custom("g4 tiny", 3, 4, 1, [2, 3, 64], [1, 3, 5], [1, 1, 1]),
]


@pytest.mark.parametrize("spec", FUZZ, ids=[s.name for s in FUZZ])
def test_fuzz_all_units(gpu, spec):
    run_spec(spec, gpu)


@pytest.mark.parametrize("spec", FUZZ[1:3], ids=[s.name for s in FUZZ[1:3]])
def test_fuzz_append_then_decode(gpu, spec):
    # the two-call path: hata_append (one token) then hata_decode_attn
    run_spec(spec, gpu, fused=False)


def test_fused_matches_two_calls(gpu):
    spec = synth.custom("paths", 3, 8, 4, [7000, 300, 12000], [100, 9, 180], [7, 1, 12], seed=9)
    a = GpuWorkload(spec, gpu, extra_ctx=2)
    b = GpuWorkload(spec, gpu, extra_ctx=2)
    oa, sa, ca = a.step(debug=True, fused=True)
    ob, sb, cb = b.step(debug=True, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(sa, sb) and torch.equal(ca, cb)
    assert torch.equal(a.cache.codes, b.cache.codes) and torch.equal(a.cache.k, b.cache.k)
    assert torch.equal(a.cache.v, b.cache.v)
    assert torch.equal(a.cache.seq_len, b.cache.seq_len)
    assert a.cache.status() == 0 and b.cache.status() == 0
    # counters are back at zero after each call
    assert int(a.cache.ctrl[1:].abs().sum().item()) == 0
    assert int(b.cache.ctrl[1:].abs().sum().item()) == 0


def test_workspace_shared_by_caches(gpu):
    # Caches (layers) whose calls are ordered may share one workspace: call
    # after call, alternating between two caches, the results equal those of
    # the same caches each with a workspace of its own.
    specs = [synth.custom(f"ws {i}", 2, 8, 2, [9000, 3100], [140, 48], [9, 3], seed=31 + i)
             for i in range(2)]
    own = [GpuWorkload(s, gpu, extra_ctx=4) for s in specs]
    shared = [GpuWorkload(s, gpu, extra_ctx=4) for s in specs]
    for w in shared[1:]:
        w.ws = shared[0].ws
    for r in range(3):
        for i in range(2):
            oa, sa, ca = own[i].step(debug=(r == 1))
            ob, sb, cb = shared[i].step(debug=(r == 1))
            torch.cuda.synchronize()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), (r, i)
            if r == 1:
                assert torch.equal(sa, sb) and torch.equal(ca, cb), (r, i)
            assert own[i].cache.status() == 0 and shared[i].cache.status() == 0


FAST = [synth.config(1), FUZZ[2], FUZZ[3],
        synth.custom("g4 long", 2, 8, 2, [40000, 17000], [625, 265], [40, 17], seed=21)]


@pytest.mark.parametrize("spec", FAST, ids=[s.name for s in FAST])
def test_step_without_debug_outputs_matches(gpu, spec):
    # Without the optional debug outputs the kernel takes its fast scoring
    # path; results must be bit-identical to the run that writes them.
    a = GpuWorkload(spec, gpu, extra_ctx=2)
    b = GpuWorkload(spec, gpu, extra_ctx=2)
    oa, _, _ = a.step(debug=True)
    ob, _, _ = b.step(debug=False)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(a.cache.codes, b.cache.codes)
    assert torch.equal(a.cache.k, b.cache.k) and torch.equal(a.cache.v, b.cache.v)
    assert torch.equal(a.cache.seq_len, b.cache.seq_len)
    assert a.cache.status() == 0 and b.cache.status() == 0


def test_many_units_dense_and_sparse(gpu):
    # 512 units, so each unit has a single split of up to 3000 keys; half the
    # sequences select everything (dense), which overflows the LDS index
    # list and exercises its flush.
    B = 32
    lens = synth.ragged_lengths(11, B, 1500, 3000)
    topk = [n if b % 2 == 0 else max(16, n // 64) for b, n in enumerate(lens)]
    spec = synth.custom("many units", B, 16, 16, lens, topk, [3] * B, seed=11)
    run_spec(spec, gpu, units=[(0, 0), (0, 15), (1, 3), (30, 7), (31, 0)])


def _bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """bf16 bits of float32 values that are exactly representable in bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("n_bits", [128, 256, 32])
def test_query_codes_in_band(gpu, n_bits):
    # Code bits whose sum x . W_j is zero or tiny next to A = sum_t |x_t W_tj|
    # cannot be decided by the kernel's fp32 sum and go to the defining
    # sequential double sum.  W's rows 2i and 2i + 1 agree in every even
    # column, and the query heads and the step's new keys are antisymmetric
    # over those pairs (x_{2i+1} = -x_{2i}, |x| in [1, 16)), so their even
    # bits sum to exactly zero (bit 0); every other head, and the second
    # batch entry's new keys, carry one imbalance, x_1 = -(1 - 2^-8) against
    # x_0 = 1, which leaves a sum of 2^-8 W_1j against an A near 2^10 |W|.
    spec = synth.custom("in band", 2, 8, 2, [5000, 1200], [64, 16], [5, 2], seed=13)
    # (at 256 bits each query-code part decides two groups of 32 columns,
    # the second after the first)
    wl = GpuWorkload(spec, gpu, extra_ctx=2, encode_prefill=False, n_bits=n_bits)
    q_keys = wl.q_host.copy()  # the keys of the context were planted from these
    w = wl.w_host.copy()
    w[:, 1::2, 0::2] = w[:, 0::2, 0::2]
    rng = np.random.default_rng(13)

    def pairs(shape, imbalance):
        mag = ((1.0 + rng.integers(0, 128, size=shape + (64,)) / 128.0)
               * 2.0 ** rng.integers(0, 4, size=shape + (64,))).astype(np.float32)
        sign = np.where(rng.random(shape + (64,)) < 0.5, -1.0, 1.0).astype(np.float32)
        x = np.empty(shape + (128,), dtype=np.float32)
        x[..., 0::2] = mag * sign
        x[..., 1::2] = -mag * sign
        x[..., 0] = np.where(imbalance, 1.0, x[..., 0])
        x[..., 1] = np.where(imbalance, -(1.0 - 2.0 ** -8), x[..., 1])
        return _bf16_bits_of(x)

    heads = np.arange(spec.Hq) % 2 == 1
    q = pairs((spec.B, spec.Hq), np.broadcast_to(heads, (spec.B, spec.Hq)))
    kn = pairs((spec.B, 1, spec.Hkv),
               np.broadcast_to((np.arange(spec.B) == 1)[:, None, None], (spec.B, 1, spec.Hkv)))
    new = (kn, wl.new_host[1])
    wl.w_host, wl.q_host, wl.new_host = w, q, new
    wl.w = torch.from_numpy(w).to(gpu)
    wl.q = torch.from_numpy(q.view(np.int16)).to(gpu).view(torch.bfloat16)
    wl.k_new = torch.from_numpy(kn.view(np.int16)).to(gpu).view(torch.bfloat16)
    wl.encode_prefill()
    out, sel, sc = wl.step(debug=True)
    torch.cuda.synchronize()
    assert wl.cache.status() == 0
    G = spec.G
    for b in range(spec.B):
        for kv in range(spec.Hkv):
            K, V = synth.unit_context(spec, b, kv, q_keys, new)
            ref = oracle.decode_unit(q[b, kv * G:(kv + 1) * G], w[kv], K, V, spec.topk[b])
            # the even bits of the antisymmetric vectors are all zero
            qc = oracle.encode(q[b, kv * G:(kv + 1) * G], w[kv])
            even = np.uint32(0x55555555)
            for h in range(G):
                if not heads[kv * G + h]:
                    assert not np.any(qc[h] & even)
            check_unit(spec, wl, b, kv, out, sel, sc, ref=ref)


def test_determinism(gpu):
    spec = synth.custom("det", 2, 8, 2, [20000, 7000], [300, 100], [20, 7], seed=5)
    wl = GpuWorkload(spec, gpu, extra_ctx=1)
    out1, sel1, sc1 = wl.step(debug=True)
    out1, sel1, sc1 = out1.clone(), sel1.clone(), sc1.clone()
    for _ in range(3):
        wl.decode()
        o2 = wl.out.clone()
        assert torch.equal(bf16_bits_t(o2), bf16_bits_t(out1))
    sel2 = torch.full_like(sel1, -7)
    sc2 = torch.zeros_like(sc1)
    wl.decode(sel_idx_out=sel2, scores_out=sc2)
    assert torch.equal(sel1, sel2) and torch.equal(sc1, sc2)
    assert torch.equal(bf16_bits_t(wl.out), bf16_bits_t(out1))


def bf16_bits_t(t):
    return t.view(torch.int16)
