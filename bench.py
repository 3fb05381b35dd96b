"""Decode-step benchmark of hashed top-k attention on one MI355X.

Workload: the long-context decode configuration -- batch 4, 32 query / 8 KV
heads (GQA 4:1), head_dim 128, context 131072, top-k 2048 (1.56 %), r = 128
bits, 0.1 % planted aligned keys, seed 0 (synthetic inputs from synth/).

One step = one attention layer's decode step through hata_decode_step: the
append of one new token per sequence (K/V row copy + its code), query codes,
Hamming scan, top-k select, gather + softmax attention -- one kernel launch.  Steps cycle over
LAYERS independent layer caches (same contents, distinct memory), as a model
visits its layers, so the 256 MB last-level cache cannot hold the scanned
codes between two visits of the same layer, and over QUERIES step queries
(step 0's is the one the planted keys align with; the others are fresh
draws), so the gathered rows change from visit to visit.

Prints one JSON line.  value = decode steps per second on one GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
LAYERS = 8
QUERIES = 7  # distinct step queries, coprime with LAYERS: 56 (layer, query) pairs
COPY_PROBE_BYTES = 256 << 20
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_decode_fused_cfg3_hbm_traffic.md")
DECODE_SOURCES = ("decode.hip", "device_util.h", "hata_internal.h")
DECODE_KERNEL = "k_decode_fused<4>"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with 4 plain 256 MiB device-to-device copies (the "
                         "calibration kernel for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic block from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --copy-probe' runs, then exit")
    return ap.parse_args()


def algorithmic_bytes(B, Hq, Hkv, n_ctx, k):
    """Bytes the method must move for one decode step: every cached code
    (16 B per key per KV head), the selected K and V rows (512 B per
    selected key per KV head), W_H, q and the output, plus the append (one
    K and V row and one code per sequence and KV head)."""
    return (16 * B * Hkv * n_ctx + 512 * B * Hkv * k + 4 * Hkv * 128 * 128 +
            2 * 2 * B * Hq * 128 + B * Hkv * (512 + 16))


def decode_sources_digest():
    """sha256 over the decode kernel's sources: a traffic figure taken from
    counters is only reported for the kernel it was measured on."""
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "hash_top_sparse_encode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _pmc_per_dispatch(path):
    """{kernel name: [counter value per dispatch, in dispatch order]}."""
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    out = {}
    for r in rows:
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_csv, write_csv):
    """Key: value lines for the traffic profile.  The decode kernel's
    counters are the median over its dispatches (the run also makes one
    decode call with the debug outputs, which writes the scores); the
    calibration copy is the
    last 4 __amd_rocclr_copyBuffer dispatches (bench.py --copy-probe ends
    with 4 copies of COPY_PROBE_BYTES)."""
    vals = {}
    for counter, path in (("fetch", fetch_csv), ("write", write_csv)):
        per = _pmc_per_dispatch(path)
        dec = [v for k, v in per.items() if DECODE_KERNEL in k]
        cp = [v for k, v in per.items() if "copyBuffer" in k]
        if len(dec) != 1 or len(cp) != 1 or len(cp[0]) < 4:
            raise SystemExit(f"{path}: expected one decode kernel and >= 4 copies")
        vals[f"decode_{counter}_kib_per_dispatch"] = statistics.median(dec[0])
        vals[f"decode_{counter}_dispatches"] = len(dec[0])
        vals[f"copy_{counter}_kib"] = statistics.mean(cp[0][-4:])
    lines = [f"decode_sources_sha256: {decode_sources_digest()}",
             f"copy_bytes: {COPY_PROBE_BYTES}"]
    lines += [f"{k}: {v}" for k, v in vals.items()]
    return "\n".join(lines)


def measured_traffic_bytes():
    """HBM bytes per decode launch from the committed counter summary:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) each scaled by copy_bytes
    over what the same counter reads for the calibration copy.  None when
    the summary is missing or the decode sources changed since."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^([a-z0-9_]+): (\S+)$", text, flags=re.M))
    try:
        if vals["decode_sources_sha256"] != decode_sources_digest():
            return None
        cb = float(vals["copy_bytes"])
        total = 0.0
        for c in ("fetch", "write"):
            scale = cb / (float(vals[f"copy_{c}_kib"]) * 1024.0)
            total += float(vals[f"decode_{c}_kib_per_dispatch"]) * 1024.0 * scale
        return total
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def cpu_baseline(spec, reps):
    """The CPU oracle's decode step (query codes, bit-by-bit Hamming over the
    cached key codes, sort-based top-k, double-precision attention) on every
    (batch, KV head) unit of the same workload, units spread over a thread
    pool.  Key codes come from the oracle's own encoder (untimed prefill)."""
    import numpy as np
    import oracle
    import synth
    q = synth.gen_q(spec)
    w = synth.gen_w(spec)
    new = synth.gen_new_token(spec)
    cores = max(1, min(16, os.cpu_count() or 1))
    units = [(b, kv) for b in range(spec.B) for kv in range(spec.Hkv)]
    ctx = {}

    def prep(u):
        b, kv = u
        K, V = synth.unit_context(spec, b, kv, q, new)
        kc = oracle.encode(K, w[kv], threads=1)
        ctx[u] = (K, V, kc)

    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(prep, units))
    G = spec.G

    def decode(u):
        b, kv = u
        K, V, kc = ctx[u]
        oracle.decode_unit(q[b, kv * G:(kv + 1) * G], w[kv], K, V, spec.topk[b], kcodes=kc,
                           threads=1)

    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(cores) as ex:
            list(ex.map(decode, units))
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    # The same step on one core, and the oracle's key encoder on its own
    # (one unit's prefilled rows, all threads): the encode is not part of a
    # decode step, so it is reported beside it.
    t0 = time.perf_counter()
    for u in units:
        decode(u)
    t_one = time.perf_counter() - t0
    K0 = ctx[units[0]][0]
    t0 = time.perf_counter()
    oracle.encode(K0, w[0], threads=cores)
    t_enc = time.perf_counter() - t0
    return {"value": 1.0 / t, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"full decode step (all {len(units)} (batch, KV head) units, context "
                      f"{spec.lengths[0]}, top-k {spec.topk[0]}), median of {reps} runs; "
                      f"{cores} threads over units",
            "one_core_steps_per_s": 1.0 / t_one,
            "encode_rows_per_s": K0.shape[0] / t_enc,
            "encode_sample": f"oracle key encode of one unit's {K0.shape[0]} rows on "
                             f"{cores} threads",
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path "
              "has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import hash_top_sparse_encode_amd as hata
    import synth
    from workload import GpuWorkload

    dev = torch.device("cuda:0")
    spec = synth.config(3)
    B, Hq, Hkv, N, K = spec.B, spec.Hq, spec.Hkv, spec.lengths[0], spec.topk[0]
    L = max(1, args.layers)
    # room for every append: the layer steps, and up to 58 steps each on the
    # offloaded and other-code-length caches (which start from the prefill)
    per_layer = max(math.ceil((args.warmup + 2 * args.steps) / L) + 2, 64)
    print(f"[bench] generating {spec.name}", file=sys.stderr, flush=True)
    base = GpuWorkload(spec, dev, extra_ctx=per_layer)
    torch.cuda.synchronize()
    print("[bench] prefill encoded; replicating layers", file=sys.stderr, flush=True)

    class Layer:
        pass

    layers = []
    for i in range(L):
        ly = Layer()
        if i == 0:
            ly.cache = base.cache
            ly.ws = base.ws
        else:
            ly.cache = hata.HataCache(B, Hq, Hkv, base.max_ctx, device=dev,
                                      k=base.cache.k.clone(), v=base.cache.v.clone(),
                                      codes=base.cache.codes.clone(),
                                      seq_len=base.cache.seq_len.clone())
            ly.ws = hata.alloc_workspace(ly.cache, base.k_max)
        ly.out = torch.empty_like(base.out)
        layers.append(ly)
    for ly in layers:
        ly.cache.seq_len.copy_(base.n_pre)
    torch.cuda.synchronize()

    k_new = base.k_new.view(B, Hkv, 128)
    v_new = base.v_new.view(B, Hkv, 128)
    # A different query at each step, as in decoding, so that consecutive
    # visits of a layer select different rows.
    from workload import bf16_dev
    queries = [base.q] + [bf16_dev(synth.gen_q(spec, i), dev) for i in range(1, QUERIES)]

    def step(s):
        ly = layers[s % L]
        hata.hata_decode_step(ly.cache, k_new, v_new, queries[s % QUERIES], base.w, base.topk,
                              base.k_max, ly.out, ly.ws)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    ctx0 = int(layers[args.warmup % L].cache.seq_len[0].item()) + 1
    # HIP events on the launch stream bracket the timed region: the decode
    # kernel is the only work in it, one launch per step, so their interval
    # over the step count is the kernel's average launch duration (with the
    # gaps between back-to-back launches).
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for s in range(args.steps):
        step(args.warmup + s)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    ms_per_step = wall * 1e3 / args.steps
    steps_per_s = args.steps / wall
    dec_ms = ev0.elapsed_time(ev1) / args.steps
    # Spread of single steps: one event pair per step over a second pass
    # (the pairs add small gaps, so this pass is not the headline).
    n_dist = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_dist)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(args.warmup + args.steps + i)
        b.record(stream)
    torch.cuda.synchronize()
    step_us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)

    def pct(p):
        return step_us[min(len(step_us) - 1, int(p * len(step_us)))]

    # Device-to-device copy bandwidth in the same run: the practical
    # streaming rate the step's bytes can be set against.
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    status = [ly.cache.status() for ly in layers]
    if any(status):
        print(f"[bench] device status flags set: {status}", file=sys.stderr)
        sys.exit(1)

    # The prefill encode of the same workload (hata_append over the N - 1
    # prefilled rows of every sequence, codes computed in place): events
    # around each call, after one warm-up.
    enc_ms = []
    for r in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        base.encode_prefill()
        e1.record(stream)
        torch.cuda.synchronize()
        if r > 0:
            enc_ms.append(e0.elapsed_time(e1))
    enc_rows = B * Hkv * (N - 1)
    enc_s = statistics.mean(enc_ms) * 1e-3
    prefill = {
        "what": "hata_append encoding the N - 1 prefilled rows of every (sequence, KV head) "
                "in place (one launch)",
        "rows": enc_rows,
        "ms": enc_s * 1e3,
        "Mrows_per_s": enc_rows / enc_s / 1e6,
        "hbm_GBps": enc_rows * (256 + 16) / enc_s / 1e9,
        "useful_TFLOPs": enc_rows * 2 * 128 * 128 / enc_s / 1e12,
        "mfma_TFLOPs": enc_rows * 2 * 2 * 128 * 128 / enc_s / 1e12,
        "mfma_peak_TFLOPs": 2500.0,
    }

    # The recall analysis of one decode call (layer 0, step query 0, no
    # append): each query head's exact top-k against its group's Hamming
    # selection, and the tie bucket at the cut.
    ly = layers[0]
    sel = torch.empty((B, Hkv, base.k_max), dtype=torch.int32, device=dev)
    sc = torch.empty((B, Hkv, base.max_ctx), dtype=torch.int16, device=dev)
    hata.hata_decode_attn(ly.cache, queries[0], base.w, base.topk, base.k_max, ly.out, ly.ws,
                          sel_idx_out=sel, scores_out=sc)
    rws = hata.alloc_recall_workspace(ly.cache)
    ov = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    tie = torch.empty((B, Hkv, 4), dtype=torch.int32, device=dev)
    rec_ms = []
    for r in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        hata.hata_exact_topk_recall(ly.cache, queries[0], base.topk, base.k_max, sel, sc, rws,
                                    overlap_out=ov, tie_out=tie)
        e1.record(stream)
        torch.cuda.synchronize()
        if r > 0:
            rec_ms.append(e0.elapsed_time(e1))
    rec_ctx = int(ly.cache.seq_len[0].item())
    tie_h = tie.cpu().numpy().astype(float)
    ov_h = ov.cpu().numpy().astype(float)
    k_eff = tie_h[..., 3]
    rec_s = statistics.mean(rec_ms) * 1e-3
    recall = {
        "what": "hata_exact_topk_recall after one decode call on the same cache: each query "
                "head's exact top-k by q.k against its group's Hamming selection, and the "
                "tie bucket at the selection's cut",
        "context": rec_ctx,
        "ms": rec_s * 1e3,
        "key_rows_GBps": B * Hkv * rec_ctx * 256 / rec_s / 1e9,
        "overlap_frac": float(ov_h.sum() / (k_eff.sum() * (Hq // Hkv))),
        "overlap_frac_min_head": float((ov_h / np.repeat(k_eff, Hq // Hkv, axis=1)).min()),
        "cut_T_mean": float(tie_h[..., 0].mean()),
        "below_cut_mean": float(tie_h[..., 1].mean()),
        "tied_at_cut_mean": float(tie_h[..., 2].mean()),
        "taken_from_tie_mean": float((k_eff - tie_h[..., 1]).mean()),
    }
    del rws

    # The offloaded layout: the same workload with the K/V rows in pinned host
    # memory (codes, workspace and queries stay in device memory); each step
    # reads its selected rows, and writes its appended ones, over the host link.
    off = hata.HataCache(B, Hq, Hkv, base.max_ctx, device=dev, offload=True,
                         codes=base.cache.codes.clone(), seq_len=base.n_pre.clone())
    off.k.copy_(base.cache.k)
    off.v.copy_(base.cache.v)
    off_ws = hata.alloc_workspace(off, base.k_max)
    off_out = torch.empty_like(base.out)

    def off_step(s):
        hata.hata_decode_step(off, k_new, v_new, queries[s % QUERIES], base.w, base.topk,
                              base.k_max, off_out, off_ws)

    n_off = max(1, min(args.steps, 50))
    for s in range(8):
        off_step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(n_off):
        off_step(8 + s)
    torch.cuda.synchronize()
    off_s = (time.perf_counter() - t0) / n_off
    if off.status():
        print(f"[bench] offload status flags set: {off.status()}", file=sys.stderr)
        sys.exit(1)
    offload = {
        "what": "hata_decode_step with the K/V cache in pinned host memory (codes in HBM)",
        "steps": n_off,
        "steps_per_s": 1.0 / off_s,
        "us_per_step": off_s * 1e6,
        "selected_rows_GBps": B * Hkv * K * 512 / off_s / 1e9,
        "vs_device_resident": (1.0 / off_s) / steps_per_s,
    }
    del off, off_ws

    # Other code lengths (the hash-length ablation): the same workload with
    # r-bit codes over the same K/V rows, one cache (the codes of r = 32 and
    # 64 bits, 17 and 34 MB, fit in the last-level cache, so they are
    # flattered), prefill encode in place, then decode steps on the
    # multi-launch path.
    code_lengths = []
    for r in (32, 64, 256):
        w_r = torch.from_numpy(synth.gen_w_bits(spec, r)).to(dev)
        c_r = hata.HataCache(B, Hq, Hkv, base.max_ctx, device=dev, k=base.cache.k,
                             v=base.cache.v, n_bits=r)
        enc_t = []
        for rep_i in range(2):
            c_r.seq_len.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            hata.hata_append(c_r, None, None, base.n_pre, N - 1, w_r)
            e1.record(stream)
            torch.cuda.synchronize()
            enc_t.append(e0.elapsed_time(e1))
        ws_r = hata.alloc_workspace(c_r, base.k_max)
        out_r = torch.empty_like(base.out)

        def step_r(s):
            hata.hata_decode_step(c_r, k_new, v_new, queries[s % QUERIES], w_r, base.topk,
                                  base.k_max, out_r, ws_r)

        for s in range(5):
            step_r(s)
        n_r = max(1, min(args.steps, 30))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(n_r):
            step_r(5 + s)
        e1.record(stream)
        torch.cuda.synchronize()
        if c_r.status():
            print(f"[bench] r={r}: device status flags set: {c_r.status()}", file=sys.stderr)
            sys.exit(1)
        us = e0.elapsed_time(e1) * 1e3 / n_r
        ctx_r = N + 5 + (n_r - 1) / 2.0  # mean context of the timed steps
        alg_r = (r // 8) * B * Hkv * ctx_r + 512 * B * Hkv * K + 4 * Hkv * 128 * r + \
            4 * B * Hq * 128 + B * Hkv * (512 + r // 8)
        code_lengths.append({"n_bits": r, "us_per_step": us, "steps_per_s": 1e6 / us,
                             "alg_bytes": alg_r, "alg_GBps": alg_r / us / 1e3,
                             "prefill_encode_ms": enc_t[-1]})
        del c_r, ws_r
    base.cache.seq_len.copy_(base.n_pre)

    n_ctx = ctx0 + (args.steps // L) / 2.0  # mean context over the timed steps
    step_bytes = algorithmic_bytes(B, Hq, Hkv, n_ctx, K)
    achieved = step_bytes / (dec_ms * 1e-3) / 1e9
    traffic_bytes = measured_traffic_bytes()

    result = {
        "metric": "decode steps/sec & HBM GB/s fraction, hashed top-k attn @128K ctx, 1 GPU",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "bf16 K/V/q/out, fp32 W_H and accumulation, u32 codes",
        "data": "synthetic (seeded SplitMix64/Box-Muller; N(0,1) K/V/q, N(0,1/128) W_H, "
                "0.1% planted aligned keys)",
        "config": {
            "workload": "hashed top-k decode step: B=4, Hq=32, Hkv=8, d=128, r=128, "
                        f"context {N} (+{args.steps // L} appended), top-k {K}, "
                        f"{L} layer caches visited in turn, {QUERIES} step queries",
            "tokens_per_s": steps_per_s * B,
            "us_per_step": ms_per_step * 1e3,
            "step_alg_bytes": step_bytes,
            "step_hbm_frac": step_bytes * steps_per_s / (HBM_PEAK_GBS * 1e9),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_decode_fused<4> (hata_decode_step: append, query codes, Hamming "
                      "scan, select, gather-attention, merge)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (traffic_bytes / (dec_ms * 1e-3) / 1e9
                        if traffic_bytes is not None else None),
            "traffic_bytes_per_launch": traffic_bytes,
            "alg_bytes_per_launch": step_bytes,
            "launch_us": dec_ms * 1e3,
            "copy_GBps": copy_gbs,
            "frac_of_copy": achieved / copy_gbs,
        },
        "step_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9),
                    "steps": n_dist, "how": "one HIP event pair per step, second pass"},
        "prefill_encode": prefill,
        "recall": recall,
        "offload": offload,
        "code_lengths": code_lengths,
    }
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(7)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(spec, args.cpu_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
