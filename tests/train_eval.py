"""Train W_H on the GPU and measure what it buys: the recall test of the HATA
review ("What would settle it": how much of each query's exact top-k the
Hamming selection finds), with a random W_H and with the trained one, on a
held-out cache drawn from the same structured q/k distribution
(synth.gen_structured_qk).  Shared by the GPU tests and the bench; all
arithmetic runs in the library's kernels (hata_hash_labels,
hata_hash_train_step, hata_append, hata_decode_attn, hata_exact_topk_recall).
"""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import hash_top_sparse_encode_amd as hata
import synth
from workload import bf16_dev

SEED = 0
N_Q, N_K = 256, 4096      # training batch: 1M (query, key) pairs
NEW_BATCH_EVERY = 10      # steps per batch


def initial_w(n_bits: int = 128) -> np.ndarray:
    """The random projection training starts from (and the baseline):
    N(0, 1/128) fp32 [128][n_bits]."""
    return synth.normal_f32(SEED, synth.T_W, 0, 128 * n_bits, 1.0 / math.sqrt(128)).reshape(128, n_bits)


def train(device, steps: int, lr: float = 0.01, n_bits: int = 128, log=None):
    """Adam steps from initial_w(); a new batch of structured queries and keys
    (and its labels) every NEW_BATCH_EVERY steps.  Returns (W, losses, ms per
    step, ms per label batch)."""
    tr = hata.HashTrainer(torch.from_numpy(initial_w(n_bits)).to(device), N_Q, N_K,
                          hata.TrainParams(lr=lr))
    losses, t_step, t_lab = [], [], []
    stream = torch.cuda.current_stream()
    for s in range(steps):
        if s % NEW_BATCH_EVERY == 0:
            q, k = synth.gen_structured_qk(SEED, s // NEW_BATCH_EVERY, N_Q, N_K)
            qd, kd = bf16_dev(q, device), bf16_dev(k, device)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lab = hata.hata_hash_labels(qd, kd)
            e1.record(stream)
            t_lab.append((e0, e1))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        loss = tr.step(qd, kd, lab)
        e1.record(stream)
        t_step.append((e0, e1))
        if s % 50 == 0 or s == steps - 1:
            losses.append((s, loss.cpu().tolist()))
            if log:
                log(f"[train] step {s}: loss {losses[-1][1]}")
    torch.cuda.synchronize()
    ms_step = float(np.median([a.elapsed_time(b) for a, b in t_step]))
    ms_lab = float(np.median([a.elapsed_time(b) for a, b in t_lab]))
    return tr.w.clone(), losses, ms_step, ms_lab


def eval_cache(device, n_ctx: int = 32768, heads: int = 8):
    """A held-out cache: one sequence, `heads` KV heads with one query head
    each, keys and queries from blocks of the structured distribution that
    training never draws (blocks 10^6 + head)."""
    cache = hata.HataCache(1, heads, heads, n_ctx, device=device)
    q = np.zeros((1, heads, 128), dtype=np.uint16)
    for h in range(heads):
        qh, kh = synth.gen_structured_qk(SEED, 10 ** 6 + h, 1, n_ctx)
        q[0, h] = qh[0]
        cache.k[0, h] = bf16_dev(kh, device)
    cache.v.copy_(bf16_dev(synth.normal_bf16(SEED, synth.T_V, 0, heads * n_ctx * 128)
                           .reshape(1, heads, n_ctx, 128), device))
    return cache, bf16_dev(q, device)


def recall(cache, q, w: torch.Tensor, k: int):
    """Encode the cache under W_H = w (every head), decode with budget k and
    return (mean overlap fraction with the exact top-k, tie bucket means)."""
    heads, n_ctx = cache.n_kv_heads, cache.max_ctx
    wh = w.reshape(1, 128, -1).expand(heads, 128, w.shape[-1]).contiguous()
    cache.seq_len.zero_()
    n = torch.full((1,), n_ctx, dtype=torch.int32, device=q.device)
    hata.hata_append(cache, None, None, n, n_ctx, wh)
    topk = torch.full((1,), k, dtype=torch.int32, device=q.device)
    out = torch.empty((1, heads, 128), dtype=torch.bfloat16, device=q.device)
    ws = hata.alloc_workspace(cache, k)
    sel = torch.empty((1, heads, k), dtype=torch.int32, device=q.device)
    sc = torch.empty((1, heads, n_ctx), dtype=torch.int16, device=q.device)
    hata.hata_decode_attn(cache, q, wh, topk, k, out, ws, sel_idx_out=sel, scores_out=sc)
    ov = torch.empty((1, heads), dtype=torch.int32, device=q.device)
    tie = torch.empty((1, heads, 4), dtype=torch.int32, device=q.device)
    hata.hata_exact_topk_recall(cache, q, topk, k, sel, sc, hata.alloc_recall_workspace(cache),
                                overlap_out=ov, tie_out=tie)
    torch.cuda.synchronize()
    assert cache.status() == 0
    t = tie.cpu().numpy().astype(float)[0]
    return float(ov.cpu().numpy().sum() / (heads * k)), {
        "cut_T_mean": float(t[:, 0].mean()), "below_cut_mean": float(t[:, 1].mean()),
        "tied_at_cut_mean": float(t[:, 2].mean())}
