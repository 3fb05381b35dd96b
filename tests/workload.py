"""Synthetic decode workloads on the GPU, built from the shared generator.

Fills a HataCache with the prefilled context of a synth.Spec (N_b - 1 rows
per sequence), encodes the prefilled keys through the library's own append
path (rows already in the cache), and runs the decode step
(hata_append of one token per sequence, then hata_decode_attn).
Used by the GPU tests and the bench; holds no method arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

import hash_top_sparse_encode_amd as hata
import synth


def bf16_dev(a: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> a bf16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class GpuWorkload:
    """Device state of one synthetic decode workload."""

    def __init__(self, spec: synth.Spec, device, extra_ctx: int = 0, units=None,
                 encode_prefill: bool = True, offload: bool = False, n_bits: int = 128,
                 unit_hook=None):
        """unit_hook(b, kv, k, v), if given, sees each unit's prefilled rows
        (host bf16 bits) as they are generated, so a caller can run the oracle
        on the very bytes uploaded without generating them twice."""
        self.spec = spec
        self.device = device
        B, Hq, Hkv = spec.B, spec.Hq, spec.Hkv
        self.max_ctx = max(spec.max_len + extra_ctx, 1)
        self.q_host = synth.gen_q(spec)
        self.n_bits = n_bits
        self.w_host = synth.gen_w(spec) if n_bits == 128 else synth.gen_w_bits(spec, n_bits)
        self.new_host = synth.gen_new_token(spec)
        self.cache = hata.HataCache(B, Hq, Hkv, self.max_ctx, device=device, offload=offload,
                                    n_bits=n_bits)
        self.cache.k.zero_()
        self.cache.v.zero_()
        for b in range(B):
            n_pre = spec.lengths[b] - 1
            for kv in range(Hkv):
                if n_pre > 0:
                    k = synth.gen_unit_k(spec, b, kv, self.q_host)
                    v = synth.gen_unit_v(spec, b, kv)
                    self.cache.k[b, kv, :n_pre] = bf16_dev(k, device)
                    self.cache.v[b, kv, :n_pre] = bf16_dev(v, device)
                    if unit_hook is not None:
                        unit_hook(b, kv, k, v)
                elif unit_hook is not None:
                    empty = np.zeros((0, 128), dtype=np.uint16)
                    unit_hook(b, kv, empty, empty)
        self.w = torch.from_numpy(self.w_host).to(device)
        self.q = bf16_dev(self.q_host, device)
        self.k_new = bf16_dev(self.new_host[0], device)
        self.v_new = bf16_dev(self.new_host[1], device)
        self.n_pre = torch.tensor([n - 1 for n in spec.lengths], dtype=torch.int32, device=device)
        self.ones = torch.ones(B, dtype=torch.int32, device=device)
        self.topk = torch.tensor(spec.topk, dtype=torch.int32, device=device)
        self.k_max = max(spec.k_max, 1)
        self.out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=device)
        self.ws = hata.alloc_workspace(self.cache, self.k_max)
        if encode_prefill:
            self.encode_prefill()

    def encode_prefill(self):
        """Codes of the prefilled rows through hata_append (encode in place)."""
        self.cache.seq_len.zero_()
        self.append_prefill()

    def append_prefill(self):
        """The hata_append call of encode_prefill, with seq_len already zero."""
        hata.hata_append(self.cache, None, None, self.n_pre, max(self.spec.max_len - 1, 0),
                         self.w)

    def reset_to_prefill(self):
        self.cache.seq_len.copy_(self.n_pre)

    def append_token(self):
        hata.hata_append(self.cache, self.k_new, self.v_new, self.ones, 1, self.w)

    def decode(self, sel_idx_out=None, scores_out=None, out=None):
        return hata.hata_decode_attn(self.cache, self.q, self.w, self.topk, self.k_max,
                                     self.out if out is None else out, self.ws,
                                     sel_idx_out=sel_idx_out, scores_out=scores_out)

    def fused_step(self, sel_idx_out=None, scores_out=None, out=None):
        return hata.hata_decode_step(self.cache, self.k_new, self.v_new, self.q, self.w,
                                     self.topk, self.k_max, self.out if out is None else out,
                                     self.ws, sel_idx_out=sel_idx_out, scores_out=scores_out)

    def debug_buffers(self):
        B, Hkv = self.spec.B, self.spec.Hkv
        sel = torch.full((B, Hkv, self.k_max), -7, dtype=torch.int32, device=self.device)
        sc = torch.zeros((B, Hkv, self.max_ctx), dtype=torch.int16, device=self.device)
        return sel, sc

    def step(self, debug: bool = False, fused: bool = True):
        """The decode step: append the step's token, then decode -- one fused
        launch (hata_decode_step) or hata_append + hata_decode_attn.  With
        debug, also return the selected indices and the scores."""
        sel, sc = self.debug_buffers() if debug else (None, None)
        if fused:
            self.fused_step(sel_idx_out=sel, scores_out=sc)
        else:
            self.append_token()
            self.decode(sel_idx_out=sel, scores_out=sc)
        return self.out, sel, sc
