"""Seeded synthetic inputs for the hash-aware top-k decode step.

This module serves both sides of every comparison: the GPU path (tests,
bench) and the CPU oracle receive the very same bytes from it.  It holds
random numbers, rounding and the workload shapes only -- none of the
method's arithmetic (no hashing, scoring, selection or attention).

Workloads follow the pages' decode setting (HATA review, "The reading" and
"What carries the argument": cached keys, one query per head per step, a
1.56 % token budget) at the sizes of the five synthetic configurations:

  1  B=1,  8 q / 8 kv heads, context 4096,  top-k 64,   16 planted keys / head
  2  B=8,  32 q / 8 kv,      context 32768, top-k 512,  0.1 % planted
  3  B=4,  32 q / 8 kv,      context 131072, top-k 2048, 0.1 % planted
  4  B=1,  32 q / 8 kv,      context 1048576, top-k 16384, 0.05 % planted
  5  B=64, 32 q / 8 kv,      contexts uniform in [1024, 65536],
     top-k = max(16, floor(N_b / 64)), 0.1 % planted

Values: Q, K, V ~ N(0, 1) rounded to bf16; W_H ~ N(0, 1/128) in fp32, one
128x128 matrix per KV head.  A planted key of KV head g is
3 * (sum of the group's query vectors) / sqrt(G) + N(0, I), rounded to bf16,
at positions drawn uniformly without replacement from [0, N-1).  The context
of length N is N-1 prefilled tokens plus the token the decode step appends
(k_new, v_new ~ N(0, 1), never planted).

Every element is a pure function of (seed, tensor id, flat index), so any
slice -- one (batch, KV head) unit, or a few rows -- can be produced without
the rest.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

HEAD_DIM = 128
N_BITS = 128

# tensor ids of the counter-based streams
T_Q, T_W, T_K, T_V, T_PLANT_NOISE, T_PLANT_POS, T_KNEW, T_VNEW, T_LEN = range(1, 10)
T_TR_BASIS, T_TR_OFFSET, T_TR_QZ, T_TR_QN, T_TR_KZ, T_TR_KN = range(20, 26)

_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c with gcc into libsynth.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11",
                               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_u64.argtypes = [u64, u64, u64, i64, vp]
        L.synth_sm64_stream.argtypes = [u64, i64, vp]
        for f in (L.synth_normal_f64, L.synth_normal_f32, L.synth_normal_bf16):
            f.argtypes = [u64, u64, u64, i64, dbl, vp]
        L.synth_f64_to_bf16.argtypes = [vp, i64, vp]
        for f in (L.synth_u64, L.synth_sm64_stream, L.synth_normal_f64, L.synth_normal_f32,
                  L.synth_normal_bf16, L.synth_f64_to_bf16):
            f.restype = None
        _lib = L
    return _lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(fn, seed, tensor, start, count, scale, out):
    """Run a generator over [start, start+count) into `out`, split across threads
    (ctypes drops the GIL during the foreign call)."""
    count = int(count)
    if count == 0:
        return out
    nt = _threads() if count >= (1 << 20) else 1
    step = (count + nt - 1) // nt
    itemsize = out.itemsize
    base = out.ctypes.data

    def run(i):
        s = i * step
        n = min(step, count - s)
        if n > 0:
            if scale is None:
                fn(seed, tensor, start + s, n, ctypes.c_void_p(base + s * itemsize))
            else:
                fn(seed, tensor, start + s, n, scale, ctypes.c_void_p(base + s * itemsize))

    if nt == 1:
        run(0)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(run, range(nt)))
    return out


def u64(seed: int, tensor: int, start: int, count: int) -> np.ndarray:
    out = np.empty(int(count), dtype=np.uint64)
    return _fill(lib().synth_u64, seed, tensor, start, count, None, out)


def sm64_stream(seed: int, count: int) -> np.ndarray:
    out = np.empty(int(count), dtype=np.uint64)
    lib().synth_sm64_stream(ctypes.c_uint64(seed), count, out.ctypes.data)
    return out


def normal_f64(seed, tensor, start, count, scale=1.0) -> np.ndarray:
    out = np.empty(int(count), dtype=np.float64)
    return _fill(lib().synth_normal_f64, seed, tensor, start, count, float(scale), out)


def normal_f32(seed, tensor, start, count, scale=1.0) -> np.ndarray:
    out = np.empty(int(count), dtype=np.float32)
    return _fill(lib().synth_normal_f32, seed, tensor, start, count, float(scale), out)


def normal_bf16(seed, tensor, start, count, scale=1.0) -> np.ndarray:
    out = np.empty(int(count), dtype=np.uint16)
    return _fill(lib().synth_normal_bf16, seed, tensor, start, count, float(scale), out)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().synth_f64_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Spec:
    """One synthetic decode workload.

    lengths[b] is the context of batch entry b *after* the step appends its
    token: lengths[b] - 1 rows are prefilled.  topk[b] is the token budget.
    planted[b] is the number of planted keys per KV head of entry b.
    stride is the logical per-(b, kv) row stride of the K / V streams
    (>= max(lengths)); it fixes the counter of every element.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    lengths: tuple
    topk: tuple
    planted: tuple
    stride: int
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_len(self) -> int:
        return max(self.lengths) if self.lengths else 0

    @property
    def k_max(self) -> int:
        return max(self.topk) if self.topk else 0


def _round_half_up(x: float) -> int:
    return int(math.floor(x + 0.5))


def ragged_lengths(seed: int, B: int, lo: int, hi: int) -> list:
    """Uniform integers in [lo, hi] by Lemire's multiply-shift on SplitMix64 outputs."""
    span = hi - lo + 1
    xs = u64(seed, T_LEN, 0, B)
    return [lo + ((int(x) * span) >> 64) for x in xs]


def config(i: int, seed: int = 0) -> Spec:
    if i == 1:
        return Spec("cfg1: B1 8q/8kv N4096 k64", 1, 8, 8, (4096,), (64,), (16,), 4096, seed)
    if i == 2:
        n, B = 32768, 8
        return Spec("cfg2: B8 32q/8kv N32768 k512", B, 32, 8, (n,) * B, (512,) * B,
                    (_round_half_up(0.001 * n),) * B, n, seed)
    if i == 3:
        n, B = 131072, 4
        return Spec("cfg3: B4 32q/8kv N131072 k2048", B, 32, 8, (n,) * B, (2048,) * B,
                    (_round_half_up(0.001 * n),) * B, n, seed)
    if i == 4:
        n = 1048576
        return Spec("cfg4: B1 32q/8kv N1048576 k16384", 1, 32, 8, (n,), (16384,),
                    (_round_half_up(0.0005 * n),), n, seed)
    if i == 5:
        B = 64
        lens = ragged_lengths(seed, B, 1024, 65536)
        return Spec("cfg5: B64 32q/8kv N~U[1024,65536] k=max(16,N/64)", B, 32, 8, tuple(lens),
                    tuple(max(16, n // 64) for n in lens),
                    tuple(_round_half_up(0.001 * n) for n in lens), 65536, seed)
    raise ValueError(f"no configuration {i}")


def custom(name, B, Hq, Hkv, lengths, topk, planted, seed=0, stride=None) -> Spec:
    lengths = tuple(int(x) for x in lengths)
    topk = tuple(int(x) for x in topk)
    planted = tuple(int(x) for x in planted)
    assert len(lengths) == len(topk) == len(planted) == B
    assert Hq % Hkv == 0
    stride = int(stride if stride is not None else max(max(lengths), 1))
    assert stride >= max(lengths)
    return Spec(name, B, Hq, Hkv, lengths, topk, planted, stride, seed)


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def gen_q(spec: Spec, step: int = 0) -> np.ndarray:
    """Decode-step queries, bf16 bits [B][Hq][128].  Step 0 is the query the
    planted keys are aligned with; step i > 0 takes the next block of the same
    stream (independent N(0, 1) draws, aligned with no planted key)."""
    n = spec.B * spec.Hq * HEAD_DIM
    return normal_bf16(spec.seed, T_Q, step * n, n).reshape(spec.B, spec.Hq, HEAD_DIM)


def gen_w(spec: Spec) -> np.ndarray:
    """Hash projections W_H, fp32 [Hkv][128 (d)][128 (bit)], N(0, 1/128)."""
    n = spec.Hkv * HEAD_DIM * N_BITS
    return normal_f32(spec.seed, T_W, 0, n, 1.0 / math.sqrt(128.0)).reshape(
        spec.Hkv, HEAD_DIM, N_BITS)


def gen_w_bits(spec: Spec, n_bits: int) -> np.ndarray:
    """Hash projections for a code length of n_bits, fp32 [Hkv][128 (d)][n_bits],
    N(0, 1/128), from the same stream as gen_w (identical at 128 bits)."""
    n = spec.Hkv * HEAD_DIM * n_bits
    return normal_f32(spec.seed, T_W, 0, n, 1.0 / math.sqrt(128.0)).reshape(
        spec.Hkv, HEAD_DIM, n_bits)


def planted_positions(spec: Spec, b: int, kv: int) -> np.ndarray:
    """Sorted planted positions of unit (b, kv): the `planted[b]` positions in
    [0, N_b - 1) with the smallest (random u64, position) pairs."""
    n_pre = spec.lengths[b] - 1
    cnt = min(spec.planted[b], max(n_pre, 0))
    if cnt <= 0:
        return np.zeros(0, dtype=np.int64)
    r = u64(spec.seed, T_PLANT_POS, (b * spec.Hkv + kv) << 32, n_pre)
    order = np.argsort(r, kind="stable")[:cnt]
    return np.sort(order.astype(np.int64))


def _unit_base(spec: Spec, b: int, kv: int) -> int:
    return (b * spec.Hkv + kv) * spec.stride * HEAD_DIM


def gen_unit_k(spec: Spec, b: int, kv: int, q: np.ndarray | None = None) -> np.ndarray:
    """Prefilled key rows of unit (b, kv), bf16 bits [N_b - 1][128], planted rows in place."""
    n_pre = spec.lengths[b] - 1
    base = _unit_base(spec, b, kv)
    k = normal_bf16(spec.seed, T_K, base, n_pre * HEAD_DIM).reshape(n_pre, HEAD_DIM)
    pos = planted_positions(spec, b, kv)
    if pos.size:
        if q is None:
            q = gen_q(spec)
        G = spec.G
        qg = bf16_to_f32(q[b, kv * G:(kv + 1) * G]).astype(np.float64)  # [G][128]
        s = qg.sum(axis=0) / math.sqrt(G)
        rows = np.empty((pos.size, HEAD_DIM), dtype=np.float64)
        for r_i, p in enumerate(pos):
            eps = normal_f64(spec.seed, T_PLANT_NOISE, base + int(p) * HEAD_DIM, HEAD_DIM)
            rows[r_i] = 3.0 * s + eps
        k[pos] = f64_to_bf16(rows)
    return k


def gen_unit_v(spec: Spec, b: int, kv: int) -> np.ndarray:
    """Prefilled value rows of unit (b, kv), bf16 bits [N_b - 1][128]."""
    n_pre = spec.lengths[b] - 1
    return normal_bf16(spec.seed, T_V, _unit_base(spec, b, kv),
                       n_pre * HEAD_DIM).reshape(n_pre, HEAD_DIM)


def gen_new_token(spec: Spec):
    """The token each sequence appends at the decode step: (k_new, v_new), bf16
    bits [B][1][Hkv][128] (token-major, the layout a projection produces)."""
    n = spec.B * spec.Hkv * HEAD_DIM
    kn = normal_bf16(spec.seed, T_KNEW, 0, n).reshape(spec.B, 1, spec.Hkv, HEAD_DIM)
    vn = normal_bf16(spec.seed, T_VNEW, 0, n).reshape(spec.B, 1, spec.Hkv, HEAD_DIM)
    return kn, vn


def unit_context(spec: Spec, b: int, kv: int, q=None, new=None):
    """Full context of unit (b, kv) after the step's append: K, V bf16 [N_b][128]."""
    if q is None:
        q = gen_q(spec)
    if new is None:
        new = gen_new_token(spec)
    k = np.concatenate([gen_unit_k(spec, b, kv, q), new[0][b, 0, kv][None]], axis=0)
    v = np.concatenate([gen_unit_v(spec, b, kv), new[1][b, 0, kv][None]], axis=0)
    return k, v


# --------------------------------------------------------------------------
# structured queries and keys (training and evaluating W_H)
# --------------------------------------------------------------------------

TRAIN_RANK = 16


def structured_basis(seed: int):
    """The fixed structure of one synthetic attention head: TRAIN_RANK
    directions G [16][128] (entries N(0, 1/128)) that carry the q.k signal,
    and a key offset k0 [128] (entries N(0, 64/128), norm about 8) shared by
    every key."""
    G = normal_f64(seed, T_TR_BASIS, 0, TRAIN_RANK * HEAD_DIM,
                   1.0 / math.sqrt(HEAD_DIM)).reshape(TRAIN_RANK, HEAD_DIM)
    k0 = normal_f64(seed, T_TR_OFFSET, 0, HEAD_DIM, 8.0 / math.sqrt(HEAD_DIM))
    return G, k0


def gen_structured_qk(seed: int, block: int, n_q: int, n_k: int):
    """Block `block` of queries and keys with the anisotropy seen in trained
    heads: q = 3 z_q G + 0.3 n_q and k = z_k G + n_k + k0 (z ~ N(0, I_16),
    n ~ N(0, I_128)), rounded to bf16 [n][128].  q.k varies with the z's; the
    keys' noise and shared offset, which dominate their direction, do not
    change a query's ranking of its keys."""
    G, k0 = structured_basis(seed)
    zq = normal_f64(seed, T_TR_QZ, block * n_q * TRAIN_RANK, n_q * TRAIN_RANK).reshape(n_q, TRAIN_RANK)
    nq = normal_f64(seed, T_TR_QN, block * n_q * HEAD_DIM, n_q * HEAD_DIM).reshape(n_q, HEAD_DIM)
    zk = normal_f64(seed, T_TR_KZ, block * n_k * TRAIN_RANK, n_k * TRAIN_RANK).reshape(n_k, TRAIN_RANK)
    nk = normal_f64(seed, T_TR_KN, block * n_k * HEAD_DIM, n_k * HEAD_DIM).reshape(n_k, HEAD_DIM)
    q = 3.0 * (zq @ G) + 0.3 * nq
    k = zk @ G + nk + k0[None, :]
    return f64_to_bf16(q), f64_to_bf16(k)
