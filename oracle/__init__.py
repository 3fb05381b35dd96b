"""CPU oracle of the hash-aware top-k decode step (HATA) -- test infrastructure.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  It never imports, loads or calls the GPU path, and the GPU
path never imports it.  The arithmetic lives in plain C (hata_oracle.c,
double precision, one step per function); this file builds and loads that
library and composes its steps for one (batch, KV head) unit, following the
decode workflow of the HATA review ("What carries the argument"): encode the
query heads, score every cached key by summed Hamming distance, keep the k
lowest, attend over them.

Threads: large calls are split into row ranges run on a thread pool; ctypes
releases the GIL, and each range runs the unchanged C step.

Parity status of each function (what pins it) is documented in the tests
under tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hata_oracle.c")
_SRC_TRAIN = os.path.join(_HERE, "hash_train_oracle.c")
# HATA_ORACLE_LIB names another build of hata_oracle.c (the sanitizer test
# loads an ASan/UBSan build this way).
_LIB_PATH = os.environ.get("HATA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

D = 128
R = 128


def build(force: bool = True) -> str:
    """Compile hata_oracle.c with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                               "-fno-fast-math", _SRC, _SRC_TRAIN, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_encode.argtypes = [vp, i64, i64, ci, vp, ci, vp]
        L.oracle_encode.restype = None
        L.oracle_hamming.argtypes = [vp, ci, vp, i64, ci, vp]
        L.oracle_hamming.restype = None
        L.oracle_select.argtypes = [vp, i64, i64, vp]
        L.oracle_select.restype = i64
        L.oracle_attend.argtypes = [vp, ci, vp, vp, i64, ci, vp, i64, vp]
        L.oracle_attend.restype = ci
        L.oracle_exact_topk.argtypes = [vp, vp, i64, ci, i64, i64, vp]
        L.oracle_exact_topk.restype = i64
        dbl = ctypes.c_double
        L.oracle_hash_labels.argtypes = [vp, ci, vp, ci, ci, vp]
        L.oracle_hash_labels.restype = ci
        L.oracle_hash_loss_grad.argtypes = [vp, ci, vp, ci, ci, vp, ci, vp, dbl, dbl, dbl, dbl,
                                            vp, vp]
        L.oracle_hash_loss_grad.restype = ci
        L.oracle_adam.argtypes = [vp, vp, vp, vp, i64, ci, dbl, dbl, dbl, dbl]
        L.oracle_adam.restype = None
        _lib = L
    return _lib


def _nthreads(n_rows: int, per_row_cost: int) -> int:
    if n_rows * per_row_cost < (1 << 22):
        return 1
    return max(1, min(16, os.cpu_count() or 1))


def _ranges(n: int, parts: int):
    step = (n + parts - 1) // parts
    return [(s, min(n, s + step)) for s in range(0, n, step)] if n else []


def encode(x: np.ndarray, w: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Sign codes of bf16 rows x [n][d] under W_H w [d][r] (fp32): u32 [n][r/32]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, d = x.shape
    assert w.shape[0] == d and w.shape[1] % 32 == 0
    r = w.shape[1]
    codes = np.zeros((n, r // 32), dtype=np.uint32)
    L = lib()
    nt = threads or _nthreads(n, d * r)

    def run(rng):
        a, b = rng
        if b > a:
            L.oracle_encode(x[a:].ctypes.data, b - a, d, d, w.ctypes.data, r,
                            codes[a:].ctypes.data)

    parts = _ranges(n, nt * 4) if nt > 1 else [(0, n)]
    if nt > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(run, parts))
    else:
        for p in parts:
            run(p)
    return codes


def hamming(qcodes: np.ndarray, kcodes: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Summed Hamming scores of every key code against the G query codes: int32 [n]."""
    qcodes = np.ascontiguousarray(qcodes, dtype=np.uint32)
    kcodes = np.ascontiguousarray(kcodes, dtype=np.uint32)
    G, words = qcodes.shape
    n = kcodes.shape[0]
    assert kcodes.shape[1] == words
    r = words * 32
    out = np.zeros(n, dtype=np.int32)
    L = lib()
    nt = threads or _nthreads(n, G * r)

    def run(rng):
        a, b = rng
        if b > a:
            L.oracle_hamming(qcodes.ctypes.data, G, kcodes[a:].ctypes.data, b - a, r,
                             out[a:].ctypes.data)

    parts = _ranges(n, nt * 4) if nt > 1 else [(0, n)]
    if nt > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(run, parts))
    else:
        for p in parts:
            run(p)
    return out


def select(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k_eff = min(k, n) lowest (score, index) pairs, ascending index."""
    scores = np.ascontiguousarray(scores, dtype=np.int32)
    n = scores.shape[0]
    idx = np.zeros(max(min(int(k), n), 0), dtype=np.int64)
    m = lib().oracle_select(scores.ctypes.data, n, int(k), idx.ctypes.data)
    if m < 0:
        raise MemoryError("oracle_select")
    return idx[:m]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Exact softmax attention of q [G][d] (bf16) over rows idx of K, V [n][d] (bf16):
    double [G][d]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    G, d = q.shape
    assert K.shape[1] == d and V.shape == K.shape
    if idx.size:
        assert idx.min() >= 0 and idx.max() < K.shape[0]
    out = np.zeros((G, d), dtype=np.float64)
    rc = lib().oracle_attend(q.ctypes.data, G, K.ctypes.data, V.ctypes.data, d, d,
                             idx.ctypes.data, idx.size, out.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_attend")
    return out


def decode_unit(q_group: np.ndarray, w: np.ndarray, K: np.ndarray, V: np.ndarray, k: int,
                kcodes: np.ndarray | None = None, threads: int | None = None) -> dict:
    """One decode step of one (batch, KV head) unit.

    q_group: bf16 [G][d], the group's query heads; w: fp32 [d][r], the KV
    head's W_H; K, V: bf16 [n][d], the whole context (including the token
    the step appended); k: token budget.  kcodes: the cached key codes if
    already known (they are a pure function of K and w).
    """
    qcodes = encode(q_group, w, threads=1)
    if kcodes is None:
        kcodes = encode(K, w, threads=threads)
    scores = hamming(qcodes, kcodes, threads=threads)
    idx = select(scores, k)
    out = attend(q_group, K, V, idx)
    return {"qcodes": qcodes, "kcodes": kcodes, "scores": scores, "idx": idx, "out": out}


def exact_topk(q: np.ndarray, K: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k_eff = min(k, n) keys of K [n][d] (bf16) with the largest
    exact logits q . k_i (q bf16 [d]; sequential double sum, lower index first
    among equal logits), in ascending order."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    K = np.ascontiguousarray(K, dtype=np.uint16)
    n, d = K.shape
    assert q.shape == (d,)
    idx = np.zeros(max(min(int(k), n), 0), dtype=np.int64)
    m = lib().oracle_exact_topk(q.ctypes.data, K.ctypes.data, d, d, n, int(k), idx.ctypes.data)
    if m < 0:
        raise MemoryError("oracle_exact_topk")
    return idx[:m]


def overlap(sel: np.ndarray, exact: np.ndarray) -> int:
    """|S intersect E|: how many of the Hamming-selected keys are in the exact top-k."""
    return int(np.intersect1d(np.asarray(sel), np.asarray(exact)).size)


def tie_bucket(scores: np.ndarray, k: int) -> tuple:
    """The Hamming selection's cut, for the review's tie analysis (major
    comment 1): with k_eff = min(k, n), T = the k_eff-th smallest score,
    below = keys scoring under T, at = keys scoring exactly T (the bucket the
    cut falls in; the selection takes k_eff - below of them).  Returns
    (T, below, at, k_eff), or (-1, 0, 0, 0) when k_eff = 0."""
    scores = np.asarray(scores)
    k_eff = max(0, min(int(k), scores.size))
    if k_eff == 0:
        return (-1, 0, 0, 0)
    T = int(np.sort(scores, kind="stable")[k_eff - 1])
    return (T, int((scores < T).sum()), int((scores == T).sum()), k_eff)


def recall_unit(q_group: np.ndarray, K: np.ndarray, k: int, sel: np.ndarray,
                scores: np.ndarray) -> dict:
    """The recall analysis of one (batch, KV head) unit: for every query head
    of the group, its exact top-k set and the overlap with the group's
    Hamming selection `sel`; and the tie bucket of the group's scores."""
    exact = [exact_topk(q_group[h], K, k) for h in range(q_group.shape[0])]
    return {"exact": exact, "overlap": [overlap(sel, e) for e in exact],
            "tie": tie_bucket(scores, k)}


# ------------------------------------------------------------ hash training
# The learning-to-hash objective that produces W_H (hash_train_oracle.c):
# relaxed codes 2 Sigmoid(sigma x W_H) - 1, labels from exact qk scores, a
# similarity-weighted Hamming loss plus bit-balance and uncorrelation
# penalties, Adam updates.

SIGMA, EPSILON, ETA, LAMBDA = 0.1, 0.01, 2.0, 1.0


def hash_labels(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Training labels [n_q][n_k] (float32) of queries q [n_q][d] and keys
    k [n_k][d] (bf16): per query, the top ceil(n_k / 10) keys by exact q.k
    (lower index first among equal scores) get 20 - 19 t / (m - 1) by rank t,
    the rest -1."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    nq, d = q.shape
    nk = k.shape[0]
    assert k.shape[1] == d
    out = np.zeros((nq, nk), dtype=np.float32)
    if lib().oracle_hash_labels(q.ctypes.data, nq, k.ctypes.data, nk, d, out.ctypes.data) != 0:
        raise MemoryError("oracle_hash_labels")
    return out


def hash_loss_grad(q: np.ndarray, k: np.ndarray, w: np.ndarray, labels: np.ndarray,
                   sigma=SIGMA, epsilon=EPSILON, eta=ETA, lam=LAMBDA):
    """(loss[4] = (L, L_sim, L_bal, L_unc), dL/dW [d][r]) in double, at W
    (fp32 [d][r]) for the batch (q [n_q][d], k [n_k][d] bf16; labels
    [n_q][n_k] fp32)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    labels = np.ascontiguousarray(labels, dtype=np.float32)
    nq, d = q.shape
    nk = k.shape[0]
    r = w.shape[1]
    assert w.shape[0] == d and labels.shape == (nq, nk)
    loss = np.zeros(4, dtype=np.float64)
    grad = np.zeros((d, r), dtype=np.float64)
    rc = lib().oracle_hash_loss_grad(q.ctypes.data, nq, k.ctypes.data, nk, d, w.ctypes.data, r,
                                     labels.ctypes.data, float(sigma), float(epsilon), float(eta),
                                     float(lam), loss.ctypes.data, grad.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_hash_loss_grad")
    return loss, grad


def adam(w, m, v, g, step: int, lr: float, b1=0.9, b2=0.999, e=1e-8):
    """One Adam step in double; returns the new (w, m, v)."""
    w = np.array(w, dtype=np.float64)
    m = np.array(m, dtype=np.float64)
    v = np.array(v, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    lib().oracle_adam(w.ctypes.data, m.ctypes.data, v.ctypes.data, g.ctypes.data, w.size,
                      int(step), float(lr), float(b1), float(b2), float(e))
    return w, m, v
