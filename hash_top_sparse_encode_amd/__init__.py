"""Python binding of libhata.so (include/hata.h): hash-aware top-k decode
attention on MI355X (gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and streams.  The
binding raises if the shared library is missing (build it with
``python -m hash_top_sparse_encode_amd._build`` or ``__graft_entry__.build()``);
there is no fallback of any kind.

Names mirror the C ABI:
  hata_encode_keys (also the other code lengths, through
  hata_encode_keys_nbits), hata_append, hata_decode_workspace_bytes,
  hata_decode_attn, hata_decode_step, hata_decode_step_static (no workspace),
  hata_recall_workspace_bytes,
  hata_exact_topk_recall, hata_status_string
plus ``HataCache``, a holder of the caller-owned cache tensors.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HATA_LIB_PATH names another build of the same library (the sanitizer test
# loads a host-side ASan/UBSan build this way).
LIB_PATH = os.environ.get("HATA_LIB_PATH") or os.path.join(_PKG, "libhata.so")

HEAD_DIM = 128
N_BITS = 128
CODE_WORDS = 4


def ctrl_words(batch: int, n_kv_heads: int) -> int:
    """int32 words of a cache's control block (HATA_CTRL_WORDS)."""
    return 16 + 64 * (int(batch) * int(n_kv_heads) + int(batch))


HATA_OK = 0
HATA_ERR_INVALID_ARG = 1
HATA_ERR_UNSUPPORTED = 2
HATA_ERR_WORKSPACE = 3
HATA_ERR_HIP = 4
HATA_ERR_SCRATCH_LIMIT = 5
STATIC_SCRATCH_BYTES = 32 << 20

HATA_DEV_APPEND_OVERFLOW = 0x1
HATA_DEV_BAD_LENGTH = 0x2
HATA_DEV_TOPK_CLAMPED = 0x4
HATA_DEV_BAD_NEW = 0x8
HATA_DEV_STALL = 0x10

EXPORTED_SYMBOLS = ("hata_encode_keys", "hata_encode_keys_nbits", "hata_append",
                    "hata_decode_workspace_bytes", "hata_decode_attn", "hata_decode_step",
                    "hata_recall_workspace_bytes", "hata_exact_topk_recall",
                    "hata_status_string", "hata_decode_step_static",
                    "hata_hash_train_workspace_bytes", "hata_hash_labels",
                    "hata_hash_train_step")


class _CCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p),
        ("ctrl", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_bits", ctypes.c_int32),
        ("max_ctx", ctypes.c_int64),
    ]


class TrainParams(ctypes.Structure):
    """hata_train_params: the objective's constants (the pages' values by
    default) and Adam's."""
    _fields_ = [("sigma", ctypes.c_float), ("epsilon", ctypes.c_float), ("eta", ctypes.c_float),
                ("lambda_", ctypes.c_float), ("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("adam_eps", ctypes.c_float)]

    def __init__(self, sigma=0.1, epsilon=0.01, eta=2.0, lambda_=1.0, lr=0.01, beta1=0.9,
                 beta2=0.999, adam_eps=1e-8):
        super().__init__(sigma, epsilon, eta, lambda_, lr, beta1, beta2, adam_eps)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhata.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -m hash_top_sparse_encode_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.hata_encode_keys.argtypes = [vp, i64, i32, i64, i64, vp, vp, vp]
        L.hata_encode_keys.restype = ctypes.c_int
        L.hata_encode_keys_nbits.argtypes = [vp, i64, i32, i64, i64, vp, i32, vp, vp]
        L.hata_encode_keys_nbits.restype = ctypes.c_int
        L.hata_append.argtypes = [ctypes.POINTER(_CCache), vp, vp, vp, i32, vp, vp]
        L.hata_append.restype = ctypes.c_int
        L.hata_decode_workspace_bytes.argtypes = [ctypes.POINTER(_CCache), i32]
        L.hata_decode_workspace_bytes.restype = sz
        L.hata_decode_attn.argtypes = [ctypes.POINTER(_CCache), vp, vp, vp, i32, vp, vp, sz, vp,
                                       vp, vp]
        L.hata_decode_attn.restype = ctypes.c_int
        L.hata_decode_step.argtypes = [ctypes.POINTER(_CCache), vp, vp, vp, vp, vp, i32, vp, vp,
                                       sz, vp, vp, vp]
        L.hata_decode_step.restype = ctypes.c_int
        L.hata_decode_step_static.argtypes = [ctypes.POINTER(_CCache), vp, vp, vp, vp, vp, i32,
                                              vp, vp, vp, vp]
        L.hata_decode_step_static.restype = ctypes.c_int
        L.hata_hash_train_workspace_bytes.argtypes = [i32, i32, i32]
        L.hata_hash_train_workspace_bytes.restype = sz
        L.hata_hash_labels.argtypes = [vp, i32, vp, i32, vp, vp]
        L.hata_hash_labels.restype = ctypes.c_int
        L.hata_hash_train_step.argtypes = [vp, i32, vp, i32, vp, i32, vp, vp, vp, i32,
                                           ctypes.POINTER(TrainParams), vp, vp, vp, sz, vp]
        L.hata_hash_train_step.restype = ctypes.c_int
        L.hata_recall_workspace_bytes.argtypes = [ctypes.POINTER(_CCache)]
        L.hata_recall_workspace_bytes.restype = sz
        L.hata_exact_topk_recall.argtypes = [ctypes.POINTER(_CCache), vp, vp, i32, vp, vp, vp,
                                             vp, vp, vp, sz, vp]
        L.hata_exact_topk_recall.restype = ctypes.c_int
        # The HIP runtime the library is linked against (dlsym on the
        # library's handle also searches its dependencies): device addresses
        # of pinned host tensors that hold an offloaded K/V cache.
        L.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(vp), vp, ctypes.c_uint]
        L.hipHostGetDevicePointer.restype = ctypes.c_int
        L.hata_status_string.argtypes = [ctypes.c_int]
        L.hata_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


class HataError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {hata_status_string(status)} (status {status})")
        self.status = status


def hata_status_string(status: int) -> str:
    return lib().hata_status_string(int(status)).decode()


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != HATA_OK:
        raise HataError(fn, status)


def _need(t: torch.Tensor, name: str, dtype, numel: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, has {t.numel()}")


def _need_kv(t: torch.Tensor, name: str, numel: int):
    """K/V cache tensors live in device memory, or in pinned host memory (the
    offloaded layout: the kernels read the selected rows over the host link)."""
    if isinstance(t, torch.Tensor) and not t.is_cuda:
        if not t.is_pinned():
            raise ValueError(f"{name} on the host must be pinned (pin_memory=True)")
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.numel() != numel:
            raise ValueError(f"{name} must be a contiguous bf16 tensor of {numel} elements")
        return
    _need(t, name, torch.bfloat16, numel)


def _device_address(t: torch.Tensor) -> int:
    """The address kernels use for t: its own for device memory, the mapped
    device address for pinned host memory."""
    if t.is_cuda:
        return t.data_ptr()
    dev = ctypes.c_void_p()
    err = lib().hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dev.value:
        raise ValueError(f"host tensor at {t.data_ptr():#x} is not mapped into the device's "
                         f"address space (hipHostGetDevicePointer error {err})")
    return dev.value


class HataCache:
    """Caller-owned cache tensors of include/hata.h's hata_cache.

    k, v   : bf16 [batch][n_kv_heads][max_ctx][128], on the device or, for the
             offloaded layout, pinned host tensors (``offload=True`` allocates
             them so)
    codes  : int32 (u32 bit patterns) [batch][n_kv_heads][max_ctx][4]
    seq_len: int32 [batch]
    ctrl   : int32 [ctrl_words(batch, n_kv_heads)], zero at creation
    """

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, max_ctx: int,
                 device="cuda", k=None, v=None, codes=None, seq_len=None, ctrl=None,
                 offload: bool = False, n_bits: int = N_BITS):
        self.batch, self.n_q_heads, self.n_kv_heads, self.max_ctx = (
            int(batch), int(n_q_heads), int(n_kv_heads), int(max_ctx))
        self.n_bits = int(n_bits)
        words = self.n_bits // 32
        shape = (self.batch, self.n_kv_heads, self.max_ctx, HEAD_DIM)
        kv_dev = dict(device="cpu", pin_memory=True) if offload else dict(device=device)
        self.k = k if k is not None else torch.empty(shape, dtype=torch.bfloat16, **kv_dev)
        self.v = v if v is not None else torch.empty(shape, dtype=torch.bfloat16, **kv_dev)
        self.codes = codes if codes is not None else torch.zeros(
            shape[:3] + (words,), dtype=torch.int32, device=device)
        self.seq_len = seq_len if seq_len is not None else torch.zeros(
            self.batch, dtype=torch.int32, device=device)
        self.ctrl = ctrl if ctrl is not None else torch.zeros(
            ctrl_words(self.batch, self.n_kv_heads), dtype=torch.int32, device=device)
        _need_kv(self.k, "k", self.batch * self.n_kv_heads * self.max_ctx * HEAD_DIM)
        _need_kv(self.v, "v", self.k.numel())
        self._kv_addr = None
        _need(self.codes, "codes", torch.int32,
              self.batch * self.n_kv_heads * self.max_ctx * words)
        _need(self.seq_len, "seq_len", torch.int32, self.batch)
        _need(self.ctrl, "ctrl", torch.int32, ctrl_words(self.batch, self.n_kv_heads))

    def c_struct(self, head_dim: int = HEAD_DIM, n_bits: int = None) -> _CCache:
        n_bits = self.n_bits if n_bits is None else n_bits
        if self._kv_addr is None:
            self._kv_addr = (_device_address(self.k), _device_address(self.v))
        return _CCache(self._kv_addr[0], self._kv_addr[1], self.codes.data_ptr(),
                       self.seq_len.data_ptr(), self.ctrl.data_ptr(), self.batch,
                       self.n_q_heads, self.n_kv_heads, head_dim, n_bits, self.max_ctx)

    def status(self) -> int:
        """Sticky device status bits (HATA_DEV_*); reads device memory (syncs)."""
        return int(self.ctrl[0].item())


def hata_encode_keys(keys: torch.Tensor, w_h: torch.Tensor, codes_out: torch.Tensor = None,
                     stream=None) -> torch.Tensor:
    """Codes of keys [n_rows][n_heads][128] (bf16; the last dim contiguous, the
    others with any stride) under w_h [n_heads][128][r] (fp32, r = 32, 64,
    128 or 256): int32 [n_rows][n_heads][r / 32]."""
    if keys.dtype != torch.bfloat16 or keys.dim() != 3 or keys.shape[2] != HEAD_DIM:
        raise ValueError("keys must be bf16 [n_rows][n_heads][128]")
    if keys.stride(2) != 1:
        raise ValueError("keys' last dimension must be contiguous")
    n_rows, n_heads = keys.shape[0], keys.shape[1]
    if w_h.dim() != 3 or w_h.shape[0] != n_heads or w_h.shape[1] != HEAD_DIM:
        raise ValueError("w_h must be fp32 [n_heads][128][n_bits]")
    n_bits = int(w_h.shape[2])
    words = max(n_bits // 32, 1)
    _need(w_h, "w_h", torch.float32, n_heads * HEAD_DIM * n_bits)
    if codes_out is None:
        codes_out = torch.empty((n_rows, n_heads, words), dtype=torch.int32, device=keys.device)
    _need(codes_out, "codes_out", torch.int32, n_rows * n_heads * words)
    if n_bits == N_BITS:
        st = lib().hata_encode_keys(keys.data_ptr(), n_rows, n_heads, keys.stride(0),
                                    keys.stride(1), w_h.data_ptr(), codes_out.data_ptr(),
                                    _stream(stream))
        _check("hata_encode_keys", st)
    else:
        st = lib().hata_encode_keys_nbits(keys.data_ptr(), n_rows, n_heads, keys.stride(0),
                                          keys.stride(1), w_h.data_ptr(), n_bits,
                                          codes_out.data_ptr(), _stream(stream))
        _check("hata_encode_keys_nbits", st)
    return codes_out


def hata_append(cache: HataCache, k_new, v_new, n_new: torch.Tensor, t_max: int,
                w_h: torch.Tensor, stream=None) -> None:
    """Append up to t_max tokens per sequence (k_new, v_new bf16
    [batch][t_max][n_kv_heads][128], or both None to encode rows already in
    the cache); n_new int32 [batch] on the device."""
    B, Hkv = cache.batch, cache.n_kv_heads
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        _need(k_new, "k_new", torch.bfloat16, B * int(t_max) * Hkv * HEAD_DIM)
        _need(v_new, "v_new", torch.bfloat16, B * int(t_max) * Hkv * HEAD_DIM)
    _need(n_new, "n_new", torch.int32, B)
    _need(w_h, "w_h", torch.float32, Hkv * HEAD_DIM * cache.n_bits)
    c = cache.c_struct()
    st = lib().hata_append(ctypes.byref(c), _ptr(k_new), _ptr(v_new), n_new.data_ptr(),
                           int(t_max), w_h.data_ptr(), _stream(stream))
    _check("hata_append", st)


def hata_decode_workspace_bytes(cache: HataCache, k_max: int) -> int:
    c = cache.c_struct()
    return int(lib().hata_decode_workspace_bytes(ctypes.byref(c), int(k_max)))


def alloc_workspace(cache: HataCache, k_max: int) -> torch.Tensor:
    """A zero-filled device byte tensor of the required size (torch
    allocations are 256-byte aligned).  It may be shared by caches whose
    calls are ordered on one stream."""
    n = hata_decode_workspace_bytes(cache, k_max)
    if n == 0:
        raise ValueError("unsupported cache shape")
    return torch.zeros(n, dtype=torch.uint8, device=cache.codes.device)


def hata_decode_attn(cache: HataCache, q: torch.Tensor, w_h: torch.Tensor, topk: torch.Tensor,
                     k_max: int, out: torch.Tensor, workspace: torch.Tensor,
                     sel_idx_out: torch.Tensor = None, scores_out: torch.Tensor = None,
                     stream=None) -> torch.Tensor:
    """One hashed top-k decode step: q bf16 [batch][n_q_heads][128] -> out
    bf16 [batch][n_q_heads][128].  Optional debug outputs: sel_idx_out int32
    [batch][n_kv_heads][k_max], scores_out int16 (u16 patterns)
    [batch][n_kv_heads][max_ctx]."""
    B, Hq, Hkv = cache.batch, cache.n_q_heads, cache.n_kv_heads
    _need(q, "q", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(out, "out", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(w_h, "w_h", torch.float32, Hkv * HEAD_DIM * cache.n_bits)
    _need(topk, "topk", torch.int32, B)
    _need(workspace, "workspace", torch.uint8)
    if sel_idx_out is not None:
        _need(sel_idx_out, "sel_idx_out", torch.int32, B * Hkv * int(k_max))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.int16, B * Hkv * cache.max_ctx)
    c = cache.c_struct()
    st = lib().hata_decode_attn(ctypes.byref(c), q.data_ptr(), w_h.data_ptr(), topk.data_ptr(),
                                int(k_max), out.data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _ptr(sel_idx_out), _ptr(scores_out),
                                _stream(stream))
    _check("hata_decode_attn", st)
    return out


def hata_decode_step(cache: HataCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                     w_h: torch.Tensor, topk: torch.Tensor, k_max: int, out: torch.Tensor,
                     workspace: torch.Tensor, sel_idx_out: torch.Tensor = None,
                     scores_out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Append one token per sequence (k_new, v_new bf16 [batch][n_kv_heads][128])
    and decode over the grown context, in one kernel launch."""
    B, Hq, Hkv = cache.batch, cache.n_q_heads, cache.n_kv_heads
    _need(k_new, "k_new", torch.bfloat16, B * Hkv * HEAD_DIM)
    _need(v_new, "v_new", torch.bfloat16, B * Hkv * HEAD_DIM)
    _need(q, "q", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(out, "out", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(w_h, "w_h", torch.float32, Hkv * HEAD_DIM * cache.n_bits)
    _need(topk, "topk", torch.int32, B)
    _need(workspace, "workspace", torch.uint8)
    if sel_idx_out is not None:
        _need(sel_idx_out, "sel_idx_out", torch.int32, B * Hkv * int(k_max))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.int16, B * Hkv * cache.max_ctx)
    c = cache.c_struct()
    st = lib().hata_decode_step(ctypes.byref(c), k_new.data_ptr(), v_new.data_ptr(),
                                q.data_ptr(), w_h.data_ptr(), topk.data_ptr(), int(k_max),
                                out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _ptr(sel_idx_out), _ptr(scores_out), _stream(stream))
    _check("hata_decode_step", st)
    return out


def hata_decode_step_static(cache: HataCache, k_new: torch.Tensor, v_new: torch.Tensor,
                            q: torch.Tensor, w_h: torch.Tensor, topk: torch.Tensor, k_max: int,
                            out: torch.Tensor, sel_idx_out: torch.Tensor = None,
                            scores_out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """hata_decode_step on the library's static scratch (no workspace, no
    allocation; n_bits = 128; calls on one GPU must not overlap)."""
    B, Hq, Hkv = cache.batch, cache.n_q_heads, cache.n_kv_heads
    _need(k_new, "k_new", torch.bfloat16, B * Hkv * HEAD_DIM)
    _need(v_new, "v_new", torch.bfloat16, B * Hkv * HEAD_DIM)
    _need(q, "q", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(out, "out", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(w_h, "w_h", torch.float32, Hkv * HEAD_DIM * cache.n_bits)
    _need(topk, "topk", torch.int32, B)
    if sel_idx_out is not None:
        _need(sel_idx_out, "sel_idx_out", torch.int32, B * Hkv * int(k_max))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.int16, B * Hkv * cache.max_ctx)
    c = cache.c_struct()
    st = lib().hata_decode_step_static(ctypes.byref(c), k_new.data_ptr(), v_new.data_ptr(),
                                       q.data_ptr(), w_h.data_ptr(), topk.data_ptr(), int(k_max),
                                       out.data_ptr(), _ptr(sel_idx_out), _ptr(scores_out),
                                       _stream(stream))
    _check("hata_decode_step_static", st)
    return out


def hata_recall_workspace_bytes(cache: HataCache) -> int:
    c = cache.c_struct()
    return int(lib().hata_recall_workspace_bytes(ctypes.byref(c)))


def alloc_recall_workspace(cache: HataCache) -> torch.Tensor:
    """A device byte tensor for hata_exact_topk_recall (no initial contents needed)."""
    n = hata_recall_workspace_bytes(cache)
    if n == 0:
        raise ValueError("unsupported cache shape")
    return torch.empty(n, dtype=torch.uint8, device=cache.codes.device)


def hata_exact_topk_recall(cache: HataCache, q: torch.Tensor, topk: torch.Tensor, k_max: int,
                           sel_idx: torch.Tensor, scores: torch.Tensor,
                           workspace: torch.Tensor, overlap_out: torch.Tensor = None,
                           tie_out: torch.Tensor = None, exact_idx_out: torch.Tensor = None,
                           stream=None):
    """Recall analysis of a decode call's selection (its sel_idx_out and
    scores_out): returns (overlap int32 [batch][n_q_heads], tie int32
    [batch][n_kv_heads][4] = (T, below, at, k_eff)); exact_idx_out (int32
    [batch][n_q_heads][k_max]) receives each head's exact top-k if given."""
    B, Hq, Hkv = cache.batch, cache.n_q_heads, cache.n_kv_heads
    dev = cache.codes.device
    _need(q, "q", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(topk, "topk", torch.int32, B)
    _need(sel_idx, "sel_idx", torch.int32, B * Hkv * int(k_max))
    _need(scores, "scores", torch.int16, B * Hkv * cache.max_ctx)
    _need(workspace, "workspace", torch.uint8)
    if overlap_out is None:
        overlap_out = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    if tie_out is None:
        tie_out = torch.empty((B, Hkv, 4), dtype=torch.int32, device=dev)
    _need(overlap_out, "overlap_out", torch.int32, B * Hq)
    _need(tie_out, "tie_out", torch.int32, B * Hkv * 4)
    if exact_idx_out is not None:
        _need(exact_idx_out, "exact_idx_out", torch.int32, B * Hq * int(k_max))
    c = cache.c_struct()
    st = lib().hata_exact_topk_recall(ctypes.byref(c), q.data_ptr(), topk.data_ptr(), int(k_max),
                                      sel_idx.data_ptr(), scores.data_ptr(),
                                      overlap_out.data_ptr(), tie_out.data_ptr(),
                                      _ptr(exact_idx_out), workspace.data_ptr(),
                                      workspace.numel(), _stream(stream))
    _check("hata_exact_topk_recall", st)
    return overlap_out, tie_out


# ------------------------------------------------------------ hash training


def hata_hash_train_workspace_bytes(n_q: int, n_k: int, n_bits: int) -> int:
    return int(lib().hata_hash_train_workspace_bytes(int(n_q), int(n_k), int(n_bits)))


def hata_hash_labels(q: torch.Tensor, k: torch.Tensor, labels: torch.Tensor = None,
                     stream=None) -> torch.Tensor:
    """Training labels [n_q][n_k] (fp32) of queries q [n_q][128] and keys
    k [n_k][128] (bf16): top ceil(n_k / 10) keys by exact q.k per query,
    linearly decayed over [20, 1]; the rest -1."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    n_q, n_k = q.numel() // HEAD_DIM, k.numel() // HEAD_DIM
    if labels is None:
        labels = torch.empty((n_q, n_k), dtype=torch.float32, device=q.device)
    _need(labels, "labels", torch.float32, n_q * n_k)
    st = lib().hata_hash_labels(q.data_ptr(), n_q, k.data_ptr(), n_k, labels.data_ptr(),
                                _stream(stream))
    _check("hata_hash_labels", st)
    return labels


class HashTrainer:
    """Device state of W_H training: the weights [128][n_bits], Adam's moments,
    a workspace for batches of n_q queries and n_k keys, the step count."""

    def __init__(self, w_init: torch.Tensor, n_q: int, n_k: int, params: TrainParams = None):
        _need(w_init, "w_init", torch.float32)
        self.n_bits = w_init.numel() // HEAD_DIM
        self.w = w_init.clone().reshape(HEAD_DIM, self.n_bits)
        self.m = torch.zeros_like(self.w)
        self.v = torch.zeros_like(self.w)
        self.n_q, self.n_k = int(n_q), int(n_k)
        n = hata_hash_train_workspace_bytes(self.n_q, self.n_k, self.n_bits)
        if n == 0:
            raise ValueError("unsupported training batch shape")
        self.ws = torch.empty(n, dtype=torch.uint8, device=w_init.device)
        self.loss = torch.zeros(4, dtype=torch.float32, device=w_init.device)
        self.params = params if params is not None else TrainParams()
        self.steps = 0

    def step(self, q: torch.Tensor, k: torch.Tensor, labels: torch.Tensor, update: bool = True,
             grad_out: torch.Tensor = None, stream=None) -> torch.Tensor:
        """One training step (hata_hash_train_step); returns the loss tensor
        (L, L_sim, L_bal, L_unc) at the weights before the update."""
        _need(q, "q", torch.bfloat16, self.n_q * HEAD_DIM)
        _need(k, "k", torch.bfloat16, self.n_k * HEAD_DIM)
        _need(labels, "labels", torch.float32, self.n_q * self.n_k)
        if grad_out is not None:
            _need(grad_out, "grad_out", torch.float32, HEAD_DIM * self.n_bits)
        step = self.steps + 1 if update else 0
        st = lib().hata_hash_train_step(q.data_ptr(), self.n_q, k.data_ptr(), self.n_k,
                                        labels.data_ptr(), self.n_bits, self.w.data_ptr(),
                                        self.m.data_ptr(), self.v.data_ptr(), step,
                                        ctypes.byref(self.params), self.loss.data_ptr(),
                                        _ptr(grad_out), self.ws.data_ptr(), self.ws.numel(),
                                        _stream(stream))
        _check("hata_hash_train_step", st)
        if update:
            self.steps += 1
        return self.loss
