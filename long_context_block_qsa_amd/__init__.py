"""Python binding of the QSA hot path (``libqsa.so``, C ABI in ``include/qsa.h``).

Argument marshalling only: every step of the path runs in the library's HIP kernels.
Tensors are torch tensors on a ROCm device; bf16 tensors may be ``torch.bfloat16`` or
16-bit integer views of the same bits. PyTorch provides device memory and streams.

The library must be built (``python -m long_context_block_qsa_amd.build``); importing
the binding without it raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libqsa.so")
HEADER = os.path.join(ROOT, "include", "qsa.h")

HQ, HKV, D, HI, DI, BS, KMAX = 24, 2, 128, 4, 64, 4, 512

QSA_OK, QSA_ERR_NULL, QSA_ERR_SHAPE, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE, QSA_ERR_DEVICE = range(6)


class QsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)}")
        self.status = status


class qsa_dims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("topk_blocks", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class qsa_seqs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32),
                ("cu_q_host", ctypes.c_void_p), ("cu_k_host", ctypes.c_void_p),
                ("cu_q_dev", ctypes.c_void_p), ("cu_k_dev", ctypes.c_void_p)]


_lib = None

_SIGS = {
    "qsa_abi_version": ([], ctypes.c_int32),
    "qsa_status_string": ([ctypes.c_int32], ctypes.c_char_p),
    "qsa_workspace_size": ([ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "qsa_compress": ([ctypes.c_void_p] * 5, ctypes.c_int),
    "qsa_select": ([ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "qsa_score": ([ctypes.c_void_p] * 6 + [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_void_p], ctypes.c_int),
    "qsa_attend": ([ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "qsa_forward": ([ctypes.c_void_p] * 13 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "qsa_forward_noalloc": ([ctypes.c_void_p] * 13, ctypes.c_int),
    "qsa_quantize_kv": ([ctypes.c_void_p] * 9, ctypes.c_int),
    "qsa_attend_fp8": ([ctypes.c_void_p] * 11 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "qsa_forward_fp8": ([ctypes.c_void_p] * 15 + [ctypes.c_size_t, ctypes.c_void_p],
                        ctypes.c_int),
    "qsa_backward_workspace_size": ([ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "qsa_attend_backward": ([ctypes.c_void_p] * 13 + [ctypes.c_size_t, ctypes.c_void_p],
                            ctypes.c_int),
    "qsa_trace_begin": ([ctypes.c_int32], ctypes.c_int),
    "qsa_trace_end": ([ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int32),
    "qsa_kernel_name": ([ctypes.c_int32], ctypes.c_char_p),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_block_qsa_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(h, name)
            f.argtypes, f.restype = args, res
        _lib = h
    return _lib


def header_functions():
    """Names of the functions include/qsa.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:qsa_status|int32_t|const char \*)\s*(qsa_\w+)\s*\(",
                                 txt, flags=re.M)))


def status_string(status: int) -> str:
    return lib().qsa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != QSA_OK:
        raise QsaError(status, where)


def make_dims(topk: int = KMAX, softmax_scale: float = 0.0) -> qsa_dims:
    return qsa_dims(HQ, HKV, D, HI, DI, BS, int(topk), float(softmax_scale))


class Seqs:
    """Sequence offsets on the host (validation, grid sizing) and on the device."""

    def __init__(self, cu_q, cu_k, device="cuda"):
        import torch
        self.cu_q_np = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int32))
        self.cu_k_np = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int32))
        if self.cu_q_np.shape != self.cu_k_np.shape or self.cu_k_np.ndim != 1:
            raise ValueError("cu_q and cu_k must be 1-D arrays of the same length")
        self.cu_q_dev = torch.from_numpy(self.cu_q_np).to(device)
        self.cu_k_dev = torch.from_numpy(self.cu_k_np).to(device)
        self.batch = len(self.cu_k_np) - 1
        self.c = qsa_seqs(self.batch, self.cu_q_np.ctypes.data, self.cu_k_np.ctypes.data,
                          self.cu_q_dev.data_ptr(), self.cu_k_dev.data_ptr())

    @property
    def n_q(self):
        return int(self.cu_q_np[-1])

    @property
    def n_k(self):
        return int(self.cu_k_np[-1])

    @property
    def n_blocks(self):
        return int((np.diff(self.cu_k_np.astype(np.int64)) // BS).sum())


def _ptr(t, name, elem_bytes=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem_bytes is not None and t.element_size() != elem_bytes:
        raise ValueError(f"{name}: expected {elem_bytes}-byte elements")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def workspace_size(seqs: Seqs, topk: int = KMAX) -> int:
    d = make_dims(topk)
    n = ctypes.c_size_t(0)
    _check(lib().qsa_workspace_size(ctypes.byref(d), ctypes.byref(seqs.c), ctypes.byref(n)),
           "qsa_workspace_size")
    return int(n.value)


def alloc_workspace(seqs: Seqs, topk: int = KMAX, device="cuda"):
    """A zero-filled device buffer of qsa_workspace_size() bytes, 256-byte aligned (the
    library expects the workspace's control block to be zero before its first use)."""
    import torch
    n = workspace_size(seqs, topk)
    buf = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + n] if n > 0 else buf[off:off + 1]


def compress(seqs: Seqs, k_idx, k_blk, topk: int = KMAX, stream=None):
    d = make_dims(topk)
    _check(lib().qsa_compress(ctypes.byref(d), ctypes.byref(seqs.c),
                              _ptr(k_idx, "k_idx", 2, (seqs.n_k, DI)),
                              _ptr(k_blk, "k_blk", 2, (seqs.n_blocks, DI)), _stream(stream)),
           "qsa_compress")


def select(seqs: Seqs, q_idx, w, k_blk, sel, ws, topk: int = KMAX, stream=None):
    d = make_dims(topk)
    _check(lib().qsa_select(ctypes.byref(d), ctypes.byref(seqs.c),
                            _ptr(q_idx, "q_idx", 2, (seqs.n_q, HI, DI)),
                            _ptr(w, "w", 4, (seqs.n_q, HI)),
                            _ptr(k_blk, "k_blk", 2, (seqs.n_blocks, DI)),
                            _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                            _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "qsa_select")


def score(seqs: Seqs, q_idx, w, k_blk, rows, scores, topk: int = KMAX, stream=None):
    """Indexer scores of the query rows listed in ``rows`` (int64 device tensor) into
    ``scores`` [len(rows), ld] fp32 (-inf past a row's visible blocks)."""
    d = make_dims(topk)
    if rows.dtype.itemsize != 8 or scores.dim() != 2 or scores.shape[0] != rows.numel():
        raise ValueError("rows: int64 [n]; scores: fp32 [n, ld]")
    _check(lib().qsa_score(ctypes.byref(d), ctypes.byref(seqs.c),
                           _ptr(q_idx, "q_idx", 2, (seqs.n_q, HI, DI)),
                           _ptr(w, "w", 4, (seqs.n_q, HI)),
                           _ptr(k_blk, "k_blk", 2, (seqs.n_blocks, DI)),
                           _ptr(rows, "rows", 8), rows.numel(), _ptr(scores, "scores", 4),
                           scores.shape[1], _stream(stream)),
           "qsa_score")


def attend(seqs: Seqs, q, k, v, sel, out, lse, ws, topk: int = KMAX, softmax_scale=0.0,
           stream=None):
    d = make_dims(topk, softmax_scale)
    _check(lib().qsa_attend(ctypes.byref(d), ctypes.byref(seqs.c),
                            _ptr(q, "q", 2, (seqs.n_q, HQ, D)),
                            _ptr(k, "k", 2, (seqs.n_k, HKV, D)),
                            _ptr(v, "v", 2, (seqs.n_k, HKV, D)),
                            _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                            _ptr(out, "out", 4, (seqs.n_q, HQ, D)),
                            _ptr(lse, "lse", 4, (seqs.n_q, HQ)),
                            _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "qsa_attend")


def forward(seqs: Seqs, q, k, v, q_idx, w, k_idx, k_blk, sel, out, lse, ws, topk: int = KMAX,
            softmax_scale=0.0, stream=None):
    """compress (blocks holding query tokens, if k_idx is given) -> select -> attend."""
    d = make_dims(topk, softmax_scale)
    _check(lib().qsa_forward(ctypes.byref(d), ctypes.byref(seqs.c),
                             _ptr(q, "q", 2, (seqs.n_q, HQ, D)),
                             _ptr(k, "k", 2, (seqs.n_k, HKV, D)),
                             _ptr(v, "v", 2, (seqs.n_k, HKV, D)),
                             _ptr(q_idx, "q_idx", 2, (seqs.n_q, HI, DI)),
                             _ptr(w, "w", 4, (seqs.n_q, HI)),
                             _ptr(k_idx, "k_idx", 2, (seqs.n_k, DI)),
                             _ptr(k_blk, "k_blk", 2, (seqs.n_blocks, DI)),
                             _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                             _ptr(out, "out", 4, (seqs.n_q, HQ, D)),
                             _ptr(lse, "lse", 4, (seqs.n_q, HQ)),
                             _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "qsa_forward")


NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(seqs: Seqs, q, k, v, q_idx, w, k_idx, k_blk, sel, out, lse,
                    topk: int = KMAX, softmax_scale=0.0, stream=None):
    """forward() without a workspace: the library's per-GPU scratch array serves as the
    workspace (calls needing more than NOALLOC_SCRATCH_BYTES are refused)."""
    d = make_dims(topk, softmax_scale)
    _check(lib().qsa_forward_noalloc(ctypes.byref(d), ctypes.byref(seqs.c),
                                     _ptr(q, "q", 2, (seqs.n_q, HQ, D)),
                                     _ptr(k, "k", 2, (seqs.n_k, HKV, D)),
                                     _ptr(v, "v", 2, (seqs.n_k, HKV, D)),
                                     _ptr(q_idx, "q_idx", 2, (seqs.n_q, HI, DI)),
                                     _ptr(w, "w", 4, (seqs.n_q, HI)),
                                     _ptr(k_idx, "k_idx", 2, (seqs.n_k, DI)),
                                     _ptr(k_blk, "k_blk", 2, (seqs.n_blocks, DI)),
                                     _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                                     _ptr(out, "out", 4, (seqs.n_q, HQ, D)),
                                     _ptr(lse, "lse", 4, (seqs.n_q, HQ)), _stream(stream)),
           "qsa_forward_noalloc")


def quantize_kv(seqs: Seqs, k, v, k8, v8, k_scale, v_scale, stream=None):
    """FP8 KV cache of bf16 K and V: E4M3 bytes k8 / v8 [Tk, 2, 128] (uint8) and fp32
    scales [Tk, 2] per (token, KV head)."""
    d = make_dims()
    _check(lib().qsa_quantize_kv(ctypes.byref(d), ctypes.byref(seqs.c),
                                 _ptr(k, "k", 2, (seqs.n_k, HKV, D)),
                                 _ptr(v, "v", 2, (seqs.n_k, HKV, D)),
                                 _ptr(k8, "k8", 1, (seqs.n_k, HKV, D)),
                                 _ptr(v8, "v8", 1, (seqs.n_k, HKV, D)),
                                 _ptr(k_scale, "k_scale", 4, (seqs.n_k, HKV)),
                                 _ptr(v_scale, "v_scale", 4, (seqs.n_k, HKV)), _stream(stream)),
           "qsa_quantize_kv")


def attend_fp8(seqs: Seqs, q, k8, v8, k_scale, v_scale, sel, out, lse, ws, topk: int = KMAX,
               softmax_scale=0.0, stream=None):
    d = make_dims(topk, softmax_scale)
    _check(lib().qsa_attend_fp8(ctypes.byref(d), ctypes.byref(seqs.c),
                                _ptr(q, "q", 2, (seqs.n_q, HQ, D)),
                                _ptr(k8, "k8", 1, (seqs.n_k, HKV, D)),
                                _ptr(v8, "v8", 1, (seqs.n_k, HKV, D)),
                                _ptr(k_scale, "k_scale", 4, (seqs.n_k, HKV)),
                                _ptr(v_scale, "v_scale", 4, (seqs.n_k, HKV)),
                                _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                                _ptr(out, "out", 4, (seqs.n_q, HQ, D)),
                                _ptr(lse, "lse", 4, (seqs.n_q, HQ)),
                                _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "qsa_attend_fp8")


def forward_fp8(seqs: Seqs, q, k8, v8, k_scale, v_scale, q_idx, w, k_idx, k_blk, sel, out, lse,
                ws, topk: int = KMAX, softmax_scale=0.0, stream=None):
    """forward() with K and V from the FP8 cache."""
    d = make_dims(topk, softmax_scale)
    _check(lib().qsa_forward_fp8(ctypes.byref(d), ctypes.byref(seqs.c),
                                 _ptr(q, "q", 2, (seqs.n_q, HQ, D)),
                                 _ptr(k8, "k8", 1, (seqs.n_k, HKV, D)),
                                 _ptr(v8, "v8", 1, (seqs.n_k, HKV, D)),
                                 _ptr(k_scale, "k_scale", 4, (seqs.n_k, HKV)),
                                 _ptr(v_scale, "v_scale", 4, (seqs.n_k, HKV)),
                                 _ptr(q_idx, "q_idx", 2, (seqs.n_q, HI, DI)),
                                 _ptr(w, "w", 4, (seqs.n_q, HI)),
                                 _ptr(k_idx, "k_idx", 2, (seqs.n_k, DI)),
                                 _ptr(k_blk, "k_blk", 2, (seqs.n_blocks, DI)),
                                 _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                                 _ptr(out, "out", 4, (seqs.n_q, HQ, D)),
                                 _ptr(lse, "lse", 4, (seqs.n_q, HQ)),
                                 _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "qsa_forward_fp8")


def backward_workspace_size(seqs: Seqs, topk: int = KMAX) -> int:
    d = make_dims(topk)
    n = ctypes.c_size_t(0)
    _check(lib().qsa_backward_workspace_size(ctypes.byref(d), ctypes.byref(seqs.c),
                                             ctypes.byref(n)), "qsa_backward_workspace_size")
    return int(n.value)


def alloc_backward_workspace(seqs: Seqs, topk: int = KMAX, device="cuda"):
    """A zero-filled device buffer of qsa_backward_workspace_size() bytes, 256-byte
    aligned."""
    import torch
    n = backward_workspace_size(seqs, topk)
    buf = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + n] if n > 0 else buf[off:off + 1]


def attend_backward(seqs: Seqs, q, k, v, sel, out, lse, dout, dq, dk, dv, ws, topk: int = KMAX,
                    softmax_scale=0.0, stream=None):
    """Gradients dq [Tq, 24, 128], dk, dv [Tk, 2, 128] (fp32) of the attention over the
    fixed selection sel, given its out and lse and the bf16 gradient dout of out."""
    d = make_dims(topk, softmax_scale)
    _check(lib().qsa_attend_backward(ctypes.byref(d), ctypes.byref(seqs.c),
                                     _ptr(q, "q", 2, (seqs.n_q, HQ, D)),
                                     _ptr(k, "k", 2, (seqs.n_k, HKV, D)),
                                     _ptr(v, "v", 2, (seqs.n_k, HKV, D)),
                                     _ptr(sel, "sel", 4, (seqs.n_q, topk)),
                                     _ptr(out, "out", 4, (seqs.n_q, HQ, D)),
                                     _ptr(lse, "lse", 4, (seqs.n_q, HQ)),
                                     _ptr(dout, "dout", 2, (seqs.n_q, HQ, D)),
                                     _ptr(dq, "dq", 4, (seqs.n_q, HQ, D)),
                                     _ptr(dk, "dk", 4, (seqs.n_k, HKV, D)),
                                     _ptr(dv, "dv", 4, (seqs.n_k, HKV, D)),
                                     _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                                     _stream(stream)),
           "qsa_attend_backward")


class trace:
    """Per-kernel HIP-event timing of the library's launches made inside the block
    (qsa_trace_begin / qsa_trace_end). ``records`` = [(kernel name, ms), ...]."""

    def __init__(self, max_kernels: int = 4096):
        self.cap = int(max_kernels)
        self.records = []

    def __enter__(self):
        _check(lib().qsa_trace_begin(self.cap), "qsa_trace_begin")
        return self

    def __exit__(self, *exc):
        kinds = np.zeros(self.cap, dtype=np.int32)
        ms = np.zeros(self.cap, dtype=np.float32)
        n = lib().qsa_trace_end(self.cap, kinds.ctypes.data, ms.ctypes.data)
        if n < 0:
            raise RuntimeError("qsa_trace_end failed")
        n = min(n, self.cap)
        self.records = [(lib().qsa_kernel_name(int(k)).decode(), float(m))
                        for k, m in zip(kinds[:n], ms[:n])]
        return False

    def mean_ms(self):
        acc = {}
        for name, m in self.records:
            acc.setdefault(name, []).append(m)
        return {k: float(np.mean(v)) for k, v in acc.items()}

    def total_ms(self):
        acc = {}
        for name, m in self.records:
            acc[name] = acc.get(name, 0.0) + m
        return acc
