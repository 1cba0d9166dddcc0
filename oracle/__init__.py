"""CPU oracle of the QSA hot path (ctypes front end of ``oracle/qsa_ref.c``).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package. It shares no code with
the HIP library in ``long_context_block_qsa_amd``; both receive the same seeded
inputs from ``qsa_inputs``.

The C file holds the arithmetic (double precision, step by step, each step citing the
page passage it follows). This module only marshals numpy arrays:
bf16 tensors are ``uint16`` arrays of raw bit patterns, ``w`` is ``float32``,
``cu_q``/``cu_k`` are ``int32`` prefix offsets, outputs are ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_ref.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_ref.so")


def build() -> str:
    """Compile the oracle with the host C compiler (plain C11, -O2)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           _SRC, "-o", _LIB_PATH + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("topk_blocks", ctypes.c_int32), ("softmax_scale", ctypes.c_double)]


@dataclass(frozen=True)
class Dims:
    """Layer dimensions. Defaults are the model's: 24/2 heads of 128, a 4-head x 64
    indexer, 4-token blocks and a 512-block budget."""
    n_q_heads: int = 24
    n_kv_heads: int = 2
    head_dim: int = 128
    n_idx_heads: int = 4
    idx_dim: int = 64
    block_size: int = 4
    topk_blocks: int = 512
    softmax_scale: float = 0.0

    def _c(self) -> _Dims:
        return _Dims(self.n_q_heads, self.n_kv_heads, self.head_dim, self.n_idx_heads,
                     self.idx_dim, self.block_size, self.topk_blocks, self.softmax_scale)


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("QSA_ORACLE_LIB")   # a deliberately mutated build (tests)
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        dp = ctypes.POINTER(_Dims)
        lib.qsa_ref_compress.argtypes = [dp, i32, P, P, P]
        lib.qsa_ref_row_scores.argtypes = [dp, i32, P, P, P, P, P, i64, P, P]
        lib.qsa_ref_select.argtypes = [dp, i32, P, P, P, P, P, P, P, i64, i32]
        lib.qsa_ref_attend.argtypes = [dp, i32, P, P, P, P, P, P, P, P, P, i64, i32]
        lib.qsa_ref_forward.argtypes = [dp, i32, P, P, P, P, P, P, P, P, P, P, P, P,
                                        P, i64, i32]
        lib.qsa_ref_quantize_kv.argtypes = [dp, i32, P, P, P, P, P, P, P]
        lib.qsa_ref_attend_fp8.argtypes = [dp, i32, P, P, P, P, P, P, P, P, P, P, P, i64,
                                           i32]
        lib.qsa_ref_attend_backward.argtypes = [dp, i32, P, P, P, P, P, P, P, P, P, P, P,
                                                i64]
        lib.qsa_ref_bf16_round.argtypes = [ctypes.c_double]
        lib.qsa_ref_bf16_round.restype = ctypes.c_uint16
        lib.qsa_ref_e4m3_round.argtypes = [ctypes.c_double]
        lib.qsa_ref_e4m3_round.restype = ctypes.c_uint8
        lib.qsa_ref_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.qsa_ref_e4m3_value.restype = ctypes.c_double
        for f in ("qsa_ref_compress", "qsa_ref_row_scores", "qsa_ref_select",
                  "qsa_ref_attend", "qsa_ref_forward", "qsa_ref_quantize_kv",
                  "qsa_ref_attend_fp8", "qsa_ref_attend_backward"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _threads(n):
    return int(n if n else min(os.cpu_count() or 1, 16))   # one GPU's share of a shared host


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, int(r.size)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments")


def bf16_round(x: float) -> int:
    """The oracle's double -> bf16 rounding (bit pattern)."""
    return int(_load().qsa_ref_bf16_round(float(x)))


def e4m3_round(x: float) -> int:
    """The oracle's double -> OCP FP8 E4M3 rounding (byte)."""
    return int(_load().qsa_ref_e4m3_round(float(x)))


def e4m3_value(b: int) -> float:
    """The value of an OCP FP8 E4M3 byte."""
    return float(_load().qsa_ref_e4m3_value(int(b)))


def quantize_kv(dims: Dims, cu_k, k, v):
    """FP8 KV cache of bf16 K and V: (k8, v8, k_scale, v_scale)."""
    cu_k = _arr(cu_k, np.int32)
    k, v = _arr(k, np.uint16), _arr(v, np.uint16)
    tk = int(cu_k[-1])
    k8 = np.zeros((tk, dims.n_kv_heads, dims.head_dim), dtype=np.uint8)
    v8 = np.zeros_like(k8)
    ks = np.zeros((tk, dims.n_kv_heads), dtype=np.float32)
    vs = np.zeros_like(ks)
    d = dims._c()
    _check(_load().qsa_ref_quantize_kv(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_k), _ptr(k),
                                       _ptr(v), _ptr(k8), _ptr(v8), _ptr(ks), _ptr(vs)),
           "quantize_kv")
    return k8, v8, ks, vs


def attend_fp8(dims: Dims, cu_q, cu_k, q, k8, v8, k_scale, v_scale, sel, rows=None,
               threads=None):
    """Attention over the dequantized FP8 KV cache. Returns (out, lse)."""
    cu_q, cu_k = _arr(cu_q, np.int32), _arr(cu_k, np.int32)
    q, k8, v8 = _arr(q, np.uint16), _arr(k8, np.uint8), _arr(v8, np.uint8)
    ks, vs = _arr(k_scale, np.float32), _arr(v_scale, np.float32)
    sel = _arr(sel, np.int32)
    tq = int(cu_q[-1])
    out = np.full((tq, dims.n_q_heads, dims.head_dim), np.nan, dtype=np.float64)
    lse = np.full((tq, dims.n_q_heads), np.nan, dtype=np.float64)
    r, nr = _rows(rows)
    d = dims._c()
    _check(_load().qsa_ref_attend_fp8(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_q), _ptr(cu_k),
                                      _ptr(q), _ptr(k8), _ptr(v8), _ptr(ks), _ptr(vs),
                                      _ptr(sel), _ptr(out), _ptr(lse), _ptr(r), nr,
                                      _threads(threads)), "attend_fp8")
    return out, lse


def attend_backward(dims: Dims, cu_q, cu_k, q, k, v, sel, dout, rows=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for attend() over fixed selections.
    With ``rows`` only those query rows contribute (dq of other rows stays 0, dk and dv
    hold those rows' shares)."""
    cu_q, cu_k = _arr(cu_q, np.int32), _arr(cu_k, np.int32)
    q, k, v = _arr(q, np.uint16), _arr(k, np.uint16), _arr(v, np.uint16)
    sel, dout = _arr(sel, np.int32), _arr(dout, np.float64)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    r, nr = _rows(rows)
    d = dims._c()
    _check(_load().qsa_ref_attend_backward(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_q),
                                           _ptr(cu_k), _ptr(q), _ptr(k), _ptr(v), _ptr(sel),
                                           _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(r),
                                           nr), "attend_backward")
    return dq, dk, dv


def n_blocks(dims: Dims, cu_k) -> int:
    lens = np.diff(np.asarray(cu_k, dtype=np.int64))
    return int((lens // dims.block_size).sum())


def compress(dims: Dims, cu_k, k_idx):
    cu_k = _arr(cu_k, np.int32)
    k_idx = _arr(k_idx, np.uint16)
    out = np.zeros((n_blocks(dims, cu_k), dims.idx_dim), dtype=np.uint16)
    d = dims._c()
    _check(_load().qsa_ref_compress(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_k),
                                    _ptr(k_idx), _ptr(out)), "compress")
    return out


def row_scores(dims: Dims, cu_q, cu_k, q_idx, w, k_blk, row: int):
    cu_q, cu_k = _arr(cu_q, np.int32), _arr(cu_k, np.int32)
    q_idx, w, k_blk = _arr(q_idx, np.uint16), _arr(w, np.float32), _arr(k_blk, np.uint16)
    lens = np.diff(cu_k.astype(np.int64))
    buf = np.zeros(int(lens.max(initial=0)) // dims.block_size + 1, dtype=np.float64)
    n = ctypes.c_int64(0)
    d = dims._c()
    _check(_load().qsa_ref_row_scores(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_q),
                                      _ptr(cu_k), _ptr(q_idx), _ptr(w), _ptr(k_blk),
                                      int(row), _ptr(buf), ctypes.byref(n)), "row_scores")
    return buf[:n.value].copy()


def select(dims: Dims, cu_q, cu_k, q_idx, w, k_blk, rows=None, threads=None):
    cu_q, cu_k = _arr(cu_q, np.int32), _arr(cu_k, np.int32)
    q_idx, w, k_blk = _arr(q_idx, np.uint16), _arr(w, np.float32), _arr(k_blk, np.uint16)
    sel = np.full((int(cu_q[-1]), dims.topk_blocks), -2, dtype=np.int32)
    r, nr = _rows(rows)
    d = dims._c()
    _check(_load().qsa_ref_select(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_q), _ptr(cu_k),
                                  _ptr(q_idx), _ptr(w), _ptr(k_blk), _ptr(sel), _ptr(r),
                                  nr, _threads(threads)), "select")
    return sel


def attend(dims: Dims, cu_q, cu_k, q, k, v, sel, rows=None, threads=None):
    cu_q, cu_k = _arr(cu_q, np.int32), _arr(cu_k, np.int32)
    q, k, v = _arr(q, np.uint16), _arr(k, np.uint16), _arr(v, np.uint16)
    sel = _arr(sel, np.int32)
    tq = int(cu_q[-1])
    out = np.full((tq, dims.n_q_heads, dims.head_dim), np.nan, dtype=np.float64)
    lse = np.full((tq, dims.n_q_heads), np.nan, dtype=np.float64)
    r, nr = _rows(rows)
    d = dims._c()
    _check(_load().qsa_ref_attend(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_q), _ptr(cu_k),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out),
                                  _ptr(lse), _ptr(r), nr, _threads(threads)), "attend")
    return out, lse


def forward(dims: Dims, cu_q, cu_k, q, k, v, q_idx, w, k_idx, rows=None, threads=None):
    """compress -> select -> attend. Returns (k_blk, sel, out, lse)."""
    cu_q, cu_k = _arr(cu_q, np.int32), _arr(cu_k, np.int32)
    q, k, v = _arr(q, np.uint16), _arr(k, np.uint16), _arr(v, np.uint16)
    q_idx, w, k_idx = _arr(q_idx, np.uint16), _arr(w, np.float32), _arr(k_idx, np.uint16)
    tq = int(cu_q[-1])
    k_blk = np.zeros((n_blocks(dims, cu_k), dims.idx_dim), dtype=np.uint16)
    sel = np.full((tq, dims.topk_blocks), -2, dtype=np.int32)
    out = np.full((tq, dims.n_q_heads, dims.head_dim), np.nan, dtype=np.float64)
    lse = np.full((tq, dims.n_q_heads), np.nan, dtype=np.float64)
    r, nr = _rows(rows)
    d = dims._c()
    _check(_load().qsa_ref_forward(ctypes.byref(d), len(cu_k) - 1, _ptr(cu_q), _ptr(cu_k),
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(w),
                                   _ptr(k_idx), _ptr(k_blk), _ptr(sel), _ptr(out),
                                   _ptr(lse), _ptr(r), nr, _threads(threads)), "forward")
    return k_blk, sel, out, lse
