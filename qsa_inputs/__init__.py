"""Seeded synthetic inputs for the QSA hot path (shared by the oracle checks, the GPU
tests and the benchmark). Holds none of the method's arithmetic.

Every tensor element comes from a counter-based stream (``qsa_gen.c``): element i of
tensor id ``tid`` under ``seed`` is a pure function of (seed, tid, i). Tensor ids:
Q 1, K 2, V 3, q_idx 4, k_idx 5, w 6, needle placement 7, outlier mask 8.

The five workloads (sizes and value laws of the layer's published shape: 24 query
heads over 2 KV heads of 128, a 4-head x 64 indexer, 4-token blocks, a 512-block
budget, 256K native context):

=================================  ===========================  ================================
workload (seed)                    shape                        values / structure
=================================  ===========================  ================================
prefill_1x1024 (1000)              prefill, 1 x 1,024 tokens    Q,K,V ~ N(0,1); indexer ints
                                                                U{-3..3}; w in {1,2}; all dense
decode_1x32768 (1001)              decode, 1 x 32,768 context   as above, plus 16 needle blocks
prefill_1x16384 (1002)             prefill, 1 x 16,384 tokens   as above
decode_16x262144 (1003)            decode, 16 x 262,144 ctx     as above, plus 32 needle blocks
                                                                per sequence
prefill_ragged_65535_40001_8190_3  ragged prefill 65,535 /      Q,K,V ~ N(0, 0.5^2); 5% of K
(1004)                             40,001 / 8,190 / 3           rows (token, kv-head) scaled x8
=================================  ===========================  ================================

A needle block of a decode sequence gets indexer keys +3 * sgn(u) on all its tokens,
u = sum_h w_h * q_idx[h] of that sequence's query (sgn(0) = +1), so its score is at
least 12 * |u|_1 and it must be selected.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_gen.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_gen.so")

TID_Q, TID_K, TID_V, TID_QIDX, TID_KIDX, TID_W, TID_NEEDLE, TID_OUTLIER = 1, 2, 3, 4, 5, 6, 7, 8
TID_DOUT = 9

HQ, HKV, D, HI, DI, BS, TOPK = 24, 2, 128, 4, 64, 4, 512


def build() -> str:
    cmd = ["gcc", "-O2", "-std=gnu11", "-Wall", "-shared", "-fPIC", _SRC,
           "-o", _LIB_PATH + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, P, c_int = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
        lib.qsa_gen_normal_bf16.argtypes = [u64, u32, u64, u64, ctypes.c_double, P, c_int]
        lib.qsa_gen_uniform_int_bf16.argtypes = [u64, u32, u64, u64, ctypes.c_int32,
                                                 ctypes.c_int32, P, c_int]
        lib.qsa_gen_weights.argtypes = [u64, u32, u64, u64, P, c_int]
        lib.qsa_gen_u64.argtypes = [u64, u32, u64, u64, P, c_int]
        for f in ("qsa_gen_normal_bf16", "qsa_gen_uniform_int_bf16", "qsa_gen_weights",
                  "qsa_gen_u64"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _nthreads(threads):
    return int(threads or min(os.cpu_count() or 1, 16))


def normal_bf16(seed, tid, n, scale=1.0, offset=0, threads=None):
    out = np.empty(int(n), dtype=np.uint16)
    _load().qsa_gen_normal_bf16(seed, tid, offset, out.size, float(scale),
                                out.ctypes.data_as(ctypes.c_void_p), _nthreads(threads))
    return out


def uniform_int_bf16(seed, tid, n, lo, hi, offset=0, threads=None):
    out = np.empty(int(n), dtype=np.uint16)
    _load().qsa_gen_uniform_int_bf16(seed, tid, offset, out.size, int(lo), int(hi),
                                     out.ctypes.data_as(ctypes.c_void_p), _nthreads(threads))
    return out


def weights(seed, tid, n, offset=0, threads=None):
    out = np.empty(int(n), dtype=np.float32)
    _load().qsa_gen_weights(seed, tid, offset, out.size,
                            out.ctypes.data_as(ctypes.c_void_p), _nthreads(threads))
    return out


def raw_u64(seed, tid, n, offset=0, threads=None):
    out = np.empty(int(n), dtype=np.uint64)
    _load().qsa_gen_u64(seed, tid, offset, out.size, out.ctypes.data_as(ctypes.c_void_p),
                        _nthreads(threads))
    return out


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_exact(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)


@dataclass
class Problem:
    """One batch of QSA inputs (host arrays; bf16 as uint16 bit patterns)."""
    cu_q: np.ndarray
    cu_k: np.ndarray
    q: np.ndarray          # [Tq, HQ, D]
    k: np.ndarray          # [Tk, HKV, D]
    v: np.ndarray          # [Tk, HKV, D]
    q_idx: np.ndarray      # [Tq, HI, DI]
    w: np.ndarray          # [Tq, HI] float32
    k_idx: np.ndarray      # [Tk, DI]
    topk: int = TOPK
    needles: dict = field(default_factory=dict)  # seq -> sorted needle block ids
    name: str = "custom"

    @property
    def batch(self):
        return len(self.cu_k) - 1

    @property
    def n_q(self):
        return int(self.cu_q[-1])

    @property
    def n_k(self):
        return int(self.cu_k[-1])


def make_problem(lens, q_lens=None, seed=1234, qkv_scale=1.0, outlier_frac=0.0,
                 outlier_mul=8.0, needles=0, topk=TOPK, idx_lo=-3, idx_hi=3,
                 float_indexer=False, threads=None, name="custom"):
    """Build a batch. ``lens`` are sequence lengths; ``q_lens`` the number of query
    tokens per sequence (its last tokens); default = lens (prefill)."""
    lens = [int(x) for x in lens]
    q_lens = list(lens) if q_lens is None else [int(x) for x in q_lens]
    if len(q_lens) != len(lens) or any(a < 0 or a > b for a, b in zip(q_lens, lens)):
        raise ValueError("each q_len must be in [0, len]")
    cu_k = np.zeros(len(lens) + 1, dtype=np.int32)
    cu_q = np.zeros(len(lens) + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(lens)
    cu_q[1:] = np.cumsum(q_lens)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    th = _nthreads(threads)

    q = normal_bf16(seed, TID_Q, tq * HQ * D, qkv_scale, threads=th).reshape(tq, HQ, D)
    k = normal_bf16(seed, TID_K, tk * HKV * D, qkv_scale, threads=th).reshape(tk, HKV, D)
    v = normal_bf16(seed, TID_V, tk * HKV * D, qkv_scale, threads=th).reshape(tk, HKV, D)
    if float_indexer:
        q_idx = normal_bf16(seed, TID_QIDX, tq * HI * DI, threads=th).reshape(tq, HI, DI)
        k_idx = normal_bf16(seed, TID_KIDX, tk * DI, threads=th).reshape(tk, DI)
    else:
        q_idx = uniform_int_bf16(seed, TID_QIDX, tq * HI * DI, idx_lo, idx_hi,
                                 threads=th).reshape(tq, HI, DI)
        k_idx = uniform_int_bf16(seed, TID_KIDX, tk * DI, idx_lo, idx_hi,
                                 threads=th).reshape(tk, DI)
    w = weights(seed, TID_W, tq * HI, threads=th).reshape(tq, HI)

    if outlier_frac > 0.0:
        draws = raw_u64(seed, TID_OUTLIER, tk * HKV, threads=th).reshape(tk, HKV)
        mask = draws < np.uint64(int(outlier_frac * 2.0 ** 64))
        kf = bf16_to_f32(k[mask])
        k[mask] = f32_to_bf16_exact(kf * np.float32(outlier_mul))

    placed = {}
    if needles:
        for b, (L, nq) in enumerate(zip(lens, q_lens)):
            if nq == 0:
                continue
            nb = L // BS
            if nb - 1 < needles:
                raise ValueError("sequence too short for its needles")
            r = int(cu_q[b + 1]) - 1            # the sequence's last query row
            u = (bf16_to_f32(q_idx[r]).astype(np.float64)
                 * w[r].astype(np.float64)[:, None]).sum(axis=0)
            pattern = f32_to_bf16_exact(np.where(u >= 0, 3.0, -3.0).astype(np.float32))
            chosen, j = [], 0
            while len(chosen) < needles:
                d = raw_u64(seed, TID_NEEDLE, 1, offset=b * 1_000_000 + j)[0]
                j += 1
                blk = int(d % np.uint64(nb - 1))   # never the query's own block
                if blk not in chosen:
                    chosen.append(blk)
            for blk in chosen:
                t0 = int(cu_k[b]) + blk * BS
                k_idx[t0:t0 + BS, :] = pattern[None, :]
            placed[b] = sorted(chosen)

    return Problem(cu_q=cu_q, cu_k=cu_k, q=q, k=k, v=v, q_idx=q_idx, w=w, k_idx=k_idx,
                   topk=int(topk), needles=placed, name=name)


def make_dout(p: "Problem", seed: int, scale: float = 1.0, threads=None) -> np.ndarray:
    """Gradient of the attention output for a backward pass: bf16 ~N(0, scale^2) bits,
    [Tq, HQ, D]."""
    return normal_bf16(seed, TID_DOUT, p.n_q * HQ * D, scale,
                       threads=_nthreads(threads)).reshape(p.n_q, HQ, D)


# The benchmark and parity workloads, by name, each with its own seed.
WORKLOADS = {
    "prefill_1x1024": dict(seed=1000, lens=[1024]),
    "decode_1x32768": dict(seed=1001, lens=[32768], q_lens=[1], needles=16),
    "prefill_1x16384": dict(seed=1002, lens=[16384]),
    "decode_16x262144": dict(seed=1003, lens=[262144] * 16, q_lens=[1] * 16, needles=32),
    "prefill_ragged_65535_40001_8190_3": dict(seed=1004, lens=[65535, 40001, 8190, 3],
                                              qkv_scale=0.5, outlier_frac=0.05,
                                              outlier_mul=8.0),
    # one prefill at the native context (values as prefill_1x1024)
    "prefill_1x262144": dict(seed=1005, lens=[262144]),
}


def workload_problem(name: str, seed: int | None = None, threads=None) -> Problem:
    """The named workload with its own seed (unless one is given)."""
    c = dict(WORKLOADS[name])
    s0 = c.pop("seed")
    return make_problem(seed=s0 if seed is None else seed, threads=threads, name=name, **c)
