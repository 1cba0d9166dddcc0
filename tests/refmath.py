"""Independent numpy/scipy formulations used to pin the oracle, and the row samplers
of the parity tests (tests only).

Each function restates a special case through a library routine: masked softmax
attention through scipy's ``softmax``/``logsumexp`` on dense matrices, block keys
through integer sums and torch's float32 -> bfloat16 conversion. None of them is
used by the oracle or by the HIP library.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp, softmax

from qsa_inputs import bf16_to_f32


def as_f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


def masked_gqa_attention(q, k, v, allowed, scale):
    """q [Tq,Hq,D], k/v [Tk,Hkv,D] (float64); allowed [Tq,Tk] bool.
    Query head h reads key/value head h // (Hq // Hkv)."""
    hq, hkv = q.shape[1], k.shape[1]
    kr = np.repeat(k, hq // hkv, axis=1)          # [Tk, Hq, D], contiguous groups
    vr = np.repeat(v, hq // hkv, axis=1)
    logits = np.einsum("qhd,khd->hqk", q, kr) * scale
    logits = np.where(allowed[None, :, :], logits, -np.inf)
    p = softmax(logits, axis=-1)
    out = np.einsum("hqk,khd->qhd", p, vr)
    lse = logsumexp(logits, axis=-1).T             # [Tq, Hq]
    return out, lse


def attended_mask(t_list, sel_rows, L, block_size):
    """Boolean [len(t_list), L]: the kept blocks' tokens plus the raw tail."""
    m = np.zeros((len(t_list), L), dtype=bool)
    for i, t in enumerate(t_list):
        nv = (t + 1) // block_size
        for b in sel_rows[i]:
            if b >= 0:
                m[i, b * block_size:(b + 1) * block_size] = True
        m[i, nv * block_size:t + 1] = True
    return m


def causal_mask(t_list, L):
    m = np.zeros((len(t_list), L), dtype=bool)
    for i, t in enumerate(t_list):
        m[i, :t + 1] = True
    return m


def row_positions(cu_q, cu_k):
    """Position t of every query row: a sequence's queries are its last tokens."""
    ts = []
    for b in range(len(cu_q) - 1):
        L, nq = int(cu_k[b + 1] - cu_k[b]), int(cu_q[b + 1] - cu_q[b])
        ts.extend(range(L - nq, L))
    return ts


def supplied_selection(ts, topk, seed):
    """A selection as a caller might supply it (topk >= 6): per row up to 3 visible blocks
    (ascending), then an id of a block that is not visible at the row's position, a -1 and
    one more visible id after it. Returns (selection, the same with only the blocks that
    count, -1 padded)."""
    rng = np.random.default_rng(seed)
    sel = np.full((len(ts), topk), -1, np.int32)
    clean = np.full((len(ts), topk), -1, np.int32)
    for i, t in enumerate(ts):
        nv = (t + 1) // 4
        vis = sorted(rng.choice(nv, size=min(nv, 3), replace=False).tolist()) if nv else []
        row = vis + [nv + 2 + t % 3, -1] + ([0] if nv else [])
        sel[i, :len(row)] = row
        clean[i, :len(vis)] = vis
    return sel, clean


def stratified_rows(cu_q, cu_k, every=64, edge=8, boundary=(2040, 2062)):
    """Every `every`-th query row, plus each sequence's first and last `edge` rows and
    the rows around the dense/sparse boundary (positions 2,040..2,061: 2,051 is the
    first position with more visible blocks than the 512-block budget)."""
    rows = set(range(0, int(cu_q[-1]), every))
    for b in range(len(cu_q) - 1):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        L = int(cu_k[b + 1] - cu_k[b])
        rows.update(range(lo, min(hi, lo + edge)))
        rows.update(range(max(lo, hi - edge), hi))
        for t in range(*boundary):
            r = lo + t - (L - (hi - lo))
            if lo <= r < hi:
                rows.add(r)
    return sorted(rows)
