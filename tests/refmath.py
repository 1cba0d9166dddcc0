"""Independent numpy/scipy formulations used to pin the oracle (tests only).

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
