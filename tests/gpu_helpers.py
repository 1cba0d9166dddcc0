"""Moving seeded problems to the device and running the library (GPU tests only)."""
from __future__ import annotations

import numpy as np
import torch

import long_context_block_qsa_amd as qsa


def dev16(a: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DeviceProblem:
    def __init__(self, p, topk=None):
        self.p = p
        self.topk = int(topk or p.topk)
        self.seqs = qsa.Seqs(p.cu_q, p.cu_k)
        self.q, self.k, self.v = dev16(p.q), dev16(p.k), dev16(p.v)
        self.q_idx, self.k_idx = dev16(p.q_idx), dev16(p.k_idx)
        self.w = torch.from_numpy(np.ascontiguousarray(p.w)).cuda()
        nb = self.seqs.n_blocks
        self.k_blk = torch.zeros((nb, qsa.DI), dtype=torch.int16, device="cuda")
        tq = self.seqs.n_q
        self.sel = torch.full((tq, self.topk), -7, dtype=torch.int32, device="cuda")
        self.out = torch.full((tq, qsa.HQ, qsa.D), float("nan"), device="cuda")
        self.lse = torch.full((tq, qsa.HQ), float("nan"), device="cuda")
        self.ws = qsa.alloc_workspace(self.seqs, self.topk)
        # the compressed-key cache a decode step reads (built once, as at prefill time)
        if nb > 0:
            qsa.compress(self.seqs, self.k_idx, self.k_blk, self.topk)

    def forward(self, with_k_idx=True):
        qsa.forward(self.seqs, self.q, self.k, self.v, self.q_idx, self.w,
                    self.k_idx if with_k_idx else None, self.k_blk, self.sel, self.out,
                    self.lse, self.ws, self.topk)
        torch.cuda.synchronize()
        return (host16(self.k_blk), self.sel.cpu().numpy(), self.out.cpu().numpy(),
                self.lse.cpu().numpy())

    def compress(self):
        qsa.compress(self.seqs, self.k_idx, self.k_blk, self.topk)
        torch.cuda.synchronize()
        return host16(self.k_blk)

    def select(self):
        qsa.select(self.seqs, self.q_idx, self.w, self.k_blk, self.sel, self.ws, self.topk)
        torch.cuda.synchronize()
        return self.sel.cpu().numpy()

    def attend(self, sel_np=None):
        sel = self.sel if sel_np is None else torch.from_numpy(
            np.ascontiguousarray(sel_np, dtype=np.int32)).cuda()
        qsa.attend(self.seqs, self.q, self.k, self.v, sel, self.out, self.lse, self.ws,
                   self.topk)
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.lse.cpu().numpy()


def errs(a, b):
    d = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    return float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0


MAX_ABS, MEAN_ABS, LSE_ABS = 2e-3, 2e-4, 1e-4
