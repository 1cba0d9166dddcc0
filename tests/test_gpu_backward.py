"""Attention backward on the HIP path (through the C ABI) against the CPU oracle.

The GPU forward gives sel, out and lse; the GPU backward takes those and a seeded bf16
dout. The oracle selects on its own (the selections must be bit-identical) and
differentiates its fp64 attention over that selection. Bars: dq, dk and dv within
max-abs 2e-3 * s and mean-abs 2e-4 * s of the oracle's, with s = max(1, max |oracle|)
per tensor (the forward's absolute bars, scaled when a gradient is larger than 1: the
GPU sums in fp32, so its error grows with the magnitude of the sum).
"""
import numpy as np
import pytest
import torch

import long_context_block_qsa_amd as qsa
import oracle
import qsa_inputs as gen
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, DeviceProblem, dev16, errs

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)


class BwdProblem(DeviceProblem):
    def __init__(self, p, topk=None, dout_seed=900):
        super().__init__(p, topk)
        self.dout_np = gen.make_dout(p, dout_seed)
        self.dout = dev16(self.dout_np)
        tq, tk = self.seqs.n_q, self.seqs.n_k
        self.dq = torch.full((tq, qsa.HQ, qsa.D), float("nan"), device="cuda")
        self.dk = torch.full((tk, qsa.HKV, qsa.D), float("nan"), device="cuda")
        self.dv = torch.full((tk, qsa.HKV, qsa.D), float("nan"), device="cuda")
        self.bws = qsa.alloc_backward_workspace(self.seqs, self.topk)

    def backward(self):
        qsa.attend_backward(self.seqs, self.q, self.k, self.v, self.sel, self.out, self.lse,
                            self.dout, self.dq, self.dk, self.dv, self.bws, self.topk)
        torch.cuda.synchronize()
        return self.dq.cpu().numpy(), self.dk.cpu().numpy(), self.dv.cpu().numpy()


def _bars(name, got, ref, mask=None):
    if mask is not None:
        got, ref = got[mask], ref[mask]
    s = max(1.0, float(np.abs(ref).max(initial=0.0)))
    mx, mean = errs(got, ref)
    print(f"[{name}] max|ref|={np.abs(ref).max(initial=0.0):.3e} max_abs={mx:.3e} "
          f"mean_abs={mean:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert mx <= MAX_ABS * s and mean <= MEAN_ABS * s, name


def _check(name, bp):
    p = bp.p
    _, sel, _, _ = bp.forward()
    dq, dk, dv = bp.backward()
    dims = oracle.Dims(topk_blocks=bp.topk)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    sel_r = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    assert np.array_equal(sel, sel_r), f"{name}: selections differ"
    dout = gen.bf16_to_f32(bp.dout_np).astype(np.float64)
    dq_r, dk_r, dv_r = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel_r, dout)
    _bars(f"{name} dq", dq, dq_r)
    _bars(f"{name} dk", dk, dk_r)
    _bars(f"{name} dv", dv, dv_r)
    return dq, dk, dv


@pytest.mark.parametrize("lens,q_lens,topk", [
    ([1], None, 1),                      # a single token: its own raw tail only
    ([7, 1, 2, 3, 0, 64], None, 4),      # tiny and empty sequences, tails of 1..3 tokens
    ([300, 45], [9, 45], 16),            # sparse decode tail + a dense short prefill
    ([1023], None, 32),                  # 4 row chunks, sparse rows past position 131
    ([700, 2100], [700, 1], 64),         # prefill next to a decode row
    ([5000], [3], 512),                  # the model's budget on a few long rows
    ([1000, 600], None, 128),            # rows within and beyond the budget
])
def test_backward_small(lens, q_lens, topk):
    _banner(f"backward lens={lens} q_lens={q_lens} topk={topk}")
    p = gen.make_problem(lens, q_lens=q_lens, seed=500 + sum(lens) + topk)
    _check(f"bwd{lens}", BwdProblem(p, topk))


def test_backward_outlier_keys():
    """Outlier keys (x8) make peaked softmax rows."""
    _banner("backward outlier keys")
    p = gen.make_problem([1500, 333], q_lens=[1500, 5], seed=510, qkv_scale=0.5,
                         outlier_frac=0.05)
    _check("bwd-outliers", BwdProblem(p, 48))


def test_backward_two_lds_passes():
    """More than 16384 key blocks in one sequence: the index kernels count and fill in
    two passes over the blocks."""
    _banner("backward 70001-token context, 3 query rows")
    p = gen.make_problem([70001], q_lens=[3], seed=520)
    _check("bwd-70001", BwdProblem(p, 512))


def test_backward_is_deterministic():
    """Two calls give bit-identical gradients (no atomics in the accumulation)."""
    _banner("backward determinism")
    p = gen.make_problem([2000, 900], q_lens=[2000, 4], seed=530)
    bp = BwdProblem(p, 64)
    bp.forward()
    a = bp.backward()
    bp.dq.fill_(float("nan"))
    bp.dk.fill_(float("nan"))
    bp.dv.fill_(float("nan"))
    bp.bws.fill_(0x5A)   # stale workspace contents must not matter
    b = bp.backward()
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
