"""Attention backward on the HIP path (through the C ABI) against the CPU oracle.

The GPU forward gives sel, out and lse; the GPU backward takes those and a seeded bf16
dout. The oracle selects on its own (the selections must be bit-identical) and
differentiates its fp64 attention over that selection. Bars: dq, dk and dv within
max-abs 5e-4 and mean-abs 2e-5 of the oracle's, absolute. Measured on every case here
(gradients up to 25 in magnitude, sums of up to ~10^5 fp32 terms): max-abs at most
1.0e-4 and mean-abs at most 6e-7, so the bars sit 5x and 30x above the worst measured
errors and a regression of one order of magnitude fails.
"""
import numpy as np
import pytest
import torch

import long_context_block_qsa_amd as qsa
import oracle
import qsa_inputs as gen
from tests.gpu_helpers import DeviceProblem, dev16, errs
from tests.refmath import row_positions, supplied_selection

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


GRAD_MAX_ABS, GRAD_MEAN_ABS = 5e-4, 2e-5


def _bars(name, got, ref, mask=None):
    if mask is not None:
        got, ref = got[mask], ref[mask]
    mx, mean = errs(got, ref)
    print(f"[{name}] max|ref|={np.abs(ref).max(initial=0.0):.3e} max_abs={mx:.3e} "
          f"mean_abs={mean:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert mx <= GRAD_MAX_ABS and mean <= GRAD_MEAN_ABS, name


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


def test_backward_row_windows():
    """More than 8192 query rows in a sequence: dK/dV are summed over row windows in
    successive launches (the second window adds to the first)."""
    _banner("backward 9000-row prefill, two row windows")
    p = gen.make_problem([9000, 50], seed=540)
    _check("bwd-9000", BwdProblem(p, 8))


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


def _attending_rows(p, dims, kb, seq, blk):
    """Rows of sequence `seq` that attend its key block `blk` by the oracle's own
    selection: rows whose kept blocks hold it, and rows whose raw tail lies in it.
    Returns (candidate rows, their oracle selections, attending rows)."""
    q0, q1 = int(p.cu_q[seq]), int(p.cu_q[seq + 1])
    L = int(p.cu_k[seq + 1] - p.cu_k[seq])
    t0 = L - (q1 - q0)
    cand = np.array([r for r in range(q0, q1) if t0 + (r - q0) >= 4 * blk], dtype=np.int64)
    sel_c = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb, rows=cand)
    att = []
    for r in cand:
        t = t0 + (r - q0)
        nv = (t + 1) // 4
        if blk in set(sel_c[r][sel_c[r] >= 0].tolist()) or (nv == blk and t + 1 > 4 * nv):
            att.append(int(r))
    return cand, sel_c, np.array(att, dtype=np.int64)


def test_backward_prefill_ragged_64k_sampled():
    """The ragged 4-sequence prefill (65535/40001/8190/3 tokens, budget 512) at full size:
    dq on sampled rows, dk and dv on sampled key blocks (from the oracle over exactly the
    rows that attend them: late blocks of each sequence, the partial final blocks)."""
    _banner("backward: ragged prefill 65535/40001/8190/3")
    p = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
    bp = BwdProblem(p, 512)
    _, sel, _, _ = bp.forward()
    dq, dk, dv = bp.backward()
    dims = oracle.Dims(topk_blocks=512)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    dout = gen.bf16_to_f32(bp.dout_np).astype(np.float64)

    cu = p.cu_q
    rng = np.random.default_rng(45)
    rows = set()
    for b in range(4):
        lo, hi = int(cu[b]), int(cu[b + 1])
        rows.update(range(lo, min(hi, lo + 3)))
        rows.update(range(max(lo, hi - 3), hi))
        if hi - lo > 10:
            rows.update(rng.integers(lo, hi, 6).tolist())
    rows = np.array(sorted(rows), dtype=np.int64)
    sel_r = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb, rows=rows)
    assert np.array_equal(sel[rows], sel_r[rows])
    dq_r, _, _ = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel_r, dout,
                                        rows=rows)
    _bars("ragged-64k dq (sampled rows)", dq[rows], dq_r[rows])

    for seq, blk in ((0, 16383), (0, 16150), (1, 9800), (2, 1950), (3, 0)):
        cand, sel_c, att = _attending_rows(p, dims, kb, seq, blk)
        assert np.array_equal(sel[cand], sel_c[cand]), (seq, blk)
        assert att.size > 0
        _, dk_r, dv_r = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel_c,
                                               dout, rows=att)
        k0 = int(p.cu_k[seq]) + 4 * blk
        k1 = min(k0 + 4, int(p.cu_k[seq + 1]))
        print(f"  block ({seq}, {blk}): {att.size} attending rows of {cand.size}", flush=True)
        _bars(f"ragged-64k dk block ({seq},{blk})", dk[k0:k1], dk_r[k0:k1])
        _bars(f"ragged-64k dv block ({seq},{blk})", dv[k0:k1], dv_r[k0:k1])


def test_backward_supplied_selection_invalid_entries():
    """Gradients over a caller's selection with an invisible block id and entries after a
    -1: only the blocks that count are differentiated, like the oracle."""
    _banner("backward over a supplied selection with invalid entries")
    p = gen.make_problem([1200, 700, 5], q_lens=[1200, 3, 5], seed=570)
    bp = BwdProblem(p, 8)
    sel, clean = supplied_selection(row_positions(p.cu_q, p.cu_k), 8, 15)
    bp.sel.copy_(torch.from_numpy(sel).cuda())
    bp.attend()
    dq, dk, dv = bp.backward()
    dims = oracle.Dims(topk_blocks=8)
    dout = gen.bf16_to_f32(bp.dout_np).astype(np.float64)
    dq_r, dk_r, dv_r = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, clean, dout)
    _bars("supplied dq", dq, dq_r)
    _bars("supplied dk", dk, dk_r)
    _bars("supplied dv", dv, dv_r)
