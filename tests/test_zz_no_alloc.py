"""qsa_forward_noalloc (the entry point for callers that cannot allocate) against
qsa_forward, through the C ABI: identical kernels on a workspace that is the library's
per-GPU scratch array instead of a caller buffer, so the results must be identical bit
for bit. Two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents), and a call whose workspace exceeds the scratch is refused
before anything runs."""
import numpy as np
import pytest
import torch

import long_context_block_qsa_amd as qsa
import qsa_inputs as gen
from tests.gpu_helpers import DeviceProblem, host16

pytestmark = pytest.mark.gpu


def _noalloc(dp):
    sel = torch.full_like(dp.sel, -7)
    out = torch.full_like(dp.out, float("nan"))
    lse = torch.full_like(dp.lse, float("nan"))
    qsa.forward_noalloc(dp.seqs, dp.q, dp.k, dp.v, dp.q_idx, dp.w, dp.k_idx, dp.k_blk, sel, out,
                        lse, dp.topk)
    torch.cuda.synchronize()
    return host16(dp.k_blk), sel.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # a decode batch (chunk candidates merged by the attention), then a smaller
    # prefill-shaped call
    (dict(lens=[60000, 30000, 9000], q_lens=[1, 1, 1], topk=512, seed=501),
     dict(lens=[3000, 700], q_lens=[40, 700], topk=64, seed=502)),
    # a decode row past 1,048,576 tokens (selected exactly behind the tile's arrival
    # counter in the control block), then a short decode
    (dict(lens=[1100001], q_lens=[1], topk=512, seed=503),
     dict(lens=[5000], q_lens=[2], topk=128, seed=504)),
])
def test_noalloc_matches_forward(first, second):
    for case in (first, second):
        print(f"\n[case] noalloc lens={case['lens']} q_lens={case['q_lens']}", flush=True)
        p = gen.make_problem(case["lens"], q_lens=case["q_lens"], seed=case["seed"])
        dp = DeviceProblem(p, case["topk"])
        assert qsa.workspace_size(dp.seqs, dp.topk) <= qsa.NOALLOC_SCRATCH_BYTES
        got = _noalloc(dp)
        ref = dp.forward()
        for name, x, y in zip(("k_blk", "sel", "out", "lse"), got, ref):
            assert np.array_equal(x, y), f"{name} differs from qsa_forward"
        again = _noalloc(dp)   # the scratch now holds this call's contents
        for name, x, y in zip(("k_blk", "sel", "out", "lse"), again, ref):
            assert np.array_equal(x, y), f"{name} differs on the repeated call"


def test_noalloc_refuses_oversized_calls():
    """A 65,535-token prefill needs about 262 MiB of workspace: refused, outputs untouched."""
    p = gen.make_problem([65535], q_lens=[65535], seed=505)
    seqs = qsa.Seqs(p.cu_q, p.cu_k)
    assert qsa.workspace_size(seqs) > qsa.NOALLOC_SCRATCH_BYTES
    dp = DeviceProblem(gen.make_problem([70], seed=506), 16)
    small = dp.forward()
    big_out = torch.full((seqs.n_q, qsa.HQ, qsa.D), 3.0, device="cuda")
    with pytest.raises(qsa.QsaError) as e:
        qsa.forward_noalloc(seqs, torch.zeros((seqs.n_q, qsa.HQ, qsa.D), dtype=torch.int16,
                                              device="cuda"),
                            torch.zeros((seqs.n_k, qsa.HKV, qsa.D), dtype=torch.int16,
                                        device="cuda"),
                            torch.zeros((seqs.n_k, qsa.HKV, qsa.D), dtype=torch.int16,
                                        device="cuda"),
                            torch.zeros((seqs.n_q, qsa.HI, qsa.DI), dtype=torch.int16,
                                        device="cuda"),
                            torch.ones((seqs.n_q, qsa.HI), device="cuda"), None,
                            torch.zeros((seqs.n_blocks, qsa.DI), dtype=torch.int16,
                                        device="cuda"),
                            None, big_out, None)
    assert e.value.status == qsa.QSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((big_out == 3.0).all())
    for x, y in zip(_noalloc(dp), small):
        assert np.array_equal(x, y)
