"""FP8 KV cache on the HIP path (through the C ABI) against the CPU oracle.

Bars: E4M3 bytes and scales bit-identical to the oracle's quantisation; selections
bit-identical (indexer inputs are unchanged); attention outputs on the FP8 cache within
max-abs 2e-3 and mean-abs 2e-4 of the oracle's attention on the same FP8 cache, lse
within 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_block_qsa_amd as qsa
import oracle
import qsa_inputs as gen
from tests.gpu_helpers import LSE_ABS, MAX_ABS, MEAN_ABS, DeviceProblem, errs
from tests.refmath import stratified_rows

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)


class Fp8Problem(DeviceProblem):
    def __init__(self, p, topk=None):
        super().__init__(p, topk)
        nk = self.seqs.n_k
        self.k8 = torch.zeros((nk, qsa.HKV, qsa.D), dtype=torch.uint8, device="cuda")
        self.v8 = torch.zeros_like(self.k8)
        self.ks = torch.zeros((nk, qsa.HKV), dtype=torch.float32, device="cuda")
        self.vs = torch.zeros_like(self.ks)
        qsa.quantize_kv(self.seqs, self.k, self.v, self.k8, self.v8, self.ks, self.vs)
        torch.cuda.synchronize()

    def forward_fp8(self):
        qsa.forward_fp8(self.seqs, self.q, self.k8, self.v8, self.ks, self.vs, self.q_idx,
                        self.w, self.k_idx, self.k_blk, self.sel, self.out, self.lse, self.ws,
                        self.topk)
        torch.cuda.synchronize()
        return self.sel.cpu().numpy(), self.out.cpu().numpy(), self.lse.cpu().numpy()

    def attend_fp8(self, sel=None):
        s = self.sel if sel is None else torch.from_numpy(sel).cuda()
        qsa.attend_fp8(self.seqs, self.q, self.k8, self.v8, self.ks, self.vs, s, self.out,
                       self.lse, self.ws, self.topk)
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.lse.cpu().numpy()


def _check(name, fp, rows=None):
    p = fp.p
    dims = oracle.Dims(topk_blocks=fp.topk)
    k8, v8, ks, vs = oracle.quantize_kv(dims, p.cu_k, p.k, p.v)
    assert np.array_equal(fp.k8.cpu().numpy(), k8) and np.array_equal(fp.v8.cpu().numpy(), v8)
    assert np.array_equal(fp.ks.cpu().numpy(), ks) and np.array_equal(fp.vs.cpu().numpy(), vs)
    sel, out, lse = fp.forward_fp8()
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    # selections of every row; attention on `rows` (None: every row)
    sel_r = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    bad = np.nonzero(~np.all(sel == sel_r, axis=1))[0]
    assert bad.size == 0, f"{name}: selection differs on {bad.size} rows, first {bad[:10]}"
    out_r, lse_r = oracle.attend_fp8(dims, p.cu_q, p.cu_k, p.q, k8, v8, ks, vs, sel_r,
                                     rows=rows)
    rows = np.arange(p.n_q) if rows is None else np.asarray(rows)
    mx, mean = errs(out[rows], out_r[rows])
    lmx, _ = errs(lse[rows], lse_r[rows])
    print(f"[{name}] rows={len(rows)} max_abs={mx:.3e} mean_abs={mean:.3e} lse={lmx:.3e}",
          flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lmx <= LSE_ABS
    return sel, out


@pytest.mark.parametrize("lens,q_lens,topk", [
    ([1], None, 1), ([7, 8], None, 1), ([203], None, 8), ([130, 77], None, 16),
    ([1000, 600], None, 64), ([4099], [1], 512), ([3000, 2500, 777, 16], [4, 2, 3, 1], 64),
])
def test_fp8_small(lens, q_lens, topk):
    _banner(f"fp8 lens={lens} q_lens={q_lens} topk={topk}")
    p = gen.make_problem(lens, q_lens=q_lens, seed=400 + sum(lens) + topk)
    _check(f"fp8{lens}", Fp8Problem(p, topk))


def test_fp8_quantize_outliers_and_zero_rows():
    """Outlier keys (x8) and an all-zero token: bytes and scales bit-exact."""
    _banner("fp8 quantize outliers")
    p = gen.make_problem([5000, 333], q_lens=[2, 333], seed=410, qkv_scale=0.5,
                         outlier_frac=0.05)
    p.k[17] = 0
    p.v[4000] = 0
    _check("fp8-outliers", Fp8Problem(p, 128))


def test_fp8_decode_16x262144():
    _banner("fp8: decode 16x262144")
    p = gen.workload_problem("decode_16x262144")
    sel, _ = _check("fp8-decode-16x262144", Fp8Problem(p))
    for b, needles in p.needles.items():
        assert set(needles) <= set(sel[b].tolist())


def test_fp8_decode_long_rows():
    """FP8 decode rows past 64 chunks (a 300,001-token row with 2 query tokens: 74 chunks,
    merged from 2,368 candidates by the attention) and at 1,048,576 tokens (256 chunks)."""
    _banner("fp8: long decode rows")
    p = gen.make_problem([300001, 1 << 20], q_lens=[2, 1], seed=430, needles=8)
    sel, _ = _check("fp8-long-decode", Fp8Problem(p))
    assert set(p.needles[1]) <= set(sel[2].tolist())


def test_fp8_prefill_ragged_64k():
    """Selections of all 113,729 rows bit-exact; attention on every 128th row plus each
    sequence's ends and its dense/sparse boundary."""
    _banner("fp8: ragged prefill 65535/40001/8190/3")
    p = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
    rows = stratified_rows(p.cu_q, p.cu_k, every=128)
    _check("fp8-ragged-64k", Fp8Problem(p), rows)


def test_fp8_forward_equals_select_then_attend():
    _banner("fp8 forward == select + attend")
    p = gen.make_problem([3333, 100], q_lens=[2, 100], seed=420)
    fp = Fp8Problem(p, 32)
    sel, out, lse = fp.forward_fp8()
    fp.sel.fill_(-9)
    assert np.array_equal(fp.select(), sel)
    out2, lse2 = fp.attend_fp8()
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)


def test_fp8_prefill_second_stream_equals_one_stream_and_graph():
    """The ragged FP8 prefill forward attends each selection pass on a second stream while
    the later passes are scored and selected: its outputs equal qsa_select followed by
    qsa_attend_fp8 on one stream, bit for bit, and a HIP graph of the forward (the fork
    and join recorded into it, captured after one eager call has created the second
    stream) replays to the same result, with eager library work between the replays."""
    _banner("fp8: ragged prefill, second stream vs one stream vs graph")
    p = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
    fp = Fp8Problem(p)
    sel, out, lse = fp.forward_fp8()
    fp.sel.fill_(-9)
    assert np.array_equal(fp.select(), sel)
    out2, lse2 = fp.attend_fp8()
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.forward_fp8(fp.seqs, fp.q, fp.k8, fp.v8, fp.ks, fp.vs, fp.q_idx, fp.w, fp.k_idx,
                        fp.k_blk, fp.sel, fp.out, fp.lse, fp.ws, fp.topk)
    for i in range(3):
        fp.sel.fill_(-7)
        fp.out.fill_(float("nan"))
        fp.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(fp.sel.cpu().numpy(), sel), f"replay {i}: selections differ"
        assert np.array_equal(fp.out.cpu().numpy(), out), f"replay {i}: outputs differ"
        assert np.array_equal(fp.lse.cpu().numpy(), lse), f"replay {i}: lse differs"
        s2, o2, l2 = fp.forward_fp8()   # eager work between the replays
        assert np.array_equal(o2, out) and np.array_equal(s2, sel)
