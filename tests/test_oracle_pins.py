"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test names the mistake it would catch. Sources of truth: hand-worked examples
(tests/golden), library routines (scipy softmax/logsumexp, torch's bf16 conversion,
integer arithmetic), closed forms and brute force.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as gen
from qsa_inputs import bf16_to_f32, f32_to_bf16_exact
from tests.refmath import (as_f64, attended_mask, causal_mask, masked_gqa_attention,
                          supplied_selection)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    return f32_to_bf16_exact(np.asarray(x, dtype=np.float32))


def _dims(d):
    return oracle.Dims(**d)


# ----------------------------------------------------------------- bf16 rounding

@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (-2.5, 0xC020), (3.0, 0x4040),
    (1 + 2 ** -8, 0x3F80),                 # halfway, ties to even (down)
    (1 + 3 * 2 ** -8, 0x3F82),             # halfway, ties to even (up)
    (1 + 2 ** -8 + 2 ** -20, 0x3F81),      # above halfway rounds up
    ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite bf16
    (2.0 ** 128 - 2.0 ** 119, 0x7F80),     # halfway to 2^128: ties to even -> inf
    (2.0 ** -133, 0x0001),                 # smallest subnormal
    (2.0 ** -134, 0x0000),                 # halfway to zero: even
    (3 * 2.0 ** -134, 0x0002),             # halfway between 1 and 2 quanta: even
    (-0.0, 0x8000),
])
def test_bf16_round_table(x, bits):
    """Catches truncation instead of round-to-nearest-even and exponent slips."""
    assert oracle.bf16_round(x) == bits


def test_bf16_round_matches_torch_on_fp32_values():
    """Library pin: for values exact in fp32, torch's fp32->bf16 is RNE."""
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_round(float(x)) for x in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------- compress

def test_compress_integer_sums_and_ragged_packing():
    """Integer data: each block key must equal the exact integer sum of its 4 rows
    (catches wrong token range, dropped token, packing across sequences); the
    trailing L mod 4 tokens form no block; a 3-token sequence has none."""
    lens = [13, 3, 8, 6]
    p = gen.make_problem(lens, seed=11)
    got = oracle.compress(oracle.Dims(), p.cu_k, p.k_idx)
    ints = bf16_to_f32(p.k_idx).astype(np.int64)
    rows = []
    for b, L in enumerate(lens):
        base = int(p.cu_k[b])
        for blk in range(L // 4):
            rows.append(ints[base + 4 * blk: base + 4 * blk + 4].sum(axis=0))
    assert got.shape == (sum(L // 4 for L in lens), 64)
    assert np.array_equal(bf16_to_f32(got), np.array(rows, dtype=np.float32))


def test_compress_float_data_matches_library_rounding():
    """Normal data: exact double sum, rounded once to bf16 (torch RNE on the exact
    fp32 value). Catches fp32 accumulation, truncation, reordering that rounds."""
    lens = [64, 37]
    p = gen.make_problem(lens, seed=12, float_indexer=True)
    got = oracle.compress(oracle.Dims(), p.cu_k, p.k_idx)
    x = as_f64(p.k_idx)
    sums = []
    for b, L in enumerate(lens):
        base = int(p.cu_k[b])
        for blk in range(L // 4):
            sums.append(x[base + 4 * blk: base + 4 * blk + 4].sum(axis=0))
    sums = np.array(sums)
    f32 = sums.astype(np.float32)
    exact = f32.astype(np.float64) == sums
    assert exact.mean() > 0.99
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[exact], ref[exact])


# --------------------------------------------------------------- worked examples

def _single_query_problem(k_idx_rows, t, q_idx_row, w_row, dims, kv_zero=True):
    """One decode row at position t over a sequence of length t+1. V rows are
    one-hot (V[j] = e_j) and K = 0, so the output is the mean of e_j over J."""
    L = t + 1
    Hq, Hkv, D = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    cu_k = np.array([0, L], dtype=np.int32)
    cu_q = np.array([0, 1], dtype=np.int32)
    k_idx = bf(np.array(k_idx_rows[:L], dtype=np.float32))
    q_idx = bf(np.array(q_idx_row, dtype=np.float32).reshape(1, dims.n_idx_heads, dims.idx_dim))
    w = np.array(w_row, dtype=np.float32).reshape(1, dims.n_idx_heads)
    q = bf(np.ones((1, Hq, D), dtype=np.float32))
    k = bf(np.zeros((L, Hkv, D), dtype=np.float32))
    v = np.zeros((L, Hkv, D), dtype=np.float32)
    for j in range(L):
        v[j, :, j] = 1.0
    return cu_q, cu_k, q, k, bf(v), q_idx, w, k_idx


def test_golden_e1_selection_tie_visibility_tail():
    g = json.load(open(os.path.join(GOLDEN, "e1_micro_blocks.json")))
    dims = _dims(g["dims"])
    kb = oracle.compress(dims, np.array([0, 9], dtype=np.int32), bf(np.array(g["k_idx"], np.float32)))
    assert bf16_to_f32(kb).tolist() == g["k_blk"]
    for case in g["cases"]:
        cu_q, cu_k, q, k, v, q_idx, w, k_idx = _single_query_problem(
            g["k_idx"], case["t"], case["q_idx"], case["w"], dims)
        k_blk, sel, out, lse = oracle.forward(dims, cu_q, cu_k, q, k, v, q_idx, w, k_idx)
        s = oracle.row_scores(dims, cu_q, cu_k, q_idx, w, k_blk, 0)
        assert s.tolist() == case["scores"], case["what"]
        assert sel[0].tolist() == case["sel"], case["what"]
        J = case["J"]
        expect = np.zeros(dims.head_dim)
        expect[J] = 1.0 / len(J)
        assert np.allclose(out[0, 0], expect, atol=1e-15), case["what"]
        assert abs(lse[0, 0] - math.log(len(J))) < 1e-12


def test_golden_e2_two_heads_weights_relu():
    g = json.load(open(os.path.join(GOLDEN, "e2_indexer_scores.json")))
    dims = _dims(g["dims"])
    cu_q, cu_k, q, k, v, q_idx, w, k_idx = _single_query_problem(
        g["k_idx"], g["t"], g["q_idx"], g["w"], dims)
    k_blk, sel, out, lse = oracle.forward(dims, cu_q, cu_k, q, k, v, q_idx, w, k_idx)
    assert bf16_to_f32(k_blk).tolist() == g["k_blk"]
    assert oracle.row_scores(dims, cu_q, cu_k, q_idx, w, k_blk, 0).tolist() == g["scores"]
    assert sel[0].tolist() == g["sel"]
    expect = np.zeros(dims.head_dim)
    expect[g["J"]] = 1.0 / len(g["J"])
    for h in range(dims.n_q_heads):
        assert np.allclose(out[0, h], expect, atol=1e-15)


# ------------------------------------------------------------------- selection

def _brute_force_topk(scores, k):
    """Among all k-subsets of maximal total score, the lexicographically smallest
    sorted index tuple. An optimisation-form definition, independent of sorting."""
    n = len(scores)
    if n <= k:
        return list(range(n))
    best, best_sum = None, None
    for comb in itertools.combinations(range(n), k):
        s = sum(scores[i] for i in comb)
        if best_sum is None or s > best_sum or (s == best_sum and comb < best):
            best, best_sum = comb, s
    return list(best)


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_exhaustive_subsets(seed):
    """Tiny rows with heavy ties (indexer values in {-1,0,1}, 1 head x 2 dims):
    selection == brute-force best subset; output ascending and -1 padded."""
    dims = oracle.Dims(n_q_heads=2, n_kv_heads=1, head_dim=8, n_idx_heads=1, idx_dim=2,
                       topk_blocks=[1, 2, 3, 4, 5, 6][seed])
    rng = np.random.default_rng(seed)
    L = 4 * 14 + int(rng.integers(0, 4))
    cu_k = np.array([0, L], dtype=np.int32)
    cu_q = np.array([0, L], dtype=np.int32)
    k_idx = bf(rng.integers(-1, 2, size=(L, 2)).astype(np.float32))
    q_idx = bf(rng.integers(-1, 2, size=(L, 1, 2)).astype(np.float32))
    w = rng.integers(1, 3, size=(L, 1)).astype(np.float32)
    k_blk = oracle.compress(dims, cu_k, k_idx)
    sel = oracle.select(dims, cu_q, cu_k, q_idx, w, k_blk)
    ties = 0
    for t in range(L):
        s = oracle.row_scores(dims, cu_q, cu_k, q_idx, w, k_blk, t)
        ties += len(s) - len(set(s.tolist()))
        expect = _brute_force_topk(s.tolist(), dims.topk_blocks)
        got = sel[t].tolist()
        assert got[:len(expect)] == expect
        assert all(x == -1 for x in got[len(expect):])
    assert ties > 0


def test_select_all_ties_keeps_lowest_blocks():
    """q_idx = 0: every score is 0, so the first min(nvis, k) blocks are kept."""
    dims = oracle.Dims(topk_blocks=5)
    p = gen.make_problem([50], seed=3)
    q_idx = np.zeros_like(p.q_idx)
    k_blk = oracle.compress(dims, p.cu_k, p.k_idx)
    sel = oracle.select(dims, p.cu_q, p.cu_k, q_idx, p.w, k_blk)
    for t in range(50):
        nv = (t + 1) // 4
        n = min(nv, 5)
        assert sel[t].tolist() == list(range(n)) + [-1] * (5 - n)


def test_select_scale_invariance():
    """Scaling w by 2 or the indexer keys by 2 (exact in bf16) keeps the selection
    (relu is positively homogeneous). Catches a bias or non-homogeneous step."""
    dims = oracle.Dims(topk_blocks=7)
    p = gen.make_problem([203], seed=5)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    s0 = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    s1 = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w * 2, kb)
    k2 = bf(bf16_to_f32(p.k_idx) * 2)
    s2 = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, oracle.compress(dims, p.cu_k, k2))
    assert np.array_equal(s0, s1) and np.array_equal(s0, s2)


def test_needles_selected_decode_32k():
    """Decode 1 x 32,768: every needle block must be among the 512 kept blocks."""
    p = gen.workload_problem("decode_1x32768")
    dims = oracle.Dims()
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    assert set(p.needles[0]) <= set(sel[0].tolist())
    assert (sel[0] >= 0).all() and np.all(np.diff(sel[0]) > 0)


# ------------------------------------------------------------------- attention

def _prefill_dense_check(p, dims, rows_t):
    k_blk, sel, out, lse = oracle.forward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, p.q_idx,
                                          p.w, p.k_idx, rows=rows_t)
    L = int(p.cu_k[1])
    scale = 1 / math.sqrt(dims.head_dim)
    ref_o, ref_l = masked_gqa_attention(as_f64(p.q[rows_t]), as_f64(p.k), as_f64(p.v),
                                        causal_mask(rows_t, L), scale)
    return out[rows_t], lse[rows_t], ref_o, ref_l, sel


def test_dense_equality_when_budget_covers_everything():
    """All blocks fit the budget (L <= 4*512+3): QSA == causal GQA attention
    (library softmax on dense matrices, heads grouped 12:1)."""
    dims = oracle.Dims()
    p = gen.make_problem([300], seed=21)
    rows = list(range(300))
    o, l, ro, rl, sel = _prefill_dense_check(p, dims, rows)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12


def test_dense_equality_prefill_1x1024_sampled_rows():
    dims = oracle.Dims()
    p = gen.workload_problem("prefill_1x1024")
    rows = [0, 1, 2, 3, 4, 511, 512, 1022, 1023]
    o, l, ro, rl, _ = _prefill_dense_check(p, dims, rows)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12


def test_sparse_rows_match_masked_attention():
    """Budget 3 blocks on a 71-token prefill: rows past 15 tokens are sparse. The
    output must equal masked attention over the oracle's kept blocks + raw tail."""
    dims = oracle.Dims(topk_blocks=3)
    p = gen.make_problem([71], seed=22)
    k_blk, sel, out, lse = oracle.forward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, p.q_idx,
                                          p.w, p.k_idx)
    ts = list(range(71))
    mask = attended_mask(ts, sel, 71, 4)
    ro, rl = masked_gqa_attention(as_f64(p.q), as_f64(p.k), as_f64(p.v), mask,
                                  1 / math.sqrt(128))
    assert np.max(np.abs(out - ro)) < 1e-12 and np.max(np.abs(lse - rl)) < 1e-12
    assert mask.sum(axis=1).max() <= 3 * 4 + 3
    assert (mask.sum(axis=1)[15:] >= 12).all()


def test_supplied_selection_reads_to_first_negative_and_skips_invisible_blocks():
    """attend() over a selection from outside: a row's entries are read up to its first
    negative one, and an entry naming a block that is not visible at the row's position
    (reading R6) is not attended. Pinned against masked attention over the blocks that
    count."""
    dims = oracle.Dims(topk_blocks=6)
    L = 45
    p = gen.make_problem([L], seed=29)
    sel, clean = supplied_selection(range(L), 6, 7)
    out, lse = oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel)
    mask = attended_mask(range(L), clean, L, 4)
    ro, rl = masked_gqa_attention(as_f64(p.q), as_f64(p.k), as_f64(p.v), mask,
                                  1 / math.sqrt(128))
    assert np.max(np.abs(out - ro)) < 1e-12 and np.max(np.abs(lse - rl)) < 1e-12
    # the backward takes the same attended set
    dout = gen.bf16_to_f32(gen.make_dout(p, 3)).astype(np.float64)
    g_sup = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, dout)
    g_cln = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, clean, dout)
    for a, b in zip(g_sup, g_cln):
        assert np.array_equal(a, b)


def test_first_token_attends_only_itself():
    """t = 0: the output is V[0] of the head's group exactly; lse = q.k0 * scale."""
    p = gen.make_problem([5], seed=23)
    _, _, out, lse = oracle.forward(oracle.Dims(), p.cu_q, p.cu_k, p.q, p.k, p.v, p.q_idx,
                                    p.w, p.k_idx)
    v = as_f64(p.v)
    for h in range(24):
        assert np.array_equal(out[0, h], v[0, h // 12])
        z = float(as_f64(p.q[0, h]) @ as_f64(p.k[0, h // 12])) / math.sqrt(128)
        assert abs(lse[0, h] - z) < 1e-12


def test_two_keys_logit_gap_ln3():
    """Two keys whose logits differ by ln 3: weights 3/4 and 1/4 (scale = ln 3,
    q.k0 = 1, q.k1 = 0). Catches a wrong exponent base or a missing scale."""
    dims = oracle.Dims(n_q_heads=1, n_kv_heads=1, head_dim=4, softmax_scale=math.log(3))
    cu = np.array([0, 2], dtype=np.int32)
    q = bf(np.array([[[1, 0, 0, 0]]], np.float32))
    k = bf(np.array([[[1, 0, 0, 0]], [[0, 1, 0, 0]]], np.float32))
    v = bf(np.array([[[4, 0, 8, 1]], [[0, 4, 8, -1]]], np.float32))
    q_idx = np.zeros((1, 4, 64), np.uint16)
    w = np.ones((1, 4), np.float32)
    k_idx = np.zeros((2, 64), np.uint16)
    _, _, out, lse = oracle.forward(dims, np.array([0, 1], np.int32), cu, q, k, v, q_idx, w,
                                    k_idx)
    assert np.allclose(out[0, 0], [3, 1, 8, 0.5], atol=1e-14)
    assert abs(lse[0, 0] - (math.log(3) + math.log(4 / 3))) < 1e-14


def test_attention_shift_invariances():
    """K + u (fixed u per kv head) leaves O unchanged; V + c shifts O by c. Values
    are quarter-integers so that every shifted input is exact in bf16."""
    dims = oracle.Dims(topk_blocks=4)
    p = gen.make_problem([61], seed=24)
    rng = np.random.default_rng(0)
    k = bf(np.clip(np.round(bf16_to_f32(p.k) * 4) / 4, -8, 8))
    v = bf(np.clip(np.round(bf16_to_f32(p.v) * 4) / 4, -8, 8))
    u = np.round(rng.standard_normal((1, 2, 128)) * 4).clip(-8, 8).astype(np.float32) / 4
    k2 = bf(bf16_to_f32(k) + u)
    v2 = bf(bf16_to_f32(v) + np.float32(3.0))
    run = lambda kk, vv: oracle.forward(dims, p.cu_q, p.cu_k, p.q, kk, vv, p.q_idx, p.w,
                                        p.k_idx)[2]
    o0 = run(k, v)
    assert np.max(np.abs(run(k2, v) - o0)) < 1e-9
    assert np.max(np.abs(run(k, v2) - (o0 + 3.0))) < 1e-12


def test_decode_equals_last_prefill_row():
    """A decode call at length L is the last row of the prefill of length L."""
    dims = oracle.Dims(topk_blocks=6)
    for L in (1, 3, 4, 29, 40, 77):
        p = gen.make_problem([L], seed=30 + L)
        _, sel_p, out_p, lse_p = oracle.forward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v,
                                                p.q_idx, p.w, p.k_idx)
        cu_q = np.array([0, 1], np.int32)
        _, sel_d, out_d, lse_d = oracle.forward(dims, cu_q, p.cu_k, p.q[-1:], p.k, p.v,
                                                p.q_idx[-1:], p.w[-1:], p.k_idx)
        assert np.array_equal(sel_d[0], sel_p[-1])
        assert np.array_equal(out_d[0], out_p[-1]) and np.array_equal(lse_d[0], lse_p[-1])


def test_ragged_batch_rows_independent():
    """Each sequence of a ragged batch gives the same rows as when run alone."""
    dims = oracle.Dims(topk_blocks=3)
    lens = [23, 3, 18]
    p = gen.make_problem(lens, seed=40)
    _, sel, out, _ = oracle.forward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, p.q_idx, p.w,
                                    p.k_idx)
    for b, L in enumerate(lens):
        k0, k1 = int(p.cu_k[b]), int(p.cu_k[b + 1])
        cu = np.array([0, L], np.int32)
        _, sel1, out1, _ = oracle.forward(dims, cu, cu, p.q[k0:k1], p.k[k0:k1], p.v[k0:k1],
                                          p.q_idx[k0:k1], p.w[k0:k1], p.k_idx[k0:k1])
        assert np.array_equal(sel[k0:k1], sel1) and np.array_equal(out[k0:k1], out1)


# ----------------------------------------------------------------- FP8 KV cache

def _e4m3_probe_values():
    rng = np.random.default_rng(50)
    return np.concatenate([
        rng.uniform(-464.0, 464.0, 20000),          # every binade of the normal range
        rng.normal(0.0, 0.01, 20000),               # subnormals and small normals
        np.arange(-464.0, 464.5, 0.5),              # exact ties in the top binades
        np.ldexp(np.arange(0, 64), -12),            # ties between subnormal steps
    ]).astype(np.float32)


def test_e4m3_round_matches_torch():
    """FP8 rounding (nearest, ties to even, subnormals) equals torch's float8_e4m3fn
    cast on fp32 values up to 464 (catches a wrong quantum, truncation, a wrong bias)."""
    vals = _e4m3_probe_values()
    ours = np.array([oracle.e4m3_round(float(x)) for x in vals], dtype=np.uint8)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes():
    """The value of every E4M3 byte equals torch's decoding (NaN codes included)."""
    ours = np.array([oracle.e4m3_value(b) for b in range(256)])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    ref = ref.numpy()
    assert np.all((ours == ref) | (np.isnan(ours) & np.isnan(ref)))


def test_quantize_kv_matches_library_cast():
    """Per (token, KV head) row: scale = fp32(amax / 448) and bytes = float8_e4m3fn cast
    of the fp32 quotient x / scale, recomputed with torch; every nonzero row reaches 448;
    all-zero rows get scale 1 and zero bytes."""
    dims = oracle.Dims()
    p = gen.make_problem([37, 9], seed=51, qkv_scale=0.5, outlier_frac=0.1)
    p.k[5] = 0                                     # an all-zero token (both heads)
    k8, v8, ks, vs = oracle.quantize_kv(dims, p.cu_k, p.k, p.v)
    for x, q8, sc in ((p.k, k8, ks), (p.v, v8, vs)):
        xf = torch.from_numpy(bf16_to_f32(x).reshape(-1, dims.head_dim))
        amax = xf.abs().amax(dim=1)
        s_ref = torch.where(amax > 0, amax / torch.tensor(448.0, dtype=torch.float32),
                            torch.ones_like(amax))
        assert np.array_equal(sc.reshape(-1), s_ref.numpy())
        q_ref = (xf / s_ref[:, None]).to(torch.float8_e4m3fn)
        assert np.array_equal(q8.reshape(-1, dims.head_dim), q_ref.view(torch.uint8).numpy())
        dec = q_ref.to(torch.float64).abs().amax(dim=1).numpy()
        assert np.all(dec[amax.numpy() > 0] == 448.0)
    assert np.all(k8[5] == 0) and np.all(ks[5] == 1.0)


def test_attend_fp8_lossless_case_equals_bf16():
    """Integer K/V in [-7, 7] with a +-7 in every (token, head) row quantize exactly
    (scale 2^-6, bytes 64*x), so FP8 attention equals bf16 attention bit for bit."""
    dims = oracle.Dims(topk_blocks=5)
    p = gen.make_problem([61, 40], q_lens=[61, 3], seed=52)
    rng = np.random.default_rng(52)
    for name in ("k", "v"):
        x = rng.integers(-7, 8, size=getattr(p, name).shape).astype(np.float32)
        x[..., 0] = np.where(rng.random(x.shape[:-1]) < 0.5, 7.0, -7.0)
        setattr(p, name, bf(x))
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    k8, v8, ks, vs = oracle.quantize_kv(dims, p.cu_k, p.k, p.v)
    assert np.all(ks == 2.0 ** -6) and np.all(vs == 2.0 ** -6)
    out, lse = oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel)
    out8, lse8 = oracle.attend_fp8(dims, p.cu_q, p.cu_k, p.q, k8, v8, ks, vs, sel)
    assert np.array_equal(out, out8) and np.array_equal(lse, lse8)


def test_attend_fp8_matches_masked_attention_on_dequantized_values():
    """FP8 attention of sparse rows equals dense GQA attention (scipy) restricted to the
    attended tokens, computed on the dequantized K and V."""
    dims = oracle.Dims(topk_blocks=4)
    p = gen.make_problem([90], seed=53)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    k8, v8, ks, vs = oracle.quantize_kv(dims, p.cu_k, p.k, p.v)
    deq = lambda q8, s: (torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64)
                         .numpy() * s[..., None].astype(np.float64))
    kd, vd = deq(k8, ks), deq(v8, vs)
    out8, lse8 = oracle.attend_fp8(dims, p.cu_q, p.cu_k, p.q, k8, v8, ks, vs, sel)
    mask = attended_mask(list(range(90)), sel, 90, dims.block_size)
    assert (mask.sum(axis=1)[40:] >= 16).all()     # rows past 19 tokens are sparse
    ref_out, ref_lse = masked_gqa_attention(as_f64(p.q), kd, vd, mask,
                                            1.0 / math.sqrt(dims.head_dim))
    assert np.max(np.abs(out8 - ref_out)) < 1e-12 and np.max(np.abs(lse8 - ref_lse)) < 1e-12


# ----------------------------------------------------------------- attention backward

def _torch_masked_gqa(q, k, v, allowed, scale):
    """Masked dense GQA attention in float64 torch (query head h reads KV head h // 12)."""
    hq, hkv = q.shape[1], k.shape[1]
    kr = k.repeat_interleave(hq // hkv, dim=1)
    vr = v.repeat_interleave(hq // hkv, dim=1)
    logits = torch.einsum("qhd,khd->hqk", q, kr) * scale
    logits = logits.masked_fill(~allowed[None], float("-inf"))
    p = torch.softmax(logits, dim=-1)
    return torch.einsum("hqk,khd->qhd", p, vr)


def test_backward_matches_torch_autograd():
    """dq, dk, dv equal torch autograd (float64) of sum(dout * out) through masked dense
    GQA attention restricted to each row's kept blocks and raw tail (catches a dropped
    softmax-Jacobian term, a wrong scale, a wrong head group, a missing raw tail)."""
    dims = oracle.Dims(topk_blocks=3)
    p = gen.make_problem([45, 30], q_lens=[45, 4], seed=60)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    dout = np.random.default_rng(60).normal(0.0, 1.0, (p.n_q, 24, 128))
    dq, dk, dv = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, dout)
    scale = 1.0 / math.sqrt(128)
    for b in range(2):
        k0, k1 = int(p.cu_k[b]), int(p.cu_k[b + 1])
        q0, q1 = int(p.cu_q[b]), int(p.cu_q[b + 1])
        L, nq = k1 - k0, q1 - q0
        ts = list(range(L - nq, L))
        mask = torch.from_numpy(attended_mask(ts, sel[q0:q1], L, 4))
        qt = torch.tensor(as_f64(p.q[q0:q1]), requires_grad=True)
        kt = torch.tensor(as_f64(p.k[k0:k1]), requires_grad=True)
        vt = torch.tensor(as_f64(p.v[k0:k1]), requires_grad=True)
        out = _torch_masked_gqa(qt, kt, vt, mask, scale)
        (out * torch.from_numpy(dout[q0:q1])).sum().backward()
        assert np.max(np.abs(dq[q0:q1] - qt.grad.numpy())) < 1e-10
        assert np.max(np.abs(dk[k0:k1] - kt.grad.numpy())) < 1e-10
        assert np.max(np.abs(dv[k0:k1] - vt.grad.numpy())) < 1e-10
        assert np.abs(kt.grad.numpy()).max() > 1e-3   # the check is not vacuous


def test_backward_single_key_closed_form():
    """Row t = 0 attends only token 0: the softmax is constant, so dq = 0 and token 0
    gets dv = sum over the row's heads of its group of dout, dk = 0 from that row."""
    dims = oracle.Dims(topk_blocks=2)
    p = gen.make_problem([1], seed=61)
    sel = np.full((1, 2), -1, np.int32)
    dout = np.random.default_rng(61).normal(0.0, 1.0, (1, 24, 128))
    dq, dk, dv = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, dout)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    for g in range(2):
        assert np.allclose(dv[0, g], dout[0, 12 * g:12 * (g + 1)].sum(axis=0), atol=1e-12)


def test_backward_row_subsets_add_up():
    """The loss sum(dout * out) is a sum over query rows, so the gradients restricted to
    a partition of the rows add up to the full ones and each part's dq rows are the full
    dq rows (pins the row-subset option the full-size GPU checks use)."""
    dims = oracle.Dims(topk_blocks=4)
    p = gen.make_problem([60, 23], q_lens=[60, 9], seed=62)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb)
    dout = np.random.default_rng(62).normal(0.0, 1.0, (p.n_q, 24, 128))
    full = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, dout)
    rows = np.random.default_rng(63).permutation(p.n_q)
    a, b = np.sort(rows[:30]), rows[30:]
    ga = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, dout, rows=a)
    gb = oracle.attend_backward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, dout, rows=b)
    for f, x, y in zip(full, ga, gb):
        assert np.max(np.abs(f - (x + y))) < 1e-10
    assert np.array_equal(ga[0][a], full[0][a]) and np.all(ga[0][b] == 0.0)
    assert np.abs(ga[1]).max() > 1e-3 and np.abs(gb[1]).max() > 1e-3


def test_e4m3_round_non_finite():
    """Outside the quantizer's domain: infinities saturate like large finite values (to
    +-448, bytes 0x7E / 0xFE) and NaN gives the NaN pattern with its sign."""
    assert oracle.e4m3_round(float("inf")) == 0x7E
    assert oracle.e4m3_round(float("-inf")) == 0xFE
    assert oracle.e4m3_round(1e300) == 0x7E
    assert oracle.e4m3_round(float("nan")) == 0x7F
