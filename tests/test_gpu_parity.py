"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by element.

Bars: compressed keys and selected block ids bit-identical (indexer inputs are small
integers, so every score is exact in fp32); attention outputs within max-abs 2e-3 and
mean-abs 2e-4 of the oracle, lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_block_qsa_amd as qsa
import oracle
import qsa_inputs as gen
from tests.refmath import row_positions, stratified_rows, supplied_selection
from tests.gpu_helpers import LSE_ABS, MAX_ABS, MEAN_ABS, DeviceProblem, errs, host16

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)


def _check_rows(name, dp, rows, topk, threads=None, gpu=None):
    p = dp.p
    dims = oracle.Dims(topk_blocks=topk)
    k_blk_r, sel_r, out_r, lse_r = oracle.forward(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, p.q_idx,
                                                  p.w, p.k_idx, rows=rows, threads=threads)
    k_blk, sel, out, lse = gpu if gpu is not None else dp.forward()
    assert np.array_equal(k_blk, k_blk_r), f"{name}: compressed keys differ"
    rows = np.arange(p.n_q) if rows is None else np.asarray(rows)
    bad = [r for r in rows if not np.array_equal(sel[r], sel_r[r])]
    assert not bad, f"{name}: selection differs on rows {bad[:10]}"
    mx, mean = errs(out[rows], out_r[rows])
    lmx, _ = errs(lse[rows], lse_r[rows])
    print(f"[{name}] rows={len(rows)} max_abs={mx:.3e} mean_abs={mean:.3e} lse={lmx:.3e}",
          flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lmx <= LSE_ABS
    return sel, out


# ----------------------------------------------------------------- small shapes

SMALL = [
    ([1], 1), ([2], 1), ([3], 2), ([4], 1), ([5], 1), ([7, 8], 1), ([13], 2), ([64], 3),
    ([64, 3, 0, 29], 8), ([203], 8), ([130, 77], 16), ([1000, 600], 64),
]


@pytest.mark.parametrize("lens,topk", SMALL)
def test_small_prefill(lens, topk):
    _banner(f"small prefill lens={lens} topk={topk}")
    p = gen.make_problem(lens, seed=100 + sum(lens) + topk)
    _check_rows(f"prefill{lens}/k{topk}", DeviceProblem(p, topk), None, topk)


@pytest.mark.parametrize("lens,topk", [([33], 2), ([64, 61, 4, 1], 3), ([4099], 512),
                                       ([2000, 1999, 6], 100)])
def test_small_decode(lens, topk):
    _banner(f"small decode lens={lens} topk={topk}")
    p = gen.make_problem(lens, q_lens=[1] * len(lens), seed=200 + sum(lens))
    _check_rows(f"decode{lens}/k{topk}", DeviceProblem(p, topk), None, topk)


@pytest.mark.parametrize("topk", [512, 100])
def test_decode_odd_split_counts(topk):
    """9 decode rows: ceil(1024 / 18) = 57 key splits per (row, KV head) are rounded up to an
    even count, so the workgroups of the attention (4 splits each) never straddle two rows;
    the rows mix scored contexts (more blocks than the budget) with short ones."""
    lens = [5000, 3000, 2100, 9000, 4097, 2049, 600, 12000, 7777]
    _banner(f"decode 9 rows topk={topk}")
    p = gen.make_problem(lens, q_lens=[1] * len(lens), seed=311 + topk)
    _check_rows(f"decode9/k{topk}", DeviceProblem(p, topk), None, topk)


def test_multi_query_odd_split_counts():
    """11 query rows (4 + 4 + 3): 47 splits rounded up to 48."""
    lens, q_lens = [6000, 3001, 2500], [4, 4, 3]
    _banner("multi-query decode, 11 rows")
    p = gen.make_problem(lens, q_lens=q_lens, seed=317)
    _check_rows("multi-query-11", DeviceProblem(p, 512), None, 512)


def test_decode_65_rows_split_combine():
    """65 decode rows, one more than the decode tables hold: the per-sequence table path
    with 8 key splits per (row, KV head) and the combine kernel (mixed lengths, some rows
    within the budget)."""
    lens = [3000 + 37 * i for i in range(60)] + [100, 2048, 2051, 900, 5]
    _banner("decode 65 rows")
    p = gen.make_problem(lens, q_lens=[1] * len(lens), seed=331)
    _check_rows("decode-65-rows", DeviceProblem(p, 512), None, 512)


def test_multi_query_rows_per_sequence():
    """2-4 query tokens per sequence (the last tokens), ragged lengths."""
    _banner("multi-query decode")
    lens, q_lens = [3000, 2500, 777, 16], [4, 2, 3, 1]
    p = gen.make_problem(lens, q_lens=q_lens, seed=301)
    _check_rows("multi-query", DeviceProblem(p, 64), None, 64)


# ----------------------------------------------------------------- configurations

def test_prefill_1x1024_dense():
    _banner("prefill 1x1024")
    p = gen.workload_problem("prefill_1x1024")
    _check_rows("prefill-1x1024", DeviceProblem(p), None, 512)


@pytest.mark.parametrize("lens,topk", [
    ([700, 1500, 33], 512),   # ragged, every row dense
    ([258, 258, 258], 64),    # dense rows t <= 258 at budget 64
    ([2051], 512),            # the longest dense rows at the model's budget
])
def test_dense_prefills(lens, topk):
    """All-dense prefills of several shapes (ragged tails, a smaller budget, the longest
    dense rows): every row checked."""
    _banner(f"dense prefill lens={lens} topk={topk}")
    p = gen.make_problem(lens, seed=600 + sum(lens) + topk)
    _check_rows(f"dense{lens}/k{topk}", DeviceProblem(p, topk), None, topk)


@pytest.mark.parametrize("lens,q_lens,topk", [
    ([100, 700, 2051, 37], [80, 650, 1000, 37], 512),   # few dense tiles (key halves)
    ([700, 300], [690, 299], 64),                        # dense/sparse boundary inside
    ([4100, 3000], [4090, 2900], 512),                   # 250 dense tiles
])
def test_dense_rows_after_cached_prefix(lens, q_lens, topk):
    """Dense-regime rows that start after a cached prefix, at positions that are not
    multiples of the key tile, so that a tile's early rows see none of the keys of some
    of the tiles its later rows attend: every row checked."""
    _banner(f"dense rows after a prefix lens={lens} q_lens={q_lens} topk={topk}")
    p = gen.make_problem(lens, q_lens=q_lens, seed=650 + sum(q_lens) + topk)
    _check_rows(f"dense-prefix{lens}/k{topk}", DeviceProblem(p, topk), None, topk)


def test_decode_1x32768_needles():
    _banner("decode 1x32768")
    p = gen.workload_problem("decode_1x32768")
    sel, _ = _check_rows("decode-1x32768", DeviceProblem(p), None, 512)
    assert set(p.needles[0]) <= set(sel[0].tolist())


def _check_all_selections(name, dp, attend_rows, topk=512, threads=None):
    """Compressed keys and the selection of EVERY row bit-exact against the oracle;
    out and lse on attend_rows (None: every row) within the forward's bars."""
    p = dp.p
    dims = oracle.Dims(topk_blocks=topk)
    k_blk, sel, out, lse = dp.forward()
    kb_r = oracle.compress(dims, p.cu_k, p.k_idx)
    assert np.array_equal(k_blk, kb_r), f"{name}: compressed keys differ"
    sel_r = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb_r, threads=threads)
    bad = np.nonzero(~np.all(sel == sel_r, axis=1))[0]
    assert bad.size == 0, f"{name}: selection differs on {bad.size} rows, first {bad[:10]}"
    out_r, lse_r = oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel_r, rows=attend_rows,
                                 threads=threads)
    rows = np.arange(p.n_q) if attend_rows is None else np.asarray(attend_rows)
    mx, mean = errs(out[rows], out_r[rows])
    lmx, _ = errs(lse[rows], lse_r[rows])
    print(f"[{name}] selections: all {p.n_q} rows equal; attention rows={len(rows)} "
          f"max_abs={mx:.3e} mean_abs={mean:.3e} lse={lmx:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lmx <= LSE_ABS
    return sel, out


def test_prefill_1x16384_all_rows():
    """Every one of the 16,384 rows: selection bit-exact, out and lse within the bars."""
    _banner("prefill 1x16384")
    p = gen.workload_problem("prefill_1x16384")
    _check_all_selections("prefill-1x16384", DeviceProblem(p), None)


def test_decode_16x262144_full():
    _banner("decode 16x262144")
    p = gen.workload_problem("decode_16x262144")
    sel, _ = _check_rows("decode-16x262144", DeviceProblem(p), None, 512)
    for b, needles in p.needles.items():
        assert set(needles) <= set(sel[b].tolist()), f"needles of sequence {b} missing"


def test_decode_multi_query_16x262144_full():
    """The multi-query decode line at its size: 16 sequences of 262,144 tokens, 4 query
    tokens each (tiles of 4 rows sharing the compressed-key scan), all 64 rows."""
    _banner("decode 16x262144, 4 query tokens per sequence")
    p = gen.make_problem([262144] * 16, q_lens=[4] * 16, seed=1003, needles=32)
    _check_rows("decode-16x262144-4q", DeviceProblem(p), None, 512)


def test_prefill_ragged_64k_all_selections():
    """Selections of all 113,729 rows bit-exact; out and lse on every 56th row plus each
    sequence's ends and its dense/sparse boundary (over 2,000 rows)."""
    _banner("ragged prefill 65535/40001/8190/3")
    p = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
    rows = stratified_rows(p.cu_q, p.cu_k, every=56)
    assert len(rows) >= 2000
    _check_all_selections("ragged-64k", DeviceProblem(p), rows)


def test_prefill_crowded_first_digit():
    """Indexer values in [2, 3] keep every score of a row within about 10% of each other,
    so the bin of the first 11-bit radix digit that holds the 512th key holds nearly all of
    the row's keys (hundreds of distinct values, heavy ties). One 70,001-token sequence: rows
    past position 65,539 see more than 16,384 blocks, so their launches take the long-row
    select, whose LDS list cannot hold such a bin and which continues the radix digits over
    global memory; earlier rows take the lean select. 160 rows across the sequence (both
    sides of that boundary, and its last rows): selections bit-exact, out and lse within
    the bars."""
    _banner("prefill, crowded first radix digit")
    p = gen.make_problem([70001], seed=23, idx_lo=2, idx_hi=3)
    rows = sorted(set(np.linspace(0, 70000, 130).astype(int).tolist())
                  | set(range(65530, 65550)) | set(range(69990, 70001)))
    _check_rows("crowded-bins", DeviceProblem(p), rows, 512)


def test_prefill_long_rows_two_sequences():
    """Two long sequences (70,001 and 66,001 tokens) whose rows see more than 16,384 blocks:
    their launches score tiles 4 at a time, and the group holding the first sequence's last
    3 tiles and the second sequence's first tile spans both sequences (scored tile by tile).
    Both sides of that boundary, the first sequence's last rows and rows spread over both:
    selections bit-exact, out and lse within the bars."""
    _banner("prefill, two long sequences")
    p = gen.make_problem([70001, 66001], seed=29)
    rows = sorted(set(np.linspace(0, p.n_q - 1, 120).astype(int).tolist())
                  | set(range(69980, 70001)) | set(range(70001 + 2040, 70001 + 2070)))
    _check_rows("two-long", DeviceProblem(p), rows, 512)


def test_prefill_1x262144_bounded_workspace():
    """One prefill at the native context, 262,144 tokens: its 8.6e9 score slots (34 GB
    of keys if kept whole) are scored and selected in passes of at most 2^26 keys, in a
    workspace of the selection plus two 256 MiB key buffers. 300 rows (spread over the sequence, its
    last rows and the dense/sparse boundary): selections bit-exact, out and lse within
    the bars."""
    _banner("prefill 1x262144")
    L = 262144
    p = gen.workload_problem("prefill_1x262144")
    dp = DeviceProblem(p)
    assert dp.ws.numel() <= 4 * 512 * L + 8 * 2**26 + 2**20
    rows = sorted(set(np.linspace(0, L - 1, 268).astype(int).tolist())
                  | set(range(2044, 2060)) | set(range(L - 16, L)))
    _check_rows("prefill-1x262144", dp, rows, 512)


def test_indexer_scores_bit_exact():
    """qsa_score on whole rows: with integer indexer data every fp32 score is exact, so
    the GPU's scores equal the oracle's double scores bit for bit (-inf past the row's
    visible blocks). Rows of the ragged prefill (each sequence's last row, rows at the
    dense/sparse boundary and inside, the length-3 sequence with no blocks) and all 16
    decode rows at 262,144 tokens (65,536 blocks each)."""
    _banner("indexer scores")
    dims = oracle.Dims()
    cases = []
    p4 = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
    cu = p4.cu_q
    rows4 = [int(cu[1]) - 1, int(cu[2]) - 1, int(cu[3]) - 1, int(cu[3]), int(cu[4]) - 1,
             2050, 2051, 30000, int(cu[1]) + 12345, int(cu[2]) + 4099]
    cases.append(("ragged-64k", p4, rows4))
    p3 = gen.workload_problem("decode_16x262144")
    cases.append(("decode-16x262144", p3, list(range(16))))
    for name, p, rows in cases:
        dp = DeviceProblem(p)
        ld = int((np.diff(p.cu_k.astype(np.int64)) // 4).max()) + 3
        rows_d = torch.tensor(rows, dtype=torch.int64, device="cuda")
        sc = torch.full((len(rows), ld), 7.0, dtype=torch.float32, device="cuda")
        qsa.score(dp.seqs, dp.q_idx, dp.w, dp.k_blk, rows_d, sc)
        torch.cuda.synchronize()
        got = sc.cpu().numpy()
        kb = oracle.compress(dims, p.cu_k, p.k_idx)
        for i, r in enumerate(rows):
            ref = oracle.row_scores(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb, r)
            n = ref.size
            assert np.array_equal(got[i, :n].astype(np.float64), ref), \
                f"{name}: scores of row {r} differ at {np.nonzero(got[i, :n] != ref)[0][:8]}"
            assert np.all(np.isneginf(got[i, n:])), f"{name}: row {r} past its blocks"
        print(f"[{name}] scores of {len(rows)} rows bit-exact", flush=True)


# ----------------------------------------------------------------- long contexts

def test_decode_1m_context():
    """One decode row at 1,048,576 tokens (262,144 blocks, 256 chunks): the attention
    workgroups merge its 8,192 chunk candidates (32 per thread); bit-exact selection,
    needles kept, outputs within tolerance."""
    _banner("decode 1M context")
    p = gen.make_problem([1 << 20], q_lens=[1], seed=17, needles=32)
    sel, _ = _check_rows("decode-1M", DeviceProblem(p, 512), None, 512)
    assert set(p.needles[0]) <= set(sel[0].tolist())


def test_decode_4x1m_full():
    """The 1M decode line's shape: 4 sequences of 1,048,576 tokens, one query each (4 score
    tiles of 256 chunks, each row merged from 8,192 candidates), all rows; the selection
    alone (merged by merge_dec_kernel) equals the forward's."""
    _banner("decode 4x1M")
    p = gen.make_problem([1 << 20] * 4, q_lens=[1] * 4, seed=23, needles=16)
    dp = DeviceProblem(p)
    sel, _ = _check_rows("4x1M", dp, None, 512)
    for b, needles in p.needles.items():
        assert set(needles) <= set(sel[b].tolist()), f"needles of sequence {b} missing"
    assert np.array_equal(dp.select(), sel)


def test_multi_query_long_rows():
    """Three query tokens of one 300,001-token sequence (one tile of 74 chunks: each row's
    2,368 candidates take the wide merge) plus a short sequence."""
    _banner("multi-query long rows")
    p = gen.make_problem([300001, 7000], q_lens=[3, 2], seed=18)
    dp = DeviceProblem(p, 512)
    sel, _ = _check_rows("mq-long", dp, None, 512)
    assert np.array_equal(dp.select(), sel)


@pytest.mark.parametrize("L", [266001, 526001])
def test_decode_chunk_counts_past_64(L):
    """65 and 129 chunks of 1,024 blocks (the last one partial): the first chunk counts
    past the 2,048-candidate merge, taken by the wide merge."""
    _banner(f"decode, {L} tokens")
    p = gen.make_problem([L], q_lens=[1], seed=20 + L % 7)
    _check_rows(f"chunks-{L}", DeviceProblem(p, 512), None, 512)


def test_wide_merge_exact_fallback():
    """A row of 100,000 blocks (98 chunks, the wide merge) whose best blocks form one run of
    300 blocks: the merge finds a chunk with every candidate kept, and the row is selected
    exactly."""
    _banner("wide merge exact fallback")
    p = gen.make_problem([400000], q_lens=[1], seed=19)
    u = (p.w[0][:, None].astype(np.float64) *
         gen.bf16_to_f32(p.q_idx[0]).astype(np.float64)).sum(axis=0)
    val = np.where(u >= 0, 0x4040, 0xC040).astype(np.uint16)
    p.k_idx[4 * 70000: 4 * 70300] = val[None, :]
    dp = DeviceProblem(p, 512)
    sel, _ = _check_rows("wide-fallback", dp, None, 512)
    assert set(range(70000, 70300)) <= set(sel[0].tolist())
    assert np.array_equal(dp.select(), sel)


def test_decode_rows_past_1m_exact():
    """Two query tokens of a 1,100,001-token sequence (275,000 blocks, 269 chunks: more than
    one merge of chunk candidates takes) plus a short sequence: the workgroup that completes
    the long tile's last chunk (arrival counter) scores its rows again and selects them
    exactly; called twice, so the counter must be back at zero after the first call."""
    _banner("decode rows past 1M tokens")
    p = gen.make_problem([1100001, 9000], q_lens=[2, 1], seed=31, needles=8)
    dp = DeviceProblem(p, 512)
    sel, _ = _check_rows("past-1M", dp, None, 512)
    assert set(p.needles[0]) <= set(sel[1].tolist())
    _, sel2, _, _ = dp.forward()
    assert np.array_equal(sel2, sel)
    assert np.array_equal(dp.select(), sel)


# ----------------------------------------------------------------- edge cases / properties

def test_all_ties_keep_lowest_blocks():
    _banner("all-tie scores")
    p = gen.make_problem([5000, 2100], q_lens=[3, 2100], seed=7)
    p.q_idx[:] = 0
    dp = DeviceProblem(p, 512)
    _, sel, _, _ = dp.forward()
    for r in range(p.n_q):
        seq = 0 if r < 3 else 1
        t = (5000 - 3 + r) if seq == 0 else (r - 3)
        n = min((t + 1) // 4, 512)
        assert sel[r].tolist() == list(range(n)) + [-1] * (512 - n)


@pytest.mark.parametrize("q_lens", [[1, 1], [3, 2]])
def test_decode_all_ties_exact_fallback(q_lens):
    """All-equal scores on decode-shaped calls: the first chunk keeps every one of its
    candidates, so the chunk union cannot be trusted and the exact path (rows scored
    again by the selecting workgroup) must give the lowest blocks."""
    _banner(f"decode all ties q_lens={q_lens}")
    p = gen.make_problem([9000, 5000], q_lens=q_lens, seed=13)
    p.q_idx[:] = 0
    sel, _ = _check_rows(f"decode-ties{q_lens}", DeviceProblem(p, 512), None, 512)
    assert sel[0].tolist() == list(range(512))


def test_decode_clustered_top_blocks_exact_fallback():
    """The best blocks of a decode row packed into one contiguous run of 300 blocks (far
    more than one chunk's candidates): exact fallback, bit-exact selection."""
    _banner("decode clustered top blocks")
    p = gen.make_problem([60000, 30000], q_lens=[1, 1], seed=14)
    for b, (k0, t) in enumerate([(0, 59999), (60000, 29999)]):
        u = (p.w[b][:, None].astype(np.float64) *
             gen.bf16_to_f32(p.q_idx[b]).astype(np.float64)).sum(axis=0)
        val = np.where(u >= 0, 0x4040, 0xC040).astype(np.uint16)   # +3 / -3 in bf16
        first = 2500 if b == 0 else 700
        p.k_idx[k0 + 4 * first: k0 + 4 * (first + 300)] = val[None, :]
    sel, _ = _check_rows("decode-cluster", DeviceProblem(p, 512), None, 512)
    assert set(range(2500, 2800)) <= set(sel[0].tolist())


def test_float_indexer_tie_tolerant():
    """Non-integer indexer data: fp32 GPU scores may round differently from the
    double oracle, so each kept block must score within 1e-5 relative of the
    oracle's budget threshold; attention is compared on the GPU's own selection."""
    _banner("float indexer")
    p = gen.make_problem([3000, 2500], q_lens=[5, 40], seed=8, float_indexer=True)
    topk = 128
    dp = DeviceProblem(p, topk)
    _, sel, out, lse = dp.forward()
    dims = oracle.Dims(topk_blocks=topk)
    kb = oracle.compress(dims, p.cu_k, p.k_idx)
    for r in range(p.n_q):
        s = oracle.row_scores(dims, p.cu_q, p.cu_k, p.q_idx, p.w, kb, r)
        kth = np.sort(s)[::-1][topk - 1]
        kept = sel[r][sel[r] >= 0]
        assert len(kept) == topk and np.all(np.diff(kept) > 0)
        assert np.all(s[kept] >= kth - 1e-5 * max(1.0, abs(kth)))
    out_r, lse_r = oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel)
    mx, mean = errs(out, out_r)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    assert errs(lse, lse_r)[0] <= LSE_ABS


def _random_case(i):
    """Shape i of a fixed, seeded family: 1-4 sequences of 0-20,000 tokens, each a prefill,
    a decode of 1-4 query tokens or without queries (at least one query in all), and a
    budget of 1-512 blocks."""
    rng = np.random.default_rng(7000 + i)
    nb = int(rng.integers(1, 5))
    lens, q_lens = [], []
    for _ in range(nb):
        L = int(rng.choice([int(rng.integers(0, 40)), int(rng.integers(40, 3000)),
                            int(rng.integers(3000, 20001))]))
        kind = rng.integers(0, 3)
        q = L if kind == 0 else (min(L, int(rng.integers(1, 5))) if kind == 1 else 0)
        lens.append(L)
        q_lens.append(q)
    if sum(q_lens) == 0:   # at least one query: a decode of the longest sequence
        j = int(np.argmax(lens))
        q_lens[j] = min(lens[j], 2)
    topk = int(rng.choice([1, 3, 16, 64, 100, 512]))
    return lens, q_lens, topk


@pytest.mark.parametrize("i", range(24))
def test_random_shapes(i):
    """24 seeded shapes mixing prefills and decodes, ragged and empty sequences, tails of
    0-3 tokens and budgets of 1-512 blocks: every row against the oracle."""
    lens, q_lens, topk = _random_case(i)
    _banner(f"random shape {i}: lens={lens} q_lens={q_lens} topk={topk}")
    p = gen.make_problem(lens, q_lens=q_lens, seed=7100 + i)
    _check_rows(f"random{i}", DeviceProblem(p, topk), None, topk)


def test_deterministic_bitwise():
    _banner("determinism")
    p = gen.make_problem([9000, 4000], q_lens=[1, 1], seed=9)
    dp = DeviceProblem(p, 512)
    a = dp.forward()
    b = dp.forward()
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decode_equals_last_prefill_row():
    _banner("decode == last prefill row")
    L = 2600
    p = gen.make_problem([L], seed=10)
    _, sel_p, out_p, lse_p = DeviceProblem(p, 256).forward()
    pd = gen.make_problem([L], seed=10)
    pd.cu_q = np.array([0, 1], np.int32)
    pd.q, pd.q_idx, pd.w = p.q[-1:].copy(), p.q_idx[-1:].copy(), p.w[-1:].copy()
    _, sel_d, out_d, lse_d = DeviceProblem(pd, 256).forward()
    assert np.array_equal(sel_d[0], sel_p[-1])
    assert errs(out_d[0], out_p[-1])[0] < 1e-5 and errs(lse_d[0], lse_p[-1])[0] < 1e-5


@pytest.mark.parametrize("lens,q_lens,topk", [
    ([4096, 1203, 8], [1, 7, 8], 512),   # some sequences have no scored row
    ([4096, 3000, 2052], [1, 2, 5], 64),  # every sequence scored: fused into scoring
])
def test_incremental_compress_completes_cache(lens, q_lens, topk):
    """forward() with k_idx recompresses only the blocks holding query tokens; with a
    cache built by compress() for the rest, the result equals a full compress and the
    selection and outputs match the oracle."""
    _banner(f"incremental compress lens={lens} q_lens={q_lens}")
    p = gen.make_problem(lens, q_lens=q_lens, seed=11)
    dp = DeviceProblem(p, topk)
    full = dp.compress()
    dp.k_blk.zero_()
    # rebuild the prefix cache only: blocks before each sequence's first query token
    dims = oracle.Dims()
    ref = oracle.compress(dims, p.cu_k, p.k_idx)
    assert np.array_equal(full, ref)
    pref = ref.copy()
    nb0 = 0
    for b in range(len(lens)):
        L = int(p.cu_k[b + 1] - p.cu_k[b])
        nq = int(p.cu_q[b + 1] - p.cu_q[b])
        first_new = (L - nq) // 4
        pref[nb0 + first_new: nb0 + L // 4] = 0x7FC0  # garbage where forward must write
        nb0 += L // 4
    dp.k_blk.copy_(torch.from_numpy(pref.view(np.int16)).cuda())
    gpu = dp.forward(with_k_idx=True)
    assert np.array_equal(gpu[0], ref)
    _check_rows(f"incremental{lens}", dp, None, topk, gpu=gpu)


def test_graph_replay_matches_eager():
    """A decode forward captured in a HIP graph, replayed several times with eager
    library work and synchronisations in between: every replay equals the eager
    result bit for bit (the workspace control block is left zero by every call)."""
    _banner("graph replay")
    p = gen.make_problem([20000, 9000], q_lens=[1, 1], seed=15)
    dp = DeviceProblem(p, 512)
    eager = dp.forward()
    other = DeviceProblem(gen.make_problem([5000], q_lens=[1], seed=16), 512)
    other_ref = other.forward()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.forward(dp.seqs, dp.q, dp.k, dp.v, dp.q_idx, dp.w, dp.k_idx, dp.k_blk, dp.sel,
                    dp.out, dp.lse, dp.ws, dp.topk)
    for i in range(4):
        dp.sel.fill_(-7)
        dp.out.fill_(float("nan"))
        dp.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (host16(dp.k_blk), dp.sel.cpu().numpy(), dp.out.cpu().numpy(), dp.lse.cpu().numpy())
        for x, y in zip(got, eager):
            assert np.array_equal(x, y), f"replay {i} differs from the eager forward"
        # eager work on the same workspace between replays
        qsa.forward(dp.seqs, dp.q, dp.k, dp.v, dp.q_idx, dp.w, dp.k_idx, dp.k_blk, dp.sel,
                    dp.out, dp.lse, dp.ws, dp.topk)
        torch.cuda.synchronize()
        for x, y in zip(other.forward(), other_ref):
            assert np.array_equal(x, y)


def test_select_and_attend_entry_points():
    """qsa_select then qsa_attend equal qsa_forward; attend accepts a caller selection."""
    _banner("separate entry points")
    p = gen.make_problem([3333, 100], q_lens=[2, 100], seed=12)
    dp = DeviceProblem(p, 32)
    kb, sel_f, out_f, lse_f = dp.forward()
    dp.sel.fill_(-9)
    sel_s = dp.select()
    assert np.array_equal(sel_s, sel_f)
    out_a, lse_a = dp.attend()
    assert np.array_equal(out_a, out_f) and np.array_equal(lse_a, lse_f)
    # a hand-made selection: every other visible block, capped at 32, -1 padded
    custom = np.full_like(sel_f, -1)
    dims = oracle.Dims(topk_blocks=32)
    for r in range(p.n_q):
        t = (3333 - 2 + r) if r < 2 else r - 2
        ids = list(range(0, (t + 1) // 4, 2))[:32]
        custom[r, :len(ids)] = ids
    out_c, lse_c = dp.attend(custom)
    out_r, lse_r = oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, custom)
    mx, mean = errs(out_c, out_r)
    assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_attend_supplied_selection_invalid_entries():
    """A caller's selection with an id of a block not yet visible at the row's position
    and entries after a -1: the library attends only the blocks that count, like the
    oracle (prefill rows in one split each; decode rows split over many waves)."""
    _banner("attend over a supplied selection with invalid entries")
    p = gen.make_problem([2000, 3000, 9], q_lens=[2000, 2, 9], seed=13)
    dp = DeviceProblem(p, 16)
    sel, clean = supplied_selection(row_positions(p.cu_q, p.cu_k), 16, 14)
    out, lse = dp.attend(sel)
    dims = oracle.Dims(topk_blocks=16)
    out_r, lse_r = oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, clean)
    mx, mean = errs(out, out_r)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    assert np.max(np.abs(lse - lse_r)) <= 1e-4
