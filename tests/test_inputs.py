"""The seeded generator: reproducible, sliceable, with the stated value laws."""
import numpy as np

import qsa_inputs as gen
from qsa_inputs import bf16_to_f32


def test_counter_based_slices_match_full_stream():
    full = gen.normal_bf16(5, gen.TID_K, 300000)
    part = gen.normal_bf16(5, gen.TID_K, 1000, offset=123456)
    assert np.array_equal(full[123456:124456], part)
    ints = gen.uniform_int_bf16(5, gen.TID_KIDX, 5000, -3, 3)
    assert np.array_equal(ints[100:200], gen.uniform_int_bf16(5, gen.TID_KIDX, 100, -3, 3,
                                                              offset=100))


def test_reproducible_and_seed_dependent():
    a = gen.make_problem([40, 7], seed=9)
    b = gen.make_problem([40, 7], seed=9)
    c = gen.make_problem([40, 7], seed=10)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q_idx, b.q_idx)
    assert not np.array_equal(a.k, c.k)


def test_value_laws():
    x = bf16_to_f32(gen.normal_bf16(1, gen.TID_Q, 200000, scale=0.5)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 0.5) < 0.01
    i = bf16_to_f32(gen.uniform_int_bf16(1, gen.TID_QIDX, 70000, -3, 3))
    assert set(np.unique(i).tolist()) == set(range(-3, 4))
    w = gen.weights(1, gen.TID_W, 10000)
    assert set(np.unique(w).tolist()) == {1.0, 2.0}


def test_outlier_rows_scaled_by_eight():
    p = gen.make_problem([2000], seed=4, qkv_scale=0.5, outlier_frac=0.05)
    base = gen.make_problem([2000], seed=4, qkv_scale=0.5)
    kf, bfv = bf16_to_f32(p.k), bf16_to_f32(base.k)
    scaled = np.all(kf == bfv * 8, axis=2) & np.any(bfv != 0, axis=2)
    same = np.all(kf == bfv, axis=2)
    assert np.all(scaled | same)
    frac = scaled.mean()
    assert 0.035 < frac < 0.065


def test_needle_blocks_point_along_query():
    p = gen.workload_problem("decode_1x32768")
    assert len(p.needles[0]) == 16 and len(set(p.needles[0])) == 16
    u = (bf16_to_f32(p.q_idx[0]) * p.w[0][:, None]).sum(axis=0)
    sgn = np.where(u >= 0, 3.0, -3.0)
    for blk in p.needles[0]:
        rows = bf16_to_f32(p.k_idx[4 * blk: 4 * blk + 4])
        assert np.all(rows == sgn[None, :])
        assert blk < 32768 // 4 - 1
