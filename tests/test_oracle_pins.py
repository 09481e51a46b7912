"""The CPU oracle against its pins (exact rationals, numpy fp64, the pages' identities)."""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import workloads as wl
from tests import pins


@pytest.mark.parametrize("check", pins.CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    assert check(0) is None


def test_half_decode_matches_numpy_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits[::7]])
    want = ref[::7]
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def _mixed_case(seed=3, n=24, d_in=128, d_out=96, S=9):
    rank = np.array([4, 8, 0, 2, 8, 1, 6, 8, 3], dtype=np.int32)[:S]
    scale = wl.scale_for_rank(rank)
    idx = np.random.default_rng([seed, 1]).integers(-1, S, size=n).astype(np.int32)
    x, y0 = wl.activations(30 + seed, 0, n, d_in, d_out)
    dense = wl.dense_store(30 + seed, 0, S, d_in, d_out, rank, scale, r_max=8)
    paged = wl.paged_store(30 + seed, 0, S, d_in, d_out, rank, scale, 32, spare_pages=5)
    return x, y0, idx, rank, scale, dense, paged


def test_permutation_equivariance_exact():
    x, y0, idx, rank, scale, dense, _ = _mixed_case()
    y, v = oracle.bgmv(dense, x, y0, idx)
    perm = np.random.default_rng(8).permutation(len(idx))
    yp, vp = oracle.bgmv(dense, x[perm], y0[perm], idx[perm])
    assert np.array_equal(yp, y[perm])
    assert np.array_equal(np.nan_to_num(vp, nan=-7.0), np.nan_to_num(v[perm], nan=-7.0))


def test_linearity_in_scale():
    x, y0, idx, rank, scale, dense, _ = _mixed_case(seed=4)
    y1, _ = oracle.bgmv(dense, x, y0, idx)
    dense.scale = (scale * 2).astype(np.float32)
    y2, _ = oracle.bgmv(dense, x, y0, idx)
    d1, d2 = y1 - y0.astype(np.float64), y2 - y0.astype(np.float64)
    assert np.abs(d2 - 2 * d1).max() <= 1e-12 * np.abs(d1).max()


def test_segment_form_equals_row_form_exactly():
    x, y0, idx, rank, scale, dense, paged = _mixed_case(seed=5)
    row_map, seg_ptr, seg_slot, _ = oracle.build_segments(idx, len(rank))
    for store in (dense, paged):
        yb, vb = oracle.bgmv(store, x, y0, idx)
        ys, vs = oracle.sgmv(store, x, y0, seg_ptr, seg_slot, row_map)
        assert np.array_equal(yb, ys)
        assert np.array_equal(np.isnan(vb), np.isnan(vs))
        assert np.array_equal(vb[~np.isnan(vb)], vs[~np.isnan(vs)])


def test_paged_equals_dense_exactly():
    x, y0, idx, rank, scale, dense, paged = _mixed_case(seed=6)
    yd, _ = oracle.bgmv(dense, x, y0, idx)
    yp, _ = oracle.bgmv(paged, x, y0, idx)
    assert np.array_equal(yd, yp)
    assert not np.isnan(yd).any()


def test_contiguous_segments_without_row_map():
    b = wl.batch_tiny_sgmv()
    d_in = d_out = 64
    store = wl.dense_store(1, 0, 4, d_in, d_out, 16, 2.0)
    x, y0 = wl.activations(1, 0, b.n, d_in, d_out)
    ys, _ = oracle.sgmv(store, x, y0, b.seg_ptr, b.seg_slot)
    yb, _ = oracle.bgmv(store, x, y0, b.idx)
    assert np.array_equal(ys, yb)


def test_openmp_mode_is_bitwise_identical():
    x, y0, idx, rank, scale, dense, _ = _mixed_case(seed=7, n=40)
    y1, _ = oracle.bgmv(dense, x, y0, idx, nthreads=1)
    y4, _ = oracle.bgmv(dense, x, y0, idx, nthreads=4)
    assert np.array_equal(y1, y4)


# ----------------------------------------------------------------- metadata reference
def test_build_segments_properties():
    rng = np.random.default_rng(11)
    for trial in range(50):
        S = int(rng.integers(1, 40))
        n = int(rng.integers(0, 200))
        idx = rng.integers(-1, S, size=n).astype(np.int32)
        row_map, seg_ptr, seg_slot, n_act = oracle.build_segments(idx, S)
        assert n_act == int((idx >= 0).sum()) == len(row_map) == seg_ptr[-1]
        assert seg_ptr[0] == 0 and np.all(np.diff(seg_ptr) > 0)
        assert np.all(np.diff(seg_slot) > 0)               # ascending slot, one segment per slot
        assert sorted(row_map.tolist()) == np.flatnonzero(idx >= 0).tolist()
        for g in range(len(seg_slot)):
            rows = row_map[seg_ptr[g]:seg_ptr[g + 1]]
            assert np.all(idx[rows] == seg_slot[g])
            assert np.all(np.diff(rows) > 0)               # stable: ascending original row


def test_build_segments_rejects_bad_slot():
    with pytest.raises(ValueError):
        oracle.build_segments([0, 5], 5)
    with pytest.raises(ValueError):
        oracle.build_segments([-2], 5)


def test_build_segments_tiny_sgmv_layout():
    b = wl.batch_tiny_sgmv()
    row_map, seg_ptr, seg_slot, n_act = oracle.build_segments(b.idx, 4)
    assert seg_ptr.tolist() == [0, 1, 4, 6, 8]
    assert seg_slot.tolist() == [0, 1, 2, 3]
    assert row_map.tolist() == list(range(8))


def test_check_tiles_flags_bad_work_lists():
    seg_ptr = np.array([0, 3, 5], dtype=np.int32)
    seg_slot = np.array([4, 7], dtype=np.int32)
    good = np.array([[4, 0, 2, 0], [4, 2, 1, 0], [7, 3, 2, 1]], dtype=np.int32)
    assert oracle.check_tiles(good, seg_ptr, seg_slot, 64)[0] == 0
    overlap = np.array([[4, 0, 3, 0], [4, 2, 1, 0], [7, 3, 2, 1]], dtype=np.int32)
    assert oracle.check_tiles(overlap, seg_ptr, seg_slot, 64)[0] > 0
    missing = np.array([[4, 0, 3, 0], [7, 3, 1, 1]], dtype=np.int32)
    assert oracle.check_tiles(missing, seg_ptr, seg_slot, 64)[0] > 0
    straddle = np.array([[4, 0, 2, 0], [4, 2, 2, 0], [7, 4, 1, 1]], dtype=np.int32)
    assert oracle.check_tiles(straddle, seg_ptr, seg_slot, 64)[0] > 0
