"""GPU: large and tiny magnitudes of s.v on the MFMA expand (tiles of 8 rows or more) and
the VALU expand, against the fp64 oracle.

The MFMA expand feeds s.v to fp16 matrix operands as a high and a low fp16 part.  Its
per-row power-of-two scaling keeps both parts in fp16's normal range, so |s.v| beyond
fp16's largest value (65504) or below its smallest normal value (2^-14) is still carried
with fp32 accuracy: every output must be finite and within one fp16 unit in the last
place of the exact result plus the fp32 accumulation bound 2^-20 (|y0| + sum_j |s v_j B_jc|).
The stated fp32 accumulation contract (Punica summary, section 3.4 "The SGMV Operator:
What It Computes", the expand y += s.v.B) does not depend on the inputs' magnitude.
"""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield


def _ulp16(a):
    """fp16 unit in the last place at |a| (subnormal spacing below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("case", ["large", "tiny"])
@pytest.mark.parametrize("tile_rows", [2, 16, 64])
def test_extreme_magnitudes_of_sv(case, tile_rows):
    lens = [70, 3, 40, 1, 20]
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.array([1, 0, 3, 2, 1], np.int32)
    rank = np.array([16, 64, 8, 33], np.int32)
    d_in, d_out = 2048, 1032
    store = wl.dense_store(29, 0, 4, d_in, d_out, rank, wl.scale_for_rank(rank), r_max=64)
    x, y0 = wl.activations(29, 0, int(seg_ptr[-1]), d_in, d_out)
    # scale the drawn fp16 values by powers of two (exact, all inside fp16's range)
    sx, sa, sb = (2.0 ** 12, 2.0 ** 12, 2.0 ** -8) if case == "large" else (2.0 ** -6, 2.0 ** -6, 2.0 ** 10)
    x = (x.astype(np.float32) * sx).astype(np.float16)
    store.a_t = (store.a_t.astype(np.float32) * sa).astype(np.float16)
    store.b = (store.b.astype(np.float32) * sb).astype(np.float16)
    idx = np.repeat(seg_slot, lens).astype(np.int32)
    y_ref, v_ref = oracle.sgmv(store, x, y0, seg_ptr, seg_slot, nthreads=16)
    sv = np.abs(np.nan_to_num(v_ref)) * store.scale[np.maximum(idx, 0)][:, None]
    big = float(sv.max())
    G.say(f"case {case} tiles={tile_rows}: max |s v| = {big:.3e}")
    if case == "large":
        assert big > 65504.0
    else:
        assert 0 < big < 2.0 ** -14
    # sum_j |s v_j B_jc| per element, masked to each row's rank
    bound = np.abs(y0.astype(np.float64)).copy()
    for s in np.unique(idx):
        r = int(rank[s])
        rows = np.where(idx == s)[0]
        bound[rows] += sv[rows, :r] @ np.abs(store.b[s, :r].astype(np.float64))
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, 64)
    y, v = G.run_sgmv(w, dc, seg_ptr=seg_ptr, seg_slot=seg_slot, max_tile_rows=tile_rows)
    yg = y[G.GUARD_ROWS:G.GUARD_ROWS + dc.n, :d_out].astype(np.float64)
    assert np.isfinite(yg).all(), "non-finite output"
    err = np.abs(yg - y_ref)
    allowed = _ulp16(y_ref) + 2.0 ** -20 * bound
    worst = float((err / allowed).max())
    G.say(f"  worst error / allowed = {worst:.3f}")
    assert worst <= 1.0
    act = G.active_rows(idx, rank)
    va, vr = v[G.GUARD_ROWS:G.GUARD_ROWS + dc.n, :64][act].astype(np.float64), v_ref[act]
    assert np.isfinite(va).all()
    assert np.linalg.norm(va - vr) / np.linalg.norm(vr) <= G.TOL_V_REL_FRO
