"""GPU: the work split fixed with lora_set_plan (rank-rows per shrink workgroup, rows
per pass of the segment-form VALU kernels) changes no bit of v or y, for both call
forms, dense and paged weights, and tiles of 1 to 64 rows."""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
PLANS = [(0, 0), (1, 1), (2, 2), (3, 4), (4, 1), (8, 2), (16, 4), (64, 0)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    B.lora_set_plan(0, 0)


def _segs(idx, S, tile_rows):
    row_map, sp, ss, n_act = B.lora_build_segments(idx, S)
    return B.segments_to_device(B.lora_build_tiles(sp, ss, tile_rows), row_map, n_act)


@pytest.mark.parametrize("layout", ["dense", "paged56"])
@pytest.mark.parametrize("form", ["bgmv", "sgmv4", "sgmv7", "sgmv64"])
def test_plan_changes_no_bits(layout, form):
    import torch
    S, d_in, outs = 7, 1288, (1064, 2632)
    rank = np.array([1, 64, 0, 17, 8, 33, 64], dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    idx = np.random.default_rng(21).integers(-1, S, size=150).astype(np.int32)
    if layout == "dense":
        stores = [wl.dense_store(21, p, S, d_in, d, rank, scale, r_max=64) for p, d in enumerate(outs)]
    else:
        stores = [wl.paged_store(21, p, S, d_in, d, rank, scale, 56, spare_pages=3) for p, d in enumerate(outs)]
    x, _ = wl.activations(21, 0, len(idx), d_in, 8)
    y0s = [wl.activations(21, 30 + p, len(idx), 8, d)[1] for p, d in enumerate(outs)]
    ws = [B.weights_from_store(st) for st in stores]
    dcs = [G.DeviceCase(x, y0, st.r_max) for y0, st in zip(y0s, stores)]
    idx_d = torch.from_numpy(idx).cuda()
    segs = None if form == "bgmv" else _segs(idx, S, int(form[4:]))
    G.say(f"case plan layout={layout} form={form}")
    results = []
    for jw, nr in PLANS:
        B.lora_set_plan(jw, nr)
        for dc in dcs:
            dc.reset()
        items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
        if segs is None:
            B.lora_bgmv_shrink_multi(dcs[0].x, idx_d, items)
            B.lora_bgmv_expand_multi(idx_d, items, len(idx))
        else:
            B.lora_sgmv_shrink_multi(dcs[0].x, segs, items)
            B.lora_sgmv_expand_multi(segs, items, len(idx))
        results.append([dc.results() for dc in dcs])
    B.lora_set_plan(0, 0)
    for plan, res in zip(PLANS, results):
        for p, ((yb, vb), (yg, vg)) in enumerate(zip(results[0], res)):
            assert np.array_equal(yb.view(np.uint16), yg.view(np.uint16)), f"plan {plan} proj {p}: y"
            assert np.array_equal(vb.view(np.uint32), vg.view(np.uint32)), f"plan {plan} proj {p}: v"
    for p, (st, dc) in enumerate(zip(stores, dcs)):
        y_ref, v_ref = oracle.bgmv(st, x, y0s[p], idx, nthreads=16)
        G.check(dc, *results[0][p], y_ref, v_ref, G.active_rows(idx, st.rank), f"plan-{layout}-{form}-p{p}")
