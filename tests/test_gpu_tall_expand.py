"""GPU: the expand for tiles of 8 to 16 rows (decode batches whose rows share adapters)
against the fp64 oracle, element by element.

The shrink runs on the batch's 2-row tiles and the expand on a tile list of its own
(8- to 16-row tiles, as lora_pick_expand_tile_rows suggests for such batches); the
results must meet the stated tolerance on the whole y, keep rows without an adapter
bit-identical, and agree bit for bit between dense and paged weights (the two differ
only in where B is read).  Cases: the 13B decode mixes at full size (identical, skewed,
uniform popularity, 10 % rows without adapter, rank 64), ranks 1..64 (both column
widths per lane), a ragged output width, tiles of 8 to 16 rows with a row map, and
tiles taller than the launch's row-height hint (the kernel walks 16-row blocks).
"""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
NTHREADS = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield


def run_split_tiles(w, dc, idx, expand_rows, hint=None):
    """Segment form with the library's row grouping: shrink on 2-row tiles, expand on
    tiles of at most `expand_rows` rows (launch hint `hint`, default the true tallest)."""
    row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(idx, w.num_slots)
    segs_s = B.segments_to_device(B.lora_build_tiles(seg_ptr, seg_slot, 2), row_map, n_act)
    tiles = B.lora_build_tiles(seg_ptr, seg_slot, expand_rows)
    nprob, msgs = oracle.check_tiles(tiles, seg_ptr, seg_slot, expand_rows)
    assert nprob == 0, msgs[:3]
    segs_e = B.segments_to_device(tiles, row_map, n_act)
    if hint is not None:
        segs_e.c.max_rows = int(hint)
    B.lora_sgmv_shrink(dc.v, dc.x, w, segs_s)
    B.lora_sgmv_expand(dc.y, dc.v, w, segs_e)
    return dc.results()


@pytest.mark.parametrize("popularity", ["identical", "skewed", "uniform"])
@pytest.mark.parametrize("d_out", [5120, 13824])
def test_decode_mix_13b(popularity, d_out):
    b = wl.batch_decode_mix(popularity)
    rank = np.full(16, 64, dtype=np.int32)
    G.say(f"case tall-expand 13b {popularity} 5120->{d_out}")
    x, y0, store = G.dense_case(3, 0, b.n, 5120, d_out, 16, rank, wl.scale_for_rank(rank), b.idx)
    y_ref, v_ref = oracle.bgmv(store, x, y0, b.idx, nthreads=NTHREADS)
    dc = G.DeviceCase(x, y0, 64)
    y, v = run_split_tiles(B.weights_from_store(store), dc, b.idx, 16)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(b.idx, rank), f"13b-{popularity}-{d_out}")


@pytest.mark.parametrize("r_max", [16, 20, 48, 64])
@pytest.mark.parametrize("expand_rows", [8, 12, 16])
def test_dense_and_paged_bitwise_identical(r_max, expand_rows):
    """Ranks 1 .. r_max over 8 slots (rank 0 on one), 1032 output columns (a ragged
    last chunk of either column width), 8-element pages; 70 rows, 10 % without adapter."""
    S, n, d_in, d_out = 8, 70, 768, 1032
    rng = np.random.default_rng([41, r_max, expand_rows])
    rank = rng.integers(1, r_max + 1, size=S).astype(np.int32)
    rank[0], rank[3] = r_max, 0
    scale = wl.scale_for_rank(rank)
    idx = wl.mask_no_adapter(rng, wl.assign_zipf(rng, n, S, 1.0), 0.1)
    x, y0 = wl.activations(41, r_max, n, d_in, d_out)
    dense = wl.dense_store(41, r_max, S, d_in, d_out, rank, scale, r_max=r_max)
    paged = wl.paged_store(41, r_max, S, d_in, d_out, rank, scale, 8, spare_pages=3)
    y_ref, v_ref = oracle.bgmv(dense, x, y0, idx, nthreads=NTHREADS)
    G.say(f"case tall-expand dense-vs-paged r_max={r_max} tiles={expand_rows}")
    outs = []
    for store in (dense, paged):
        dc = G.DeviceCase(x, y0, r_max)
        y, v = run_split_tiles(B.weights_from_store(store), dc, idx, expand_rows)
        G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), f"r{r_max}-t{expand_rows}-"
                f"{'paged' if hasattr(store, 'pool') else 'dense'}")
        outs.append((y, v))
    assert np.array_equal(outs[0][0].view(np.uint16), outs[1][0].view(np.uint16)), "dense and paged y differ"
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32)), "dense and paged v differ"


@pytest.mark.parametrize("r_max", [32, 64])
def test_tiles_taller_than_the_hint(r_max):
    """Tiles of up to 40 rows launched with a 12-row hint (the row height is only a
    hint): the 8..16-row kernel walks each tile in 16-row blocks with B kept in
    registers, and the result must still meet the tolerance against the oracle."""
    S, n, d_in, d_out = 4, 96, 512, 2048
    rank = np.array([r_max, 9, 17, r_max], dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    rng = np.random.default_rng([42, r_max])
    idx = wl.mask_no_adapter(rng, wl.assign_zipf(rng, n, S, 0.5), 0.1)
    x, y0, store = G.dense_case(42, r_max, n, d_in, d_out, S, rank, scale, idx)
    y_ref, v_ref = oracle.bgmv(store, x, y0, idx, nthreads=NTHREADS)
    G.say(f"case tall-expand tiles over the hint r_max={r_max}")
    dc = G.DeviceCase(x, y0, r_max)
    y, v = run_split_tiles(B.weights_from_store(store), dc, idx, 40, hint=12)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), f"hint12-r{r_max}")


def test_repeat_is_bitwise_deterministic():
    """The same call twice gives the same bits (no atomics, fixed summation order)."""
    b = wl.batch_decode_mix("skewed")
    rank = np.full(16, 64, dtype=np.int32)
    x, y0, store = G.dense_case(3, 1, b.n, 5120, 5120, 16, rank, wl.scale_for_rank(rank), b.idx)
    w = B.weights_from_store(store)
    outs = []
    for _ in range(2):
        dc = G.DeviceCase(x, y0, 64)
        outs.append(run_split_tiles(w, dc, b.idx, 16))
    assert np.array_equal(outs[0][0].view(np.uint16), outs[1][0].view(np.uint16))
