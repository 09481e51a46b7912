"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Workloads are the five synthetic configurations at full size (tiny SGMV; 7B decode
with distinct adapters; 13B decode with uniform / skewed / identical popularity and
10% rows without adapter; 7B prefill with 16 log-uniform prompts; 70B paged decode
with 2000 mixed-rank adapters) plus edge cases (ragged widths, tile boundaries,
rank 0, empty segments, tiny pages).  Tolerances are in tests/gpu_cases.py.
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


def _oracle(store, x, y0, idx):
    return oracle.bgmv(store, x, y0, idx, nthreads=NTHREADS)


def _run(form, w, dc, idx, seg_ptr=None, seg_slot=None):
    if form == "bgmv":
        return G.run_bgmv(w, dc, idx)
    if form == "bgmv_split":
        return G.run_bgmv(w, dc, idx, split_calls=True)
    if form == "sgmv_rowmap":
        return G.run_sgmv(w, dc, idx=idx)
    if form == "sgmv":
        return G.run_sgmv(w, dc, seg_ptr=seg_ptr, seg_slot=seg_slot)
    if form == "mixed":
        return G.run_mixed(w, dc, idx)
    raise ValueError(form)


def _dense_check(label, cfg_id, proj, idx, d_in, d_out, num_slots, rank, scale, form, r_max=None,
                 seg_ptr=None, seg_slot=None):
    G.say(f"case {label} form={form} n={len(idx)} {d_in}->{d_out}")
    x, y0, store = G.dense_case(cfg_id, proj, len(idx), d_in, d_out, num_slots, rank, scale, idx, r_max=r_max)
    y_ref, v_ref = _oracle(store, x, y0, idx)
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, store.r_max)
    y, v = _run(form, w, dc, idx, seg_ptr, seg_slot)
    return G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, store.rank), label)


@pytest.mark.parametrize("form", ["sgmv", "sgmv_rowmap", "bgmv", "bgmv_split"])
def test_tiny_sgmv(form):
    b = wl.batch_tiny_sgmv()
    _dense_check("tiny", 1, 0, b.idx, 1024, 1024, 4, 16, wl.scale_for_rank(16), form,
                 seg_ptr=b.seg_ptr, seg_slot=b.seg_slot)


@pytest.mark.parametrize("shape", [(4096, 4096), (4096, 11008), (11008, 4096)], ids=str)
@pytest.mark.parametrize("form", ["bgmv", "sgmv_rowmap"])
def test_decode_distinct_7b(shape, form):
    b = wl.batch_decode_distinct(32)
    _dense_check("decode-distinct-7b", 2, wl.PROJ_IDS["q"], b.idx, shape[0], shape[1], 32, 16, 2.0, form)


@pytest.mark.parametrize("popularity", ["uniform", "skewed", "identical"])
@pytest.mark.parametrize("shape", [(5120, 5120), (5120, 13824), (13824, 5120)], ids=str)
@pytest.mark.parametrize("form", ["bgmv", "sgmv_rowmap"])
def test_decode_mix_13b(popularity, shape, form):
    b = wl.batch_decode_mix(popularity)
    assert (b.idx < 0).sum() == 6
    _dense_check(f"decode-{popularity}-13b", 3, wl.PROJ_IDS["q"], b.idx, shape[0], shape[1], 16, 64,
                 wl.scale_for_rank(64), form)


@pytest.mark.parametrize("shape", [(4096, 4096), (4096, 11008)], ids=str)
def test_prefill_7b(shape):
    b = wl.batch_prefill()
    _dense_check("prefill-7b", 4, wl.PROJ_IDS["q"], b.idx, shape[0], shape[1], 16, 16, 2.0, "sgmv",
                 seg_ptr=b.seg_ptr, seg_slot=b.seg_slot)


@pytest.mark.parametrize("d_out", [1024, 8192, 28672])
@pytest.mark.parametrize("form", ["bgmv", "sgmv_rowmap", "mixed"])
def test_paged_mixed_rank_70b(d_out, form):
    import torch
    d_in, P, S = 8192, 1024, 2000
    rank = wl.paged_ranks(S)
    scale = wl.scale_for_rank(rank)
    b = wl.batch_paged_zipf(256, S)
    proj = {1024: wl.PROJ_IDS["k"], 8192: wl.PROJ_IDS["q"], 28672: wl.PROJ_IDS["gate"]}[d_out]
    G.say(f"case paged-70b form={form} n=256 {d_in}->{d_out} distinct={len(np.unique(b.idx))}")
    pool, pt, a_off, b_off, rows, compact_pt = G.paged_device_pool(5, proj, rank, d_in, d_out, P, b.idx)
    ostore = wl.PagedStore(S, d_in, d_out, 64, P, rank, scale, rows, compact_pt, a_off, b_off)
    x, y0 = wl.activations(5, proj, 256, d_in, d_out)
    y_ref, v_ref = _oracle(ostore, x, y0, b.idx)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=64, rank=dev(rank), scale=dev(scale), pool=pool,
                  page_elems=P, page_table=dev(pt), a_pt_off=dev(a_off), b_pt_off=dev(b_off))
    host = B.CWeights.from_buffer_copy(w.c)
    keep = [np.ascontiguousarray(rank), np.ascontiguousarray(pt), np.ascontiguousarray(a_off),
            np.ascontiguousarray(b_off)]
    host.rank, host.page_table, host.a_pt_off, host.b_pt_off = [k.ctypes.data for k in keep]
    B.lora_validate_weights_host(host)
    dc = G.DeviceCase(x, y0, 64)
    y, v = _run(form, w, dc, b.idx)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(b.idx, rank), f"paged-70b-{d_out}")


@pytest.mark.parametrize("proj", ["k", "o", "down"])
def test_paged_70b_tp8_shard_shapes(proj):
    """One GPU's shard under 8-way tensor parallelism (k 8192->128, o 1024->8192, down
    3584->8192) with 128-element pages, 256 rows by Zipf 1.2 over 2000 mixed-rank adapters."""
    import torch
    d_in, d_out = wl.LLAMA2_70B_TP8[proj]
    P, S = 128, 2000
    rank = wl.paged_ranks(S)
    scale = wl.scale_for_rank(rank)
    b = wl.batch_paged_zipf(256, S)
    pid = wl.PROJ_IDS[proj] + 10
    G.say(f"case paged-70b-tp8 {proj} {d_in}->{d_out}")
    pool, pt, a_off, b_off, rows, compact_pt = G.paged_device_pool(5, pid, rank, d_in, d_out, P, b.idx)
    ostore = wl.PagedStore(S, d_in, d_out, 64, P, rank, scale, rows, compact_pt, a_off, b_off)
    x, y0 = wl.activations(5, pid, 256, d_in, d_out)
    y_ref, v_ref = _oracle(ostore, x, y0, b.idx)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=64, rank=dev(rank), scale=dev(scale), pool=pool,
                  page_elems=P, page_table=dev(pt), a_pt_off=dev(a_off), b_pt_off=dev(b_off))
    for form in ("bgmv", "sgmv_rowmap"):
        dc = G.DeviceCase(x, y0, 64)
        y, v = _run(form, w, dc, b.idx)
        G.check(dc, y, v, y_ref, v_ref, G.active_rows(b.idx, rank), f"paged-70b-tp8-{proj}-{form}")



@pytest.mark.parametrize("proj", ["q", "gate"])
def test_paged_70b_tp8_rank_column_shard(proj):
    """One GPU's share when A of a column-parallel projection is split by rank columns
    over 8 GPUs: the shrink over ceil(r / 8) rank-rows of the full 8192-wide input
    (ranks 1, 2, 4, 8 from the pool's 8..64) into the d_out / 8 shard, 128-element
    pages; the segment-form shrink with the per-row expand, as the bench runs it."""
    import torch
    d_in, d_out = wl.LLAMA2_70B_TP8[proj]
    P, S = 128, 2000
    rank = (wl.paged_ranks(S) + 7) // 8
    scale = wl.scale_for_rank(rank)
    b = wl.batch_paged_zipf(256, S)
    pid = wl.PROJ_IDS[proj] + 20
    G.say(f"case paged-70b-tp8-rank-shard {proj} {d_in}->{d_out}")
    pool, pt, a_off, b_off, rows, compact_pt = G.paged_device_pool(5, pid, rank, d_in, d_out, P, b.idx)
    ostore = wl.PagedStore(S, d_in, d_out, 8, P, rank, scale, rows, compact_pt, a_off, b_off)
    x, y0 = wl.activations(5, pid, 256, d_in, d_out)
    y_ref, v_ref = _oracle(ostore, x, y0, b.idx)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=8, rank=dev(rank), scale=dev(scale), pool=pool,
                  page_elems=P, page_table=dev(pt), a_pt_off=dev(a_off), b_pt_off=dev(b_off))
    dc = G.DeviceCase(x, y0, 8)
    y, v = _run("mixed", w, dc, b.idx)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(b.idx, rank), f"paged-70b-tp8-rank-shard-{proj}")

# ------------------------------------------------------------------ edge cases
def _mixed_rank_store(cfg, d_in, d_out, S=7, paged_P=None):
    rank = np.array([1, 64, 0, 17, 8, 33, 64], dtype=np.int32)[:S]
    scale = wl.scale_for_rank(rank)
    if paged_P:
        return wl.paged_store(cfg, 0, S, d_in, d_out, rank, scale, paged_P, spare_pages=11)
    return wl.dense_store(cfg, 0, S, d_in, d_out, rank, scale, r_max=64)


@pytest.mark.parametrize("layout", ["dense", "paged8", "paged56"])
@pytest.mark.parametrize("form", ["bgmv", "sgmv_rowmap", "mixed"])
def test_ragged_widths_mixed_ranks(layout, form):
    d_in, d_out = 1288, 1064        # neither is a multiple of the 256-wide k-block or 512-wide column chunk
    P = {"dense": None, "paged8": 8, "paged56": 56}[layout]
    store = _mixed_rank_store(11, d_in, d_out, paged_P=P)
    idx = np.random.default_rng(3).integers(-1, store.num_slots, size=150).astype(np.int32)
    x, y0 = wl.activations(11, 0, len(idx), d_in, d_out)
    y_ref, v_ref = _oracle(store, x, y0, idx)
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, 64)
    y, v = _run(form, w, dc, idx)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, store.rank), f"ragged-{layout}")


def test_tile_boundaries_and_empty_segments():
    lens = [64, 65, 1, 0, 127, 128, 129, 0, 16, 15, 17, 2048]
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.array([0, 1, 2, 3, 4, -1, 5, 6, 0, 3, 1, 4], dtype=np.int32)
    idx = np.repeat(seg_slot, lens).astype(np.int32)
    rank = np.array([16, 64, 1, 8, 0, 32, 16], dtype=np.int32)
    store = wl.dense_store(12, 0, 7, 1024, 1536, rank, wl.scale_for_rank(rank), r_max=64)
    x, y0 = wl.activations(12, 0, len(idx), 1024, 1536)
    y_ref, v_ref = _oracle(store, x, y0, idx)
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, 64)
    y, v = G.run_sgmv(w, dc, seg_ptr=seg_ptr, seg_slot=seg_slot)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), "tile-boundaries")


def test_no_active_rows_is_noop():
    idx = np.full(40, -1, dtype=np.int32)
    store = wl.dense_store(13, 0, 4, 512, 512, 16, 2.0)
    x, y0 = wl.activations(13, 0, 40, 512, 512)
    w = B.weights_from_store(store)
    for form in ("bgmv", "sgmv_rowmap"):
        dc = G.DeviceCase(x, y0, 16)
        y, v = _run(form, w, dc, idx)
        assert np.array_equal(y.view(np.uint16), dc.y_init.view(np.uint16))
        assert np.isnan(v).all()


def test_rank_zero_slots_untouched():
    idx = np.array([0, 1, 1, 0, 2, -1, 1], dtype=np.int32)
    rank = np.array([0, 16, 0], dtype=np.int32)
    store = wl.dense_store(14, 0, 3, 2048, 1024, rank, wl.scale_for_rank(rank), r_max=16)
    x, y0 = wl.activations(14, 0, len(idx), 2048, 1024)
    y_ref, v_ref = _oracle(store, x, y0, idx)
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, 16)
    y, v = G.run_bgmv(w, dc, idx)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), "rank-zero")


def test_dense_and_paged_are_bitwise_identical():
    d_in, d_out, S = 2048, 3072, 9
    rank = np.array([16, 8, 64, 4, 16, 32, 1, 64, 12], dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    idx = np.random.default_rng(4).integers(-1, S, size=48).astype(np.int32)
    dense = wl.dense_store(15, 0, S, d_in, d_out, rank, scale, r_max=64)
    paged = wl.paged_store(15, 0, S, d_in, d_out, rank, scale, 512, spare_pages=7)
    x, y0 = wl.activations(15, 0, len(idx), d_in, d_out)
    outs = []
    for store in (dense, paged):
        dc = G.DeviceCase(x, y0, 64)
        outs.append(G.run_bgmv(B.weights_from_store(store), dc, idx))
    assert np.array_equal(outs[0][0].view(np.uint16), outs[1][0].view(np.uint16))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


@pytest.mark.parametrize("d_in,r_max,page,shuffled", [(2048, 16, 512, False), (1288, 16, 8, True),
                                                      (1288, 12, 8, True)])
def test_mfma_shrink_row_blocks_match_paged_bitwise(d_in, r_max, page, shuffled):
    """64-row tiles of one projection of rank <= 16: the dense shrink takes the wave-staged
    kernel (two 32-row workgroups per tile, four wavefronts staging their own 128-column
    chunks), the paged one keeps a tile in one 16-wavefront workgroup; every element is
    summed in the same order, so y and v must agree bit for bit (and with the oracle).
    Cases: d_in a multiple of the chunk, and 1288 (a last chunk of one 16-byte group);
    r_max 12 (A^T rank-rows past r_max masked); rows in batch order or shuffled (a row
    map from the library's builder); tiles of 64 down to 1 rows."""
    lens = [64, 130, 17, 200, 3, 64]
    seg_slot = np.array([0, 1, 2, 3, 4, 1], dtype=np.int32)
    idx = np.repeat(seg_slot, lens).astype(np.int32)
    rank = np.minimum(np.array([16, 8, 16, 1, 12], dtype=np.int32), r_max)
    scale = wl.scale_for_rank(rank)
    dense = wl.dense_store(19, r_max, 5, d_in, 1536, rank, scale, r_max=r_max)
    paged = wl.paged_store(19, r_max, 5, d_in, 1536, rank, scale, page, spare_pages=5)
    if shuffled:
        idx = np.random.default_rng([19, d_in]).permutation(idx).astype(np.int32)
    x, y0 = wl.activations(19, r_max, len(idx), d_in, 1536)
    y_ref, v_ref = _oracle(dense, x, y0, idx)
    G.say(f"case wave-shrink d_in={d_in} r_max={r_max} shuffled={shuffled}")
    outs = []
    for store in (dense, paged):
        dc = G.DeviceCase(x, y0, r_max)
        if shuffled:
            outs.append(G.run_sgmv(B.weights_from_store(store), dc, idx=idx, max_tile_rows=64))
        else:
            outs.append(G.run_sgmv(B.weights_from_store(store), dc, seg_ptr=wl.segments_from_lengths(lens),
                                   seg_slot=seg_slot, max_tile_rows=64))
        G.check(dc, *outs[-1], y_ref, v_ref, G.active_rows(idx, rank), f"row-blocks-{d_in}-{r_max}")
    assert np.array_equal(outs[0][0].view(np.uint16), outs[1][0].view(np.uint16))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_run_to_run_determinism():
    b = wl.batch_decode_mix("skewed")
    x, y0, store = G.dense_case(3, 5, b.n, 5120, 13824, 16, 64, 0.5, b.idx)
    w = B.weights_from_store(store)
    for form in ("bgmv", "sgmv_rowmap"):
        dc = G.DeviceCase(x, y0, 64)
        y1, v1 = _run(form, w, dc, b.idx)
        dc.reset()
        y2, v2 = _run(form, w, dc, b.idx)
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), form
        assert np.array_equal(v1.view(np.uint32), v2.view(np.uint32)), form


def test_segment_and_row_forms_agree():
    b = wl.batch_decode_mix("uniform")
    x, y0, store = G.dense_case(3, 6, b.n, 5120, 5120, 16, 64, 0.5, b.idx)
    w = B.weights_from_store(store)
    dc1, dc2 = G.DeviceCase(x, y0, 64), G.DeviceCase(x, y0, 64)
    yb, _ = G.run_bgmv(w, dc1, b.idx)
    ys, _ = G.run_sgmv(w, dc2, idx=b.idx)
    d = np.abs(yb.astype(np.float64) - ys.astype(np.float64))
    assert d.max() <= G.TOL_MAX_ABS


def test_repeated_calls_of_different_sizes():
    """Calls of decreasing and increasing size in a row on one descriptor."""
    import torch
    store = wl.dense_store(16, 0, 32, 4096, 4096, 16, 2.0)
    w = B.weights_from_store(store)
    for n in (32, 7, 32, 1):
        idx = np.arange(n, dtype=np.int32)
        x, y0 = wl.activations(16, n, n, 4096, 4096)
        y_ref, v_ref = _oracle(store, x, y0, idx)
        dc = G.DeviceCase(x, y0, 16)
        B.lora_bgmv(dc.y, dc.x, torch.from_numpy(idx).cuda(), w, dc.v)
        y, v = dc.results()
        G.check(dc, y, v, y_ref, v_ref, np.ones(n, bool), f"repeat-{n}")


@pytest.mark.parametrize("max_tile_rows", [1, 7, 8, 16, 33, 64])
def test_tile_size_does_not_change_results_beyond_tolerance(max_tile_rows):
    """Prefill-like segments cut into tiles of different sizes (VALU and MFMA paths)."""
    lens = [300, 17, 64, 5, 129]
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.array([0, 1, 2, 3, 0], dtype=np.int32)
    idx = np.repeat(seg_slot, lens).astype(np.int32)
    rank = np.array([16, 64, 8, 33], dtype=np.int32)
    store = wl.dense_store(17, 0, 4, 2048, 2560, rank, wl.scale_for_rank(rank), r_max=64)
    x, y0 = wl.activations(17, 0, len(idx), 2048, 2560)
    y_ref, v_ref = _oracle(store, x, y0, idx)
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, 64)
    y, v = G.run_sgmv(w, dc, seg_ptr=seg_ptr, seg_slot=seg_slot, max_tile_rows=max_tile_rows)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), f"tiles-{max_tile_rows}")


@pytest.mark.parametrize("form", ["bgmv", "sgmv_rowmap", "sgmv_prefill"])
def test_multi_projection_launch_matches_single_calls(form):
    """q/k/v-like grouping (one x, three outputs): each projection bit-identical to its
    single-projection call and within tolerance of the oracle."""
    import torch
    if form == "sgmv_prefill":
        lens = [40, 3, 100, 17]
        seg_ptr = wl.segments_from_lengths(lens)
        seg_slot = np.array([1, 0, 3, 2], dtype=np.int32)
        idx = np.repeat(seg_slot, lens).astype(np.int32)
        n = len(idx)
    else:
        b = wl.batch_decode_mix("skewed")
        idx, n = b.idx, b.n
    d_in, outs, S = 2048, (2048, 512, 512), 16
    rank = np.array([16, 8, 64, 32] * 4, dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    x, _ = wl.activations(18, 0, n, d_in, 8)
    stores, y0s, refs = [], [], []
    for p, d_out in enumerate(outs):
        store = wl.dense_store(18, 10 + p, S, d_in, d_out, rank, scale, r_max=64)
        _, y0 = wl.activations(18, 10 + p, n, d_in, d_out)
        stores.append(store)
        y0s.append(y0)
        refs.append(_oracle(store, x, y0, idx))
    ws = [B.weights_from_store(st) for st in stores]
    xd = torch.from_numpy(x).cuda()
    idx_d = torch.from_numpy(idx).cuda()
    if form == "bgmv":
        segs = None
    elif form == "sgmv_rowmap":
        row_map, sp, ss, n_act = B.lora_build_segments(idx, S)
        segs = B.segments_to_device(B.lora_build_tiles(sp, ss, 16), row_map, n_act)
    else:
        segs = B.segments_to_device(B.lora_build_tiles(seg_ptr, seg_slot, 16), None, n)
    single, multi = [], []
    for mode in ("single", "multi"):
        vs = [torch.full((n, 64), float("nan"), dtype=torch.float32, device="cuda") for _ in outs]
        ys = [torch.from_numpy(y0.copy()).cuda() for y0 in y0s]
        items = list(zip(ws, vs, ys))
        if mode == "single":
            for w, v, y in items:
                if segs is None:
                    B.lora_bgmv_shrink(v, xd, idx_d, w)
                    B.lora_bgmv_expand(y, v, idx_d, w)
                else:
                    B.lora_sgmv_shrink(v, xd, w, segs)
                    B.lora_sgmv_expand(y, v, w, segs)
        else:
            if segs is None:
                B.lora_bgmv_shrink_multi(xd, idx_d, items)
                B.lora_bgmv_expand_multi(idx_d, items, n)
            else:
                B.lora_sgmv_shrink_multi(xd, segs, items)
                B.lora_sgmv_expand_multi(segs, items, n)
        torch.cuda.synchronize()
        (single if mode == "single" else multi).extend((y.cpu().numpy(), v.cpu().numpy()) for _, v, y in items)
    act = G.active_rows(idx, rank)
    for p in range(len(outs)):
        (ys_, vs_), (ym, vm) = single[p], multi[p]
        assert np.array_equal(ys_.view(np.uint16), ym.view(np.uint16)), f"projection {p}: y differs"
        assert np.array_equal(np.nan_to_num(vs_, nan=-1).view(np.uint32), np.nan_to_num(vm, nan=-1).view(np.uint32))
        y_ref = refs[p][0]
        err = np.abs(ym.astype(np.float64) - y_ref)
        assert err.max() <= G.TOL_MAX_ABS
        assert np.linalg.norm(ym.astype(np.float64) - y_ref) / np.linalg.norm(y_ref) <= G.TOL_REL_FRO
        assert np.array_equal(ym[~act].view(np.uint16), y0s[p][~act].view(np.uint16))


@pytest.mark.parametrize("layout", ["dense", "paged"])
def test_mfma_paths_with_rank_not_multiple_of_16(layout):
    """r_max = 20 with MFMA-sized tiles that use the last slot: the expand's LDS staging
    pads ranks to 16 and must not read past the slot storage."""
    lens = [30, 9, 50, 7]
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.array([3, 0, 2, 1], dtype=np.int32)
    idx = np.repeat(seg_slot, lens).astype(np.int32)
    rank = np.array([5, 20, 17, 20], dtype=np.int32)
    d_in, d_out = 1536, 2048
    if layout == "dense":
        store = wl.dense_store(19, 0, 4, d_in, d_out, rank, wl.scale_for_rank(rank), r_max=20)
    else:
        store = wl.paged_store(19, 0, 4, d_in, d_out, rank, wl.scale_for_rank(rank), 512, spare_pages=4)
    x, y0 = wl.activations(19, 0, len(idx), d_in, d_out)
    y_ref, v_ref = _oracle(store, x, y0, idx)
    w = B.weights_from_store(store)
    dc = G.DeviceCase(x, y0, 20)
    y, v = G.run_sgmv(w, dc, seg_ptr=seg_ptr, seg_slot=seg_slot, max_tile_rows=16)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), f"rmax20-{layout}")


@pytest.mark.parametrize("max_tile_rows", [16, 32, 64])
@pytest.mark.parametrize("d_in", [1288, 4096])
def test_mfma_dense_and_paged_are_bitwise_identical(max_tile_rows, d_in):
    """Long segments on the MFMA kernels: the dense shrink stages x and A^T through LDS
    and groups up to 4 rank slices per workgroup, the paged one reads its operands
    straight from memory one slice at a time; both sum every element in the same order,
    so v and y agree bit for bit (d_in 1288 leaves a ragged last 512-column chunk)."""
    lens = [150, 9, 70, 33, 1, 64]
    seg_ptr = wl.segments_from_lengths(lens)
    S = len(lens)
    seg_slot = np.arange(S, dtype=np.int32)[::-1].copy()
    rank = np.array([64, 16, 33, 8, 1, 48], dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    d_out = 1032
    dense = wl.dense_store(23, 0, S, d_in, d_out, rank, scale, r_max=64)
    paged = wl.paged_store(23, 0, S, d_in, d_out, rank, scale, 8, spare_pages=5)
    idx = np.repeat(seg_slot, lens).astype(np.int32)
    x, y0 = wl.activations(23, 0, len(idx), d_in, d_out)
    G.say(f"case mfma-dense-vs-paged d_in={d_in} tiles={max_tile_rows}")
    outs = []
    for store in (dense, paged):
        dc = G.DeviceCase(x, y0, 64)
        outs.append(G.run_sgmv(B.weights_from_store(store), dc, seg_ptr=seg_ptr, seg_slot=seg_slot,
                               max_tile_rows=max_tile_rows))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32)), "v"
    assert np.array_equal(outs[0][0].view(np.uint16), outs[1][0].view(np.uint16)), "y"
    y_ref, v_ref = _oracle(dense, x, y0, idx)
    G.check(dc, *outs[1], y_ref, v_ref, G.active_rows(idx, rank), f"mfma-dense-vs-paged-{d_in}-{max_tile_rows}")
