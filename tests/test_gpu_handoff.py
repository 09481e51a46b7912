"""GPU: shrink and expand in one launch with v handed from the shrink's workgroups to the
expand's, against the two-launch path bit for bit on whole buffers (guard rows and
padding included), and the two-launch path against the fp64 oracle: the per-row form
(lora_bgmv_multi_handoff vs lora_bgmv_multi) and the segment form
(lora_sgmv_multi_handoff vs lora_sgmv_shrink_multi + lora_sgmv_expand_multi, over tiles
of 1, 2 and 4 rows, and over taller tiles and paged weights, where it makes the two
launches itself).

Every case runs the hand-off form twice: with the default poll limit, and with the limit
at zero, where every expand workgroup computes its row's v itself (the path taken when
the hand-off does not arrive in time).  All cases share one workspace, so each call
also checks that the previous one left it cleared; the test reads it back as zero after
every call.  A graph replay test interleaves replays with eager calls on other inputs
that share the workspace.
"""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
MAX_ROWS = 512


@pytest.fixture(scope="module")
def work():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    w = B.handoff_workspace(MAX_ROWS)
    yield w
    B.lora_set_handoff_polls(-1)


def _stores(cfg, layout, d_in, outs, rank, r_max):
    scale = wl.scale_for_rank(rank)
    S = len(rank)
    P = {"dense": None, "paged8": 8, "paged56": 56}[layout]
    if P:
        return [wl.paged_store(cfg, p, S, d_in, d_out, rank, scale, P, spare_pages=5) for p, d_out in enumerate(outs)]
    return [wl.dense_store(cfg, p, S, d_in, d_out, rank, scale, r_max=r_max) for p, d_out in enumerate(outs)]


def _assert_clear(work, label):
    assert int(work.count_nonzero()) == 0, f"{label}: workspace not cleared"


def _compare(label, x_d, idx_d, ws, dcs, work):
    """Two launches, then the hand-off form at the default and at a zero poll limit, and
    both forms again with the streaming-weights hint (lora_set_stream_weights; same bits
    whether or not the rows' adapters are distinct); returns the two-launch results."""
    results = {}
    for mode in ("two", "handoff", "local", "two-sw", "handoff-sw"):
        for dc in dcs:
            dc.reset()
        items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
        B.lora_set_stream_weights(mode.endswith("-sw"))
        try:
            if mode.startswith("two"):
                B.lora_bgmv_multi(x_d, idx_d, items)
            else:
                B.lora_set_handoff_polls(0 if mode == "local" else -1)
                try:
                    B.lora_bgmv_multi_handoff(x_d, idx_d, items, work)
                finally:
                    B.lora_set_handoff_polls(-1)
        finally:
            B.lora_set_stream_weights(False)
        results[mode] = [dc.results() for dc in dcs]
        _assert_clear(work, f"{label} {mode}")
    base = results["two"]
    for mode in ("handoff", "local", "two-sw", "handoff-sw"):
        for p, ((yb, vb), (yg, vg)) in enumerate(zip(base, results[mode])):
            assert np.array_equal(yb.view(np.uint16), yg.view(np.uint16)), f"{label}: {mode} proj {p}: y"
            assert np.array_equal(vb.view(np.uint32), vg.view(np.uint32)), f"{label}: {mode} proj {p}: v"
    return base


def _case(work, label, cfg, layout, d_in, outs, rank, idx, r_max=64):
    import torch
    G.say(f"case handoff-{label} layout={layout} n={len(idx)} {d_in}->{outs} r_max={r_max}")
    stores = _stores(cfg, layout, d_in, outs, np.asarray(rank, dtype=np.int32), r_max)
    x, _ = wl.activations(cfg, 0, len(idx), d_in, 8)
    y0s = [wl.activations(cfg, 20 + p, len(idx), 8, d_out)[1] for p, d_out in enumerate(outs)]
    ws = [B.weights_from_store(st) for st in stores]
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    dcs = [G.DeviceCase(x, y0, st.r_max) for y0, st in zip(y0s, stores)]
    base = _compare(label, dcs[0].x, idx_d, ws, dcs, work)
    for p, (st, dc) in enumerate(zip(stores, dcs)):
        y_ref, v_ref = oracle.bgmv(st, x, y0s[p], idx, nthreads=16)
        yb, vb = base[p]
        G.check(dc, yb, vb, y_ref, v_ref, G.active_rows(idx, st.rank), f"handoff-{label}-p{p}")


def test_decode_7b_qkv(work):
    """32 rows, 32 distinct rank-16 adapters, q/k/v of 4096 in one call."""
    b = wl.batch_decode_distinct()
    _case(work, "7b-qkv", 2, "dense", 4096, (4096, 4096, 4096), [16] * 32, b.idx, r_max=16)


def test_decode_7b_gate_up_and_down(work):
    b = wl.batch_decode_distinct()
    _case(work, "7b-gate-up", 2, "dense", 4096, (11008, 11008), [16] * 32, b.idx, r_max=16)
    _case(work, "7b-down", 2, "dense", 11008, (4096,), [16] * 32, b.idx, r_max=16)


def test_one_row(work):
    _case(work, "one-row", 3, "dense", 4096, (4096,), [16, 16], np.array([1], dtype=np.int32), r_max=16)


@pytest.mark.parametrize("layout", ["dense", "paged8", "paged56"])
def test_ragged_mixed_ranks(work, layout):
    """Widths that are not multiples of 512 columns or 256 octets; ranks 0..64 with
    r_max 64, rows without adapter."""
    idx = np.random.default_rng(7).integers(-1, 7, size=150).astype(np.int32)
    _case(work, f"ragged-{layout}", 11, layout, 1288, (1064, 56, 2632), [1, 64, 0, 17, 8, 33, 64], idx)


@pytest.mark.parametrize("r_max", [20, 32])
def test_r_max_between_blocks(work, r_max):
    rank = [r_max, 3, 16, 0, 9]
    idx = np.random.default_rng(r_max).integers(-1, 5, size=40).astype(np.int32)
    _case(work, f"r_max-{r_max}", 12, "dense", 2056, (2048, 1032), rank, idx, r_max=r_max)


def test_more_workgroups_than_fit_at_once(work):
    """512 rows x 4 projections: far more shrink and expand workgroups than the CUs hold
    together, so expand workgroups start while others are still queued."""
    idx = np.random.default_rng(5).integers(-1, 9, size=MAX_ROWS).astype(np.int32)
    _case(work, "many-rows", 13, "dense", 2048, (4096, 1024, 2048, 512), [16, 8, 64, 32, 0, 16, 1, 48, 16], idx)


def test_paged_70b_shapes(work):
    """70B k/v width with 1024-element pages, 256 rows over 2000 adapters of ranks 8..64."""
    import torch
    d_in, d_out, P, S = 8192, 1024, 1024, 2000
    rank = wl.paged_ranks(S)
    b = wl.batch_paged_zipf(256, S)
    scale = wl.scale_for_rank(rank)
    G.say(f"case handoff-paged-70b n=256 {d_in}->{d_out}")
    pool, pt, a_off, b_off, rows, compact_pt = G.paged_device_pool(5, wl.PROJ_IDS["k"], rank, d_in, d_out, P, b.idx)
    ostore = wl.PagedStore(S, d_in, d_out, 64, P, rank, scale, rows, compact_pt, a_off, b_off)
    x, y0 = wl.activations(5, wl.PROJ_IDS["k"], 256, d_in, d_out)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=64, rank=dev(rank), scale=dev(scale), pool=pool,
                  page_elems=P, page_table=dev(pt), a_pt_off=dev(a_off), b_pt_off=dev(b_off))
    dc = G.DeviceCase(x, y0, 64)
    base = _compare("paged-70b", dc.x, dev(b.idx), [w], [dc], work)
    y_ref, v_ref = oracle.bgmv(ostore, x, y0, b.idx, nthreads=16)
    G.check(dc, *base[0], y_ref, v_ref, G.active_rows(b.idx, rank), "handoff-paged-70b")


def _segs(idx, num_slots, tile_rows, hint=None):
    row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(idx, num_slots)
    tiles = B.lora_build_tiles(seg_ptr, seg_slot, tile_rows)
    segs = B.segments_to_device(tiles, row_map, n_act)
    if hint is not None:
        segs.c.max_rows = hint  # a launch-shape hint below the real tile height
    return segs


def _compare_sgmv(label, x_d, segs, n, ws, dcs, work, expect_clear=True):
    """Two launches, then the segment-form hand-off at the default and at a zero poll
    limit; returns the two-launch results."""
    results = {}
    for mode in ("two", "handoff", "local"):
        for dc in dcs:
            dc.reset()
        items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
        if mode == "two":
            B.lora_sgmv_shrink_multi(x_d, segs, items, n)
            B.lora_sgmv_expand_multi(segs, items, n)
        else:
            B.lora_set_handoff_polls(0 if mode == "local" else -1)
            try:
                B.lora_sgmv_multi_handoff(x_d, segs, items, n, work)
            finally:
                B.lora_set_handoff_polls(-1)
        results[mode] = [dc.results() for dc in dcs]
        _assert_clear(work, f"{label} {mode}")
    base = results["two"]
    for mode in ("handoff", "local"):
        for p, ((yb, vb), (yg, vg)) in enumerate(zip(base, results[mode])):
            assert np.array_equal(yb.view(np.uint16), yg.view(np.uint16)), f"{label}: {mode} proj {p}: y"
            assert np.array_equal(vb.view(np.uint32), vg.view(np.uint32)), f"{label}: {mode} proj {p}: v"
    return base


def _case_sgmv(work, label, cfg, layout, d_in, outs, rank, idx, tile_rows, r_max=64, hint=None):
    G.say(f"case handoff-sgmv-{label} layout={layout} n={len(idx)} {d_in}->{outs} r_max={r_max} tiles={tile_rows}")
    stores = _stores(cfg, layout, d_in, outs, np.asarray(rank, dtype=np.int32), r_max)
    x, _ = wl.activations(cfg, 0, len(idx), d_in, 8)
    y0s = [wl.activations(cfg, 20 + p, len(idx), 8, d_out)[1] for p, d_out in enumerate(outs)]
    ws = [B.weights_from_store(st) for st in stores]
    dcs = [G.DeviceCase(x, y0, st.r_max) for y0, st in zip(y0s, stores)]
    segs = _segs(idx, len(rank), tile_rows, hint)
    base = _compare_sgmv(label, dcs[0].x, segs, len(idx), ws, dcs, work)
    for p, (st, dc) in enumerate(zip(stores, dcs)):
        y_ref, v_ref = oracle.bgmv(st, x, y0s[p], idx, nthreads=16)
        yb, vb = base[p]
        G.check(dc, yb, vb, y_ref, v_ref, G.active_rows(idx, st.rank), f"handoff-sgmv-{label}-p{p}")


@pytest.mark.parametrize("pop", ["uniform", "skewed", "identical"])
def test_sgmv_decode_13b_mixes(work, pop):
    """The 13B decode mixes (64 rows, 16 slots of rank 64, 10 % of rows without
    adapter) at their own tile heights, q/k/v in one call."""
    b = wl.batch_decode_mix(pop)
    seg_ptr = B.lora_build_segments(b.idx, 16)[1]
    _case_sgmv(work, f"13b-{pop}", 3, "dense", 5120, (5120, 5120, 5120), [64] * 16, b.idx,
               B.lora_pick_tile_rows(seg_ptr))


@pytest.mark.parametrize("tile_rows,hint", [(1, None), (2, None), (4, None), (6, None), (4, 1), (3, 2)])
def test_sgmv_ragged_mixed_ranks(work, tile_rows, hint):
    """Rows in shuffled order (row map), ranks 0..64, widths off the 512-column and
    256-octet grids, tiles of 1, 2, 4 and 6 rows; and tiles taller than the descriptor's
    row-height hint says (the hint plans fewer rows per pass than a tile has)."""
    idx = np.random.default_rng(17).integers(-1, 7, size=150).astype(np.int32)
    _case_sgmv(work, f"ragged-t{tile_rows}-h{hint}", 11, "dense", 1288, (1064, 56, 2632), [1, 64, 0, 17, 8, 33, 64],
               idx, tile_rows, hint=hint)


@pytest.mark.parametrize("layout,tile_rows,hint", [("dense", 16, None), ("dense", 64, None), ("paged8", 4, None),
                                                   ("dense", 64, 16), ("dense", 32, 8), ("paged8", 32, 8),
                                                   ("paged8", 6, None), ("paged8", 3, 1), ("paged8", 4, 2)])
def test_sgmv_two_launch_cases(work, layout, tile_rows, hint):
    """Taller tiles (MFMA kernels) and paged weights: the call makes the two launches;
    also with a row-height hint below the tiles' height (the MFMA shrinks then take the
    tile's rows in several blocks, the VALU expand one row per pass)."""
    idx = np.random.default_rng(19).integers(-1, 5, size=96).astype(np.int32)
    _case_sgmv(work, f"{layout}-t{tile_rows}-h{hint}", 12, layout, 2048, (2048, 1024), [16, 8, 64, 0, 32], idx,
               tile_rows, hint=hint)


def test_graph_replays_share_the_workspace_with_eager_calls(work):
    """A captured hand-off call replayed four times; between replays an eager hand-off
    call on other inputs (same workspace).  Every replay must give the eager bits of its
    own inputs, and every eager call those of the two-launch path."""
    import torch
    G.say("case handoff-graph")
    rank = np.array([16, 8, 0, 16, 4], dtype=np.int32)
    mk = lambda cfg, n: (_stores(cfg, "dense", 2048, (2048, 1024), rank, 16),
                         np.random.default_rng(cfg).integers(-1, 5, size=n).astype(np.int32),
                         wl.activations(cfg, 0, n, 2048, 8)[0])
    sa, ia, xa = mk(21, 48)
    sb, ib, xb = mk(22, 33)
    wa, wb = [B.weights_from_store(s) for s in sa], [B.weights_from_store(s) for s in sb]
    da = [G.DeviceCase(xa, wl.activations(21, 20 + p, 48, 8, s.d_out)[1], 16) for p, s in enumerate(sa)]
    db = [G.DeviceCase(xb, wl.activations(22, 20 + p, 33, 8, s.d_out)[1], 16) for p, s in enumerate(sb)]
    ia_d, ib_d = torch.from_numpy(ia).cuda(), torch.from_numpy(ib).cuda()
    want_b = _compare("graph-b", db[0].x, ib_d, wb, db, work)
    want_a = _compare("graph-a", da[0].x, ia_d, wa, da, work)
    items_a = [(w, dc.v, dc.y) for w, dc in zip(wa, da)]
    items_b = [(w, dc.v, dc.y) for w, dc in zip(wb, db)]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        B.lora_bgmv_multi_handoff(da[0].x, ia_d, items_a, work, stream=torch.cuda.current_stream())
    for i in range(4):
        for dc in da:
            dc.reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p, dc in enumerate(da):
            y, v = dc.results()
            assert np.array_equal(y.view(np.uint16), want_a[p][0].view(np.uint16)), f"replay {i} proj {p}: y"
            assert np.array_equal(v.view(np.uint32), want_a[p][1].view(np.uint32)), f"replay {i} proj {p}: v"
        _assert_clear(work, f"replay {i}")
        for dc in db:
            dc.reset()
        B.lora_bgmv_multi_handoff(db[0].x, ib_d, items_b, work)
        for p, dc in enumerate(db):
            y, v = dc.results()
            assert np.array_equal(y.view(np.uint16), want_b[p][0].view(np.uint16)), f"eager {i} proj {p}: y"
        _assert_clear(work, f"eager {i}")
    del g
