"""GPU: the segment form given as offsets, the way the pages' SGMV call takes it.

Punica's SGMV call takes the segment offsets s (s[0] = 0, s[-1] = the batch) and one
adapter index per segment directly (Punica digest, section 5.4; Punica summary,
section 3.4 "The SGMV Operator: What It Computes").  Here lora_sgmv_shrink and
lora_sgmv_expand receive the device arrays seg_ptr / seg_slot (and a row map when the
rows are grouped by the metadata builder), and every workgroup finds its own tile on the
device.  Each case is checked against the fp64 oracle within the stated tolerance
(max |dy| <= 1e-2, relative Frobenius <= 1e-3 over the whole y; v within 1e-5; untouched
rows, guard rows and padding bit-identical) and bit for bit against the same call with
the host-built tile list, whose cut is the same.
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


def _both_forms(label, store, x, y0, seg_ptr, seg_slot, row_map=None, tile_rows=0, check_tiles_equal=True):
    """Offsets form and tile-list form of the same segments: each against the oracle,
    and against each other bit for bit."""
    n = x.shape[0]
    idx = np.full(n, -1, np.int32)
    rows = np.arange(n) if row_map is None else np.asarray(row_map)
    for g in range(len(seg_slot)):
        idx[rows[seg_ptr[g]:seg_ptr[g + 1]]] = seg_slot[g]
    y_ref, v_ref = oracle.sgmv(store, x, y0, seg_ptr, seg_slot, row_map, nthreads=NTHREADS)
    w = B.weights_from_store(store)
    T = tile_rows if tile_rows else (64 if n >= 128 * len(seg_slot) else 2)
    out = {}
    for form in ("offsets", "tiles"):
        dc = G.DeviceCase(x, y0, store.r_max)
        if form == "offsets":
            segs = B.segments_from_offsets(seg_ptr, seg_slot, row_map, tile_rows, n_rows=n,
                                           num_slots=store.num_slots)
        else:
            tiles = B.lora_build_tiles(seg_ptr, seg_slot, T)
            n_pos = len(row_map) if row_map is not None else n
            segs = B.segments_to_device(tiles, row_map, n_pos, n_rows=n, num_slots=store.num_slots)
        G.say(f"case {label} {form} n={n} n_seg={len(seg_slot)} tile_rows={T}")
        B.lora_sgmv_shrink(dc.v, dc.x, w, segs)
        B.lora_sgmv_expand(dc.y, dc.v, w, segs)
        out[form] = dc.results()
        G.check(dc, *out[form], y_ref, v_ref, G.active_rows(idx, store.rank), f"{label}-{form}")
    if check_tiles_equal:
        assert np.array_equal(out["offsets"][0].view(np.uint16), out["tiles"][0].view(np.uint16)), f"{label}: y"
        assert np.array_equal(out["offsets"][1].view(np.uint32), out["tiles"][1].view(np.uint32)), f"{label}: v"
    return out


def test_tiny_sgmv_offsets():
    """The tiny workload: 8 rows in segments [1, 3, 2, 2], seg_ptr = [0, 1, 4, 6, 8]."""
    b = wl.batch_tiny_sgmv()
    assert b.seg_ptr.tolist() == [0, 1, 4, 6, 8]
    store = wl.dense_store(1, 0, 4, 1024, 1024, 16, wl.scale_for_rank(16))
    x, y0 = wl.activations(1, 0, b.n, 1024, 1024)
    _both_forms("tiny", store, x, y0, b.seg_ptr, b.seg_slot)


@pytest.mark.parametrize("d_out", [4096, 11008])
def test_prefill_7b_offsets(d_out):
    """The prefill workload's offsets straight to the calls: 16 log-uniform prompts,
    12,907 rows, 64-row tiles chosen by the library from n_rows and n_seg."""
    b = wl.batch_prefill()
    store = wl.dense_store(4, wl.PROJ_IDS["q"], 16, 4096, d_out, 16, 2.0, fill=np.unique(b.idx))
    x, y0 = wl.activations(4, wl.PROJ_IDS["q"], b.n, 4096, d_out)
    _both_forms(f"prefill-7b-{d_out}", store, x, y0, b.seg_ptr, b.seg_slot)


@pytest.mark.parametrize("popularity", ["uniform", "skewed", "identical"])
def test_decode_13b_offsets_with_row_map(popularity):
    """Rows grouped by adapter through the builder's row map (6 of 64 rows without one)."""
    b = wl.batch_decode_mix(popularity)
    row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(b.idx, 16)
    store = wl.dense_store(3, 5, 16, 5120, 13824, 64, 0.5, fill=np.unique(b.idx))
    x, y0 = wl.activations(3, 5, b.n, 5120, 13824)
    _both_forms(f"decode-13b-{popularity}", store, x, y0, seg_ptr, seg_slot, row_map=row_map)


@pytest.mark.parametrize("tile_rows", [1, 2, 4, 16, 64])
def test_empty_and_unassigned_segments_and_spare_capacity(tile_rows):
    """Empty segments, a segment with slot -1, rank-0 slots, segments longer than a
    tile, and a capacity of 40 segments of which the last 30 are empty."""
    lens = [3, 0, 70, 1, 0, 17, 9, 2, 130, 5] + [0] * 30
    slots = [4, 2, 0, -1, 3, 1, 5, 4, 2, 6] + [0] * 30
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.array(slots, np.int32)
    rank = np.array([16, 8, 0, 33, 64, 5, 12], np.int32)
    store = wl.dense_store(25, 0, 7, 1288, 1064, rank, wl.scale_for_rank(rank), r_max=64)
    n = int(seg_ptr[-1]) + 6      # rows past the last segment stay untouched
    x, y0 = wl.activations(25, 0, n, 1288, 1064)
    _both_forms(f"capacity-{tile_rows}", store, x, y0, seg_ptr, seg_slot, tile_rows=tile_rows)


@pytest.mark.parametrize("kind", ["decode_1500", "long_1100"])
def test_more_segments_than_one_scan_chunk(kind):
    """More segments than threads in a workgroup: 1500 one-row segments (2-row VALU
    tiles, 256-thread workgroups scan 6 chunks) and 1100 segments of 1 or 40 rows on
    64-row MFMA tiles (1024-thread shrink workgroups scan 2 chunks)."""
    if kind == "decode_1500":
        lens = [1] * 1500
        T, d = 0, 1024
    else:
        lens = [1] * 1000 + [40] * 100
        lens = list(np.random.default_rng(7).permutation(lens))
        T, d = 64, 512
    S = len(lens)
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.random.default_rng(8).permutation(S).astype(np.int32)
    store = wl.dense_store(26, 0, S, d, d, 16, 2.0)
    x, y0 = wl.activations(26, 0, int(seg_ptr[-1]), d, d)
    _both_forms(kind, store, x, y0, seg_ptr, seg_slot, tile_rows=T)


@pytest.mark.parametrize("tile_rows", [2, 64])
def test_paged_offsets(tile_rows):
    """Paged weights (56-element pages) with the offsets form, VALU and MFMA tiles."""
    lens = [1, 90, 3, 0, 40, 2]
    seg_ptr = wl.segments_from_lengths(lens)
    seg_slot = np.array([2, 0, 4, 1, 3, 2], np.int32)
    rank = np.array([16, 64, 0, 17, 8], np.int32)
    store = wl.paged_store(27, 0, 5, 1288, 1064, rank, wl.scale_for_rank(rank), 56, spare_pages=9)
    x, y0 = wl.activations(27, 0, int(seg_ptr[-1]), 1288, 1064)
    _both_forms(f"paged-{tile_rows}", store, x, y0, seg_ptr, seg_slot, tile_rows=tile_rows)


def test_one_launch_handoff_with_offsets():
    """The one-launch form (v handed from the shrink's workgroups to the expand's) over
    offsets with 2-row tiles: bit for bit the two launches, workspace left cleared."""
    import torch
    b = wl.batch_decode_mix("skewed")
    row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(b.idx, 16)
    d_in, outs = 5120, (5120, 1024, 1024)
    stores = [wl.dense_store(3, 40 + p, 16, d_in, d_out, 64, 0.5, fill=np.unique(b.idx)) for p, d_out in enumerate(outs)]
    x, _ = wl.activations(3, 40, b.n, d_in, 8)
    y0s = [wl.activations(3, 40 + p, b.n, d_in, d_out)[1] for p, d_out in enumerate(outs)]
    ws = [B.weights_from_store(s) for s in stores]
    segs = B.segments_from_offsets(seg_ptr, seg_slot, row_map, 0, n_rows=b.n, num_slots=16)
    work = B.handoff_workspace(b.n)
    res = {}
    for mode in ("two", "one"):
        dcs = [G.DeviceCase(x, y0, 64) for y0 in y0s]
        items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
        if mode == "two":
            B.lora_sgmv_shrink_multi(dcs[0].x, segs, items, n_rows=b.n)
            B.lora_sgmv_expand_multi(segs, items, b.n)
        else:
            B.lora_sgmv_multi_handoff(dcs[0].x, segs, items, b.n, work)
        res[mode] = [dc.results() for dc in dcs]
        torch.cuda.synchronize()
        assert int(work.count_nonzero()) == 0, f"{mode}: workspace not cleared"
    act = G.active_rows(b.idx, stores[0].rank)
    for p in range(len(outs)):
        assert np.array_equal(res["two"][p][0].view(np.uint16), res["one"][p][0].view(np.uint16)), f"y {p}"
        assert np.array_equal(res["two"][p][1].view(np.uint32), res["one"][p][1].view(np.uint32)), f"v {p}"
        y_ref, v_ref = oracle.sgmv(stores[p], x, y0s[p], seg_ptr, seg_slot, row_map, nthreads=NTHREADS)
        dc = G.DeviceCase(x, y0s[p], 64)
        G.check(dc, *res["one"][p], y_ref, v_ref, act, f"handoff-offsets-p{p}")


def test_graph_replays_new_batches_in_place():
    """One captured graph (shrink + expand over offsets with a capacity of 24 segments)
    replayed for three different batches written into the same device arrays between
    replays; every replay against the oracle and against an eager call."""
    import torch
    S, d_in, d_out, n = 12, 1024, 1536, 96
    rank = np.array([16, 8, 0, 33, 64, 5, 12, 16, 1, 40, 64, 7], np.int32)
    store = wl.dense_store(28, 0, S, d_in, d_out, rank, wl.scale_for_rank(rank), r_max=64)
    w = B.weights_from_store(store)
    cap = 24
    sp_d = torch.zeros(cap + 1, dtype=torch.int32, device="cuda")
    ss_d = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    rm_d = torch.zeros(n, dtype=torch.int32, device="cuda")
    segs = B.Segments.offsets(sp_d, ss_d, rm_d, tile_rows=4)
    x, y0 = wl.activations(28, 0, n, d_in, d_out)
    dc = G.DeviceCase(x, y0, 64)
    rng = np.random.default_rng(11)
    batches = []
    for k in range(3):
        idx = rng.integers(-1, S, size=n).astype(np.int32)
        row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(idx, S)
        batches.append((idx, row_map, seg_ptr, seg_slot))

    def load(batch):
        idx, row_map, seg_ptr, seg_slot = batch
        g = len(seg_slot)
        sp = np.full(cap + 1, seg_ptr[-1], np.int32)
        sp[:g + 1] = seg_ptr
        ss = np.full(cap, -1, np.int32)
        ss[:g] = seg_slot
        rm = np.zeros(n, np.int32)
        rm[:len(row_map)] = row_map
        sp_d.copy_(torch.from_numpy(sp))
        ss_d.copy_(torch.from_numpy(ss))
        rm_d.copy_(torch.from_numpy(rm))
        dc.reset()
        torch.cuda.synchronize()

    def call():
        B.lora_sgmv_shrink(dc.v, dc.x, w, segs)
        B.lora_sgmv_expand(dc.y, dc.v, w, segs)

    load(batches[0])
    call()                                   # eager pass before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep, batch in enumerate(batches + batches[:1]):
        idx, row_map, seg_ptr, seg_slot = batch
        y_ref, v_ref = oracle.sgmv(store, x, y0, seg_ptr, seg_slot, row_map, nthreads=NTHREADS)
        load(batch)
        call()
        eager = dc.results()
        load(batch)
        g.replay()
        replay = dc.results()
        G.say(f"case graph replay {rep}: {len(seg_slot)} segments")
        assert np.array_equal(eager[0].view(np.uint16), replay[0].view(np.uint16)), f"replay {rep}: y"
        assert np.array_equal(eager[1].view(np.uint32), replay[1].view(np.uint32)), f"replay {rep}: v"
        G.check(dc, *replay, y_ref, v_ref, G.active_rows(idx, rank), f"graph-replay-{rep}")
