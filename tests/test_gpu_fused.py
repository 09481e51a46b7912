"""GPU: the one-launch decode path (lora_bgmv_multi with chunks >= 1) against the
two-launch path (chunks = -1) and the fp64 oracle.

The one-launch kernel recomputes each row's v in every workgroup of the row and is
documented to give the same bits as the separate shrink and expand, so every case
compares whole buffers (guard rows and padding included) bitwise across chunk counts,
and the two-launch result against the oracle within the usual tolerance.
"""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
CHUNKS = (-1, 1, 2, 3, 4, 5, 8, 64, 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield


def _stores(cfg, layout, d_in, outs, rank, r_max):
    scale = wl.scale_for_rank(rank)
    S = len(rank)
    P = {"dense": None, "paged8": 8, "paged56": 56}[layout]
    if P:
        return [wl.paged_store(cfg, p, S, d_in, d_out, rank, scale, P, spare_pages=5) for p, d_out in enumerate(outs)]
    return [wl.dense_store(cfg, p, S, d_in, d_out, rank, scale, r_max=r_max) for p, d_out in enumerate(outs)]


def _case(label, cfg, layout, d_in, outs, rank, idx, r_max=64):
    import torch
    G.say(f"case {label} layout={layout} n={len(idx)} {d_in}->{outs} r_max={r_max}")
    stores = _stores(cfg, layout, d_in, outs, np.asarray(rank, dtype=np.int32), r_max)
    x, _ = wl.activations(cfg, 0, len(idx), d_in, 8)
    y0s = [wl.activations(cfg, 20 + p, len(idx), 8, d_out)[1] for p, d_out in enumerate(outs)]
    ws = [B.weights_from_store(st) for st in stores]
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    dcs = [G.DeviceCase(x, y0, st.r_max) for y0, st in zip(y0s, stores)]
    results = {}
    for chunks in CHUNKS:
        for dc in dcs:
            dc.reset()
        items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
        B.lora_bgmv_multi(dcs[0].x, idx_d, items, chunks=chunks)
        results[chunks] = [dc.results() for dc in dcs]
    base = results[-1]
    for chunks, got in results.items():
        for p, ((yb, vb), (yg, vg)) in enumerate(zip(base, got)):
            assert np.array_equal(yb.view(np.uint16), yg.view(np.uint16)), f"{label}: chunks={chunks} proj {p}: y"
            assert np.array_equal(vb.view(np.uint32), vg.view(np.uint32)), f"{label}: chunks={chunks} proj {p}: v"
    for p, (st, dc) in enumerate(zip(stores, dcs)):
        y_ref, v_ref = oracle.bgmv(st, x, y0s[p], idx, nthreads=16)
        yb, vb = base[p]
        G.check(dc, yb, vb, y_ref, v_ref, G.active_rows(idx, st.rank), f"{label}-p{p}")


def test_decode_7b_qkv_shapes():
    """32 rows, 32 distinct rank-16 adapters, q/k/v of 4096 in one call."""
    b = wl.batch_decode_distinct()
    _case("7b-qkv", 2, "dense", 4096, (4096, 4096, 4096), [16] * 32, b.idx, r_max=16)


def test_decode_7b_down_and_gate_up_shapes():
    b = wl.batch_decode_distinct()
    _case("7b-down", 2, "dense", 11008, (4096,), [16] * 32, b.idx, r_max=16)
    _case("7b-gate-up", 2, "dense", 4096, (11008, 11008), [16] * 32, b.idx, r_max=16)


@pytest.mark.parametrize("layout", ["dense", "paged8", "paged56"])
def test_ragged_mixed_ranks(layout):
    """Widths that are not multiples of 512 columns or 256 octets; ranks 0..64 with
    r_max 64 (blocks of B loads), rows without adapter."""
    idx = np.random.default_rng(7).integers(-1, 7, size=150).astype(np.int32)
    _case(f"ragged-{layout}", 11, layout, 1288, (1064, 56, 2632), [1, 64, 0, 17, 8, 33, 64], idx)


@pytest.mark.parametrize("r_max", [20, 32])
def test_r_max_between_blocks(r_max):
    """r_max that is not a multiple of 16 rank-rows (last shrink batch partly empty)."""
    rank = [r_max, 3, 16, 0, 9]
    idx = np.random.default_rng(r_max).integers(-1, 5, size=40).astype(np.int32)
    _case(f"r_max-{r_max}", 12, "dense", 2056, (2048, 1032), rank, idx, r_max=r_max)


def test_paged_70b_shapes():
    """70B k/v width with 1024-element pages, the production page size."""
    import torch
    d_in, d_out, P, S = 8192, 1024, 1024, 2000
    rank = wl.paged_ranks(S)
    b = wl.batch_paged_zipf(256, S)
    scale = wl.scale_for_rank(rank)
    G.say(f"case paged-70b-fused n=256 {d_in}->{d_out}")
    pool, pt, a_off, b_off, rows, compact_pt = G.paged_device_pool(5, wl.PROJ_IDS["k"], rank, d_in, d_out, P, b.idx)
    ostore = wl.PagedStore(S, d_in, d_out, 64, P, rank, scale, rows, compact_pt, a_off, b_off)
    x, y0 = wl.activations(5, wl.PROJ_IDS["k"], 256, d_in, d_out)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=64, rank=dev(rank), scale=dev(scale), pool=pool,
                  page_elems=P, page_table=dev(pt), a_pt_off=dev(a_off), b_pt_off=dev(b_off))
    idx_d = dev(b.idx)
    dc = G.DeviceCase(x, y0, 64)
    out = {}
    for chunks in (-1, 1, 2):
        dc.reset()
        B.lora_bgmv_multi(dc.x, idx_d, [(w, dc.v, dc.y)], chunks=chunks)
        out[chunks] = dc.results()
    for chunks in (1, 2):
        assert np.array_equal(out[-1][0].view(np.uint16), out[chunks][0].view(np.uint16)), f"chunks={chunks}: y"
        assert np.array_equal(out[-1][1].view(np.uint32), out[chunks][1].view(np.uint32)), f"chunks={chunks}: v"
    y_ref, v_ref = oracle.bgmv(ostore, x, y0, b.idx, nthreads=16)
    G.check(dc, *out[-1], y_ref, v_ref, G.active_rows(b.idx, rank), "paged-70b-fused")
