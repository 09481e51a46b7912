"""GPU parity of the grouped MFMA launches that a 7B prefill step makes.

A prefill batch (16 prompts of log-uniform length, 64-row tiles) runs q/k/v in one
shrink and one expand launch, gate/up in another pair, and o and down alone.  With
rank 16 each projection is one 16-rank slice, so a q/k/v shrink workgroup holds the
slices of three different projections and a gate/up workgroup those of two: the
slices of one workgroup straddle projections.  Each projection of a grouped launch
must equal its single-projection call bit for bit and the fp64 oracle within the
stated tolerance (max |dy| <= 1e-2, relative Frobenius <= 1e-3 over the whole y;
v within 1e-5), with untouched rows, guard rows and padding columns bit-identical.

The pages count seven adapted projections per layer, one segment layout shared by all
of them (Punica digest, section 5.3); the operator is the SGMV of the Punica summary,
section 3.4 "The SGMV Operator: What It Computes".
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


def _grouped_vs_single(label, cfg_id, pids, d_in, d_outs, num_slots, ranks, r_maxs, seg_ptr, seg_slot,
                       max_tile_rows, x_pid):
    """Builds one store per projection, runs the projections one call each and as one
    grouped launch pair, and checks both against the oracle and each other."""
    n = int(seg_ptr[-1])
    idx = np.repeat(seg_slot, np.diff(seg_ptr)).astype(np.int32)
    x, _ = wl.activations(cfg_id, x_pid, n, d_in, 8)
    stores, y0s, refs = [], [], []
    for pid, d_out, rank, r_max in zip(pids, d_outs, ranks, r_maxs):
        store = wl.dense_store(cfg_id, pid, num_slots, d_in, d_out, rank, wl.scale_for_rank(rank), r_max=r_max,
                               fill=np.unique(idx))
        _, y0 = wl.activations(cfg_id, pid, n, d_in, d_out)
        stores.append(store)
        y0s.append(y0)
        refs.append(oracle.sgmv(store, x, y0, seg_ptr, seg_slot, nthreads=NTHREADS))
    tiles = B.lora_build_tiles(seg_ptr, seg_slot, max_tile_rows)
    nprob, msgs = oracle.check_tiles(tiles, seg_ptr, seg_slot, max_tile_rows)
    assert nprob == 0, msgs[:3]
    segs = B.segments_to_device(tiles, None, n)
    ws = [B.weights_from_store(st) for st in stores]
    out = {}
    for mode in ("single", "grouped"):
        dcs = [G.DeviceCase(x, y0, st.r_max) for st, y0 in zip(stores, y0s)]
        items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
        xd = dcs[0].x
        G.say(f"case {label} {mode} n={n} {d_in}->{'/'.join(map(str, d_outs))} tiles={len(tiles)}x{max_tile_rows}")
        if mode == "single":
            for w, v, y in items:
                B.lora_sgmv_shrink(v, xd, w, segs)
                B.lora_sgmv_expand(y, v, w, segs)
        else:
            B.lora_sgmv_shrink_multi(xd, segs, items)
            B.lora_sgmv_expand_multi(segs, items, n)
        out[mode] = [dc.results() for dc in dcs]
        for p, dc in enumerate(dcs):
            y_ref, v_ref = refs[p]
            G.check(dc, *out[mode][p], y_ref, v_ref, G.active_rows(idx, stores[p].rank), f"{label}-{mode}-p{p}")
    for p in range(len(pids)):
        (ys, vs), (yg, vg) = out["single"][p], out["grouped"][p]
        dv = np.argwhere(vs.view(np.uint32) != vg.view(np.uint32))
        dy = np.argwhere(ys.view(np.uint16) != yg.view(np.uint16))
        if len(dv) or len(dy):
            G.say(f"  {label} p{p}: {len(dv)} v words differ (first {dv[:4].tolist()}), {len(dy)} y elements differ "
                  f"(first {dy[:4].tolist()}, rows {np.unique(dy[:, 0])[:12].tolist()})")
            if len(dv):
                r, c = dv[0]
                G.say(f"  v single {vs[r, c]!r} grouped {vg[r, c]!r}")
        assert not len(dv), f"{label}: projection {p} v differs"
        assert not len(dy), f"{label}: projection {p} y differs"


@pytest.mark.parametrize("group", ["qkv", "gate_up", "o", "down"])
def test_prefill_7b_launch_groups(group):
    """The bench's prefill launches at full size: 12,907 rows in 16 segments, 64-row tiles,
    rank 16: q/k/v (3 x 4096 -> 4096) and gate/up (2 x 4096 -> 11008) grouped, o and
    down (11008 -> 4096) alone."""
    b = wl.batch_prefill()
    names = {"qkv": ("q", "k", "v"), "gate_up": ("gate", "up"), "o": ("o",), "down": ("down",)}[group]
    d_in = wl.LLAMA2_7B[names[0]][0]
    d_outs = [wl.LLAMA2_7B[p][1] for p in names]
    pids = [wl.PROJ_IDS[p] for p in names]
    k = len(names)
    _grouped_vs_single(f"prefill-7b-{group}", 4, pids, d_in, d_outs, 16, [16] * k, [16] * k, b.seg_ptr,
                       b.seg_slot, B.lora_pick_tile_rows(b.seg_ptr), pids[0])


@pytest.mark.parametrize("max_tile_rows", [16, 32, 64])
@pytest.mark.parametrize("layout", ["r32_16_32", "r16x4", "r8_24"])
def test_grouped_slices_straddle_projections(layout, max_tile_rows):
    """Projections whose rank slices do not line up with a workgroup's slice group:
    r_max (32, 16, 32) gives slices 2 + 1 + 2 (groups of three straddle the first two
    projections), four rank-16 projections fill a group of four (three at 64-row
    tiles), and r_max (8, 24) gives 1 + 2 slices.  Mixed ranks per slot, a ragged d_in
    (last 512-column chunk partial) and different widths per projection."""
    lens = [150, 9, 70, 33, 1, 64, 200]
    seg_ptr = wl.segments_from_lengths(lens)
    S = 9
    seg_slot = np.array([3, 0, 8, 5, 1, 2, 7], dtype=np.int32)
    d_in = 1288
    base = np.array([16, 8, 1, 12, 16, 5, 9, 16, 3], dtype=np.int32)
    if layout == "r32_16_32":
        r_maxs, d_outs = [32, 16, 32], [1032, 520, 2056]
        ranks = [np.minimum(base * 2, 32), base, np.minimum(base * 2 + 1, 32)]
    elif layout == "r16x4":
        r_maxs, d_outs = [16, 16, 16, 16], [1032, 512, 520, 1544]
        ranks = [base, np.maximum(base - 1, 0), np.minimum(base + 3, 16), base[::-1].copy()]
    else:
        r_maxs, d_outs = [8, 24], [2056, 1032]
        ranks = [np.minimum(base, 8), np.minimum(base + 8, 24)]
    pids = [30 + p for p in range(len(r_maxs))]
    _grouped_vs_single(f"straddle-{layout}-{max_tile_rows}", 24, pids, d_in, d_outs, S, ranks, r_maxs, seg_ptr,
                       seg_slot, max_tile_rows, 29)
