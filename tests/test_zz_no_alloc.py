"""GPU: the allocation-free hand-off entry point (lora_bgmv_multi_handoff_noalloc, for
callers that cannot allocate) against lora_bgmv_multi_handoff with a caller workspace,
bit for bit on whole buffers (guard rows and padding included), and against the fp64
oracle within the stated tolerance.  Two calls in a row, the second with fewer rows, so
the second finds the library's scratch as the first left it; then a captured graph of
the call replayed between eager calls."""
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


def _case(n, d_in, outs, rank, idx, key):
    S = len(rank)
    stores = [wl.dense_store(31, key + p, S, d_in, d_out, rank, wl.scale_for_rank(rank), r_max=int(rank.max()))
              for p, d_out in enumerate(outs)]
    x, _ = wl.activations(31, key, n, d_in, 8)
    y0s = [wl.activations(31, key + p, n, d_in, d_out)[1] for p, d_out in enumerate(outs)]
    return stores, x, y0s


def _run(stores, x, y0s, idx, noalloc, work=None):
    import torch
    ws = [B.weights_from_store(s) for s in stores]
    dcs = [G.DeviceCase(x, y0, s.r_max) for s, y0 in zip(stores, y0s)]
    items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    if noalloc:
        B.lora_bgmv_multi_handoff_noalloc(dcs[0].x, idx_d, items)
    else:
        B.lora_bgmv_multi_handoff(dcs[0].x, idx_d, items, work)
    return dcs, [dc.results() for dc in dcs]


def test_noalloc_equals_workspace_form_on_two_calls_second_smaller():
    cases = []
    # 1: a 7B decode q/k/v unit, 32 rows each with its own rank-16 adapter
    cases.append((32, 4096, (4096, 4096, 4096), np.full(32, 16, np.int32), np.arange(32, dtype=np.int32), 0))
    # 2: fewer rows, mixed ranks (one 0), rows without adapter, ragged widths
    rank = np.array([16, 64, 0, 8, 33], np.int32)
    cases.append((7, 1288, (1064, 520), rank, np.array([1, -1, 0, 2, 4, 1, 3], np.int32), 10))
    work = B.handoff_workspace(64)
    for n, d_in, outs, rank, idx, key in cases:
        G.say(f"case noalloc n={n} {d_in}->{'/'.join(map(str, outs))}")
        stores, x, y0s = _case(n, d_in, outs, rank, idx, key)
        _, ref = _run(stores, x, y0s, idx, False, work)
        dcs, got = _run(stores, x, y0s, idx, True)
        act = G.active_rows(idx, rank)
        for p in range(len(outs)):
            assert np.array_equal(ref[p][0].view(np.uint16), got[p][0].view(np.uint16)), f"n={n} p={p}: y"
            assert np.array_equal(ref[p][1].view(np.uint32), got[p][1].view(np.uint32)), f"n={n} p={p}: v"
            y_ref, v_ref = oracle.bgmv(stores[p], x, y0s[p], idx, nthreads=16)
            G.check(dcs[p], *got[p], y_ref, v_ref, act, f"noalloc-n{n}-p{p}")
        assert int(work.count_nonzero()) == 0


def test_noalloc_in_a_captured_graph_replayed_between_eager_calls():
    import torch
    n, d_in, outs = 16, 2048, (2048, 1024)
    rank = np.array([16, 8, 32, 0, 16, 24], np.int32)
    idx = np.array([0, 1, 2, 3, -1, 5, 4, 0, 2, 2, 1, 5, 4, 3, 0, 1], np.int32)
    stores, x, y0s = _case(n, d_in, outs, rank, idx, 20)
    ws = [B.weights_from_store(s) for s in stores]
    dcs = [G.DeviceCase(x, y0, s.r_max) for s, y0 in zip(stores, y0s)]
    items = [(w, dc.v, dc.y) for w, dc in zip(ws, dcs)]
    idx_d = torch.from_numpy(idx).cuda()
    call = lambda: B.lora_bgmv_multi_handoff_noalloc(dcs[0].x, idx_d, items)
    call()
    eager = [dc.results() for dc in dcs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    other = _case(9, 1288, (1064,), rank, idx[:9], 30)
    for rep in range(3):
        _run(*other, idx[:9], True)                     # an eager call on other inputs in between
        for dc in dcs:
            dc.reset()
        torch.cuda.synchronize()
        g.replay()
        got = [dc.results() for dc in dcs]
        for p in range(len(outs)):
            assert np.array_equal(eager[p][0].view(np.uint16), got[p][0].view(np.uint16)), f"replay {rep} p={p}: y"
            assert np.array_equal(eager[p][1].view(np.uint32), got[p][1].view(np.uint32)), f"replay {rep} p={p}: v"
