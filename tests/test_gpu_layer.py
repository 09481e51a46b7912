"""GPU: the decoder-layer decode step (backbone in PyTorch, the seven add-ons through the
library, one metadata build shared by all of them) against the CPU layer reference, in
the per-row and the segment form, at a small shape with mixed ranks and rows without an
adapter and at the Llama-2-7B shape; and the step captured in a HIP graph, replayed with
eager work in between, against the eager step bit for bit."""
import functools

import numpy as np
import pytest

from tests import gpu_cases as G
from tests import layer_ref as R

pytestmark = pytest.mark.gpu
TOL = 5e-3   # relative Frobenius per tensor; a dropped add-on moves its tensor by > 10x this


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from segmented_gather_matmul_amd import binding as B
    B.lib()
    yield


@functools.lru_cache(maxsize=2)
def _case(name):
    G.say(f"case layer-{name}: drawing inputs and the CPU reference")
    case = R.make_case(name)
    return case, R.reference(case)


def _build(case, overlap=False):
    import torch
    from segmented_gather_matmul_amd import layer as LY
    h, f, H, dh, eps = case["dims"]
    shape = LY.LlamaShape("case", h, f, H, dh, eps)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bb = {k: dev(v) for k, v in case["bb"].items()}
    ads = {p: (dev(st.a_t), dev(st.b)) for p, st in case["stores"].items()}
    n = case["hidden"].shape[0]
    layer = LY.LoraDecoderLayer(shape, bb, ads, dev(case["rank"]), dev(case["scale"]), max_rows=n, overlap=overlap)
    return layer, LY.KVCache(dev(case["k_t"]), dev(case["v_cache"])), dev(case["hidden"])


@pytest.mark.parametrize("name", ["tiny", "7b"])
@pytest.mark.parametrize("form", ["bgmv", "sgmv"])
def test_layer_step_matches_reference(name, form):
    import torch
    from segmented_gather_matmul_amd import layer as LY
    case, want = _case(name)
    G.say(f"case layer-{name} form={form} n={case['hidden'].shape[0]} dims={case['dims'][:4]}")
    layer, cache, hidden = _build(case)
    meta = LY.BatchMeta(case["idx"], layer.num_slots, form)
    trace = {}
    out = layer.forward(hidden, cache, meta, trace=trace)
    base = {}
    layer.forward(hidden, LY.KVCache(cache.k_t.clone(), cache.v.clone()), None, trace=base)
    torch.cuda.synchronize()
    inact = (case["idx"] < 0) | (case["rank"][np.maximum(case["idx"], 0)] == 0)
    for p in R.PROJS + ("out",):
        got = (out if p == "out" else trace[p]).cpu().numpy()
        assert np.isfinite(got).all(), f"{p}: non-finite"
        rel = R.rel_fro(got, want[p])
        G.say(f"  {name}-{form} {p}: rel_F = {rel:.2e}")
        assert rel <= TOL, f"{p}: relative Frobenius {rel}"
    for p in ("q", "k", "v", "gate", "up"):     # inputs independent of earlier add-ons
        got, b = trace[p].cpu().numpy(), base[p].cpu().numpy()
        assert np.array_equal(got[inact].view(np.uint16), b[inact].view(np.uint16)), f"{p}: inactive row changed"
        assert not np.array_equal(got[~inact].view(np.uint16), b[~inact].view(np.uint16)), f"{p}: no add-on landed"
    # shrinks on a second stream, overlapping the backbone GEMMs: the same bits
    layer2, cache2, _ = _build(case, overlap=True)
    trace2 = {}
    out2 = layer2.forward(hidden, cache2, meta, trace=trace2)
    torch.cuda.synchronize()
    for p in R.PROJS:
        assert torch.equal(trace2[p], trace[p]), f"{p}: overlapped shrink changed the result"
    assert torch.equal(out2, out)


@pytest.mark.parametrize("form,overlap", [("bgmv", False), ("sgmv", False), ("bgmv", True), ("sgmv", True)])
def test_graph_replays_match_eager(form, overlap):
    import torch
    from segmented_gather_matmul_amd import layer as LY
    case, _ = _case("tiny")
    G.say(f"case layer-graph form={form} overlap={overlap}")
    layer, cache, hidden = _build(case, overlap)
    meta = LY.BatchMeta(case["idx"], layer.num_slots, form)
    other = LY.BatchMeta(case["idx"][::-1].copy(), layer.num_slots, "sgmv" if form == "bgmv" else "bgmv")
    eager = layer.forward(hidden, cache, meta).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward(hidden, cache, meta)
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.cpu().numpy().view(np.uint16)), \
            f"replay {i} differs from the eager step"
        layer.forward(hidden.flip(0).contiguous(), cache, other)   # eager work between replays
        torch.cuda.synchronize()
    del g
