"""CPU: the decoder-layer reference the GPU layer step is checked against, and the power
of that check.  Dropping any one of the seven add-ons must move that projection's output
(and the layer output) far beyond the tolerance the GPU comparison uses, so a missing,
misrouted or mis-strided add-on on the GPU cannot pass."""
import numpy as np
import pytest

from tests import layer_ref as R

TOL = 5e-3   # relative Frobenius, per tensor (fp16 storage roundings of the backbone)


@pytest.fixture(scope="module")
def tiny():
    case = R.make_case("tiny")
    return case, R.reference(case)


def test_no_adapter_rows_match_the_backbone_alone(tiny):
    """With every add-on dropped the projections are the backbone's; rows with idx = -1 or
    a rank-0 slot give the same bits with and without add-ons in q/k/v and gate/up
    (their inputs do not depend on the add-ons)."""
    case, full = tiny
    none = R.reference(case, drop=R.PROJS)
    inact = (case["idx"] < 0) | (case["rank"][np.maximum(case["idx"], 0)] == 0)
    assert inact.any() and (~inact).any()
    for p in ("q", "k", "v"):
        assert np.array_equal(full[p][inact].view(np.uint16), none[p][inact].view(np.uint16)), p


@pytest.mark.parametrize("proj", R.PROJS)
def test_a_dropped_add_on_is_far_outside_the_tolerance(tiny, proj):
    case, full = tiny
    dropped = R.reference(case, drop=(proj,))
    assert R.rel_fro(dropped[proj], full[proj]) > 10 * TOL, proj
    if proj in ("k", "v"):      # reaches the output only through the cache's last position
        assert not np.array_equal(dropped["out"].view(np.uint16), full["out"].view(np.uint16)), proj
    else:
        assert R.rel_fro(dropped["out"], full["out"]) > TOL, proj
    for p in R.PROJS[:R.PROJS.index(proj)]:                 # earlier projections unchanged
        assert np.array_equal(dropped[p].view(np.uint16), full[p].view(np.uint16)), (proj, p)


def test_backbone_step_on_cpu_matches_reference(tiny):
    """The package's layer step with no add-ons (meta None), run by PyTorch on the CPU,
    against the reference with every add-on dropped: checks the backbone's slicing, cache
    writes and attention layout that the GPU comparison relies on."""
    import torch
    from segmented_gather_matmul_amd import layer as LY
    case, _ = tiny
    want = R.reference(case, drop=R.PROJS)
    h, f, H, dh, eps = case["dims"]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    layer = LY.LoraDecoderLayer(LY.LlamaShape("case", h, f, H, dh, eps), {k: t(v) for k, v in case["bb"].items()},
                                {p: (t(s.a_t), t(s.b)) for p, s in case["stores"].items()}, t(case["rank"]),
                                t(case["scale"]), max_rows=len(case["idx"]))
    trace = {}
    out = layer.forward(t(case["hidden"]), LY.KVCache(t(case["k_t"].copy()), t(case["v_cache"].copy())), None,
                        trace=trace)
    for p in R.PROJS + ("out",):
        got = (out if p == "out" else trace[p]).numpy()
        assert R.rel_fro(got, want[p]) <= TOL / 5, p
