"""GPU: batches served from an adapter cache over a paged pool.  Every batch's missing
adapters load on a side stream (evicting least recently used ones), the compute stream
waits on the cache's event, and each projection's y matches the fp64 oracle on the
batch's adapters.  Batches are queued without synchronizing in between, so loads that
reuse an evicted adapter's slot or pages must wait for the batches still reading them;
the next batch's adapters are prefetched while the current batch runs."""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from segmented_gather_matmul_amd.adapters import AdapterCache, HostAdapter, PagedModel
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
SHAPES = [(256, 128), (256, 64), (128, 256), (256, 64)]   # two layers x two projections
P, R_MAX, SLOTS, N = 64, 16, 4, 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield


def _store(model, n_adapters, seed):
    """Host adapters of ranks 4, 8 or 16, and their A^T / B per target for the oracle."""
    rng = np.random.default_rng(seed)
    store, host = {}, {}
    for a in range(n_adapters):
        r = int(rng.choice([4, 8, 16]))
        a_t = [(rng.standard_normal((r, di)) * 0.02).astype(np.float16) for di, _ in model.shapes]
        b = [(rng.standard_normal((r, do)) * 0.02).astype(np.float16) for _, do in model.shapes]
        store[f"ad{a}"] = HostAdapter(model, r, float(wl.scale_for_rank(np.array([r]))[0]), a_t, b)
        host[f"ad{a}"] = (a_t, b)
    return store, host


def _dense_view(model, store, host, cache, t):
    """The slots' adapters of target t as the oracle's dense store (empty slots: rank 0)."""
    di, do = model.shapes[t]
    rank = np.zeros(SLOTS, np.int32)
    scale = np.zeros(SLOTS, np.float32)
    a_t = np.full((SLOTS, R_MAX, di), np.nan, np.float16)
    b = np.full((SLOTS, R_MAX, do), np.nan, np.float16)
    for s, k in enumerate(cache.key_in):
        if k is None:
            continue
        ad = store[k]
        rank[s], scale[s] = ad.rank, np.float32(ad.scale)
        a_t[s, :ad.rank], b[s, :ad.rank] = host[k][0][t], host[k][1][t]
    return wl.DenseStore(num_slots=SLOTS, d_in=di, d_out=do, r_max=R_MAX, rank=rank, scale=scale, a_t=a_t, b=b)


def test_batches_through_the_cache():
    import torch
    # room for any 4 adapters, so slots (4) decide the evictions
    pages = SLOTS * sum(B.lora_pool_pages_for(R_MAX, di, do, P) for di, do in SHAPES)
    model = PagedModel(SHAPES, SLOTS, R_MAX, P, pages)
    store, host = _store(model, 7, 11)
    cache = AdapterCache(model, store)
    batches = [["ad0", "ad1", None, "ad0", "ad2", "ad3", "ad1", None],
               ["ad4", "ad0", "ad5", None, "ad4", "ad0", "ad5", "ad5"],
               ["ad6", "ad1", None, "ad6", "ad1", "ad4", "ad4", "ad0"],
               ["ad2", "ad3", "ad2", "ad3", None, None, "ad5", "ad6"]]
    cur = torch.cuda.current_stream()
    results = []
    G.say(f"case adapter-cache slots={SLOTS} pages={pages} batches={len(batches)}")
    slots, ready = cache.ensure(batches[0])
    for i, keys in enumerate(batches):
        if i > 0:
            slots, ready = cache.ensure(keys)          # resident already: prefetched below
        for e in ready:
            cur.wait_event(e)
        views = [_dense_view(model, store, host, cache, t) for t in range(len(SHAPES))]
        idx = torch.from_numpy(slots).cuda()
        outs = []
        for t, (w, (di, do)) in enumerate(zip(model.targets, SHAPES)):
            x, y0 = wl.activations(40 + i, t, N, di, do)
            xd = torch.from_numpy(x).cuda()
            yd = torch.from_numpy(y0).cuda()
            vd = torch.zeros((N, R_MAX), dtype=torch.float32, device="cuda")
            B.lora_bgmv(yd, xd, idx, w, vd)
            outs.append((x, y0, yd, views[t]))
        cache.mark_used(keys, cur)
        results.append((slots.copy(), outs))
        if i + 1 < len(batches):
            cache.prefetch(batches[i + 1])               # loads overlap this batch's kernels
    torch.cuda.synchronize()
    assert cache.loads >= 9                              # evictions happened
    for i, (slots, outs) in enumerate(results):
        for t, (x, y0, yd, view) in enumerate(outs):
            y_ref, _ = oracle.bgmv(view, x, y0, slots, nthreads=4)
            y = yd.cpu().numpy()
            act = slots >= 0
            err = np.abs(y.astype(np.float64) - y_ref)
            assert np.nanmax(err) <= 1e-2, f"batch {i} target {t}: max |dy| {np.nanmax(err)}"
            fro = np.sqrt(np.nansum((y.astype(np.float64) - y_ref) ** 2) / np.sum(y_ref ** 2))
            assert fro <= 1e-3, f"batch {i} target {t}: rel_F {fro}"
            assert np.array_equal(y[~act].view(np.uint16), y0[~act].view(np.uint16)), f"batch {i}: idle rows"
