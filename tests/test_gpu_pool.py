"""GPU: adapters placed into a paged pool by lora_pool_load (one copy, one kernel) land
bit for bit in their pages, page-table entries and slot fields, and the shrink/expand
kernels on that pool match the fp64 oracle on the same adapters; unloading and
reloading into freed pages keeps every other slot intact."""
import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import workloads as wl
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
CFG, D_IN, P, R_MAX, S = 31, 2048, 256, 64, 6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield


def _target(d_out, num_pages, rank_t, scale_t, pool):
    import torch
    cap = R_MAX * (D_IN // P + d_out // P)
    return B.Weights(num_slots=S, d_in=D_IN, d_out=d_out, r_max=R_MAX, rank=rank_t, scale=scale_t, pool=pool,
                     page_elems=P, page_table=torch.full((S * cap,), -1, dtype=torch.int32, device="cuda"),
                     a_pt_off=torch.zeros(S, dtype=torch.int64, device="cuda"),
                     b_pt_off=torch.zeros(S, dtype=torch.int64, device="cuda")), cap


def _fragmented_pool(num_pages, seed):
    st = B.PoolState(num_pages)
    every = st.alloc(num_pages)
    st.release(np.random.default_rng(seed).permutation(every))
    return st


def _adapter(w, cap, st, proj, slot, rank, d_out):
    a_t, b = wl.slot_matrices(CFG, proj, slot, rank, D_IN, d_out)
    return dict(w=w, slot=slot, rank=rank, scale=float(wl.scale_for_rank(rank)), pt_off=slot * cap, a_t=a_t, b=b,
                pages=st.alloc(B.lora_pool_pages_for(rank, D_IN, d_out, P)))


def _load(adapters):
    import torch
    blob, jobs = B.pack_adapters(adapters, pinned=True)
    staging = torch.empty(blob.numel(), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    B.lora_pool_load(jobs, blob, staging, stream=side)
    side.synchronize()
    return staging


def _check_placed(w, pool, ad, d_out):
    """Pages, page-table entries and slot fields of one loaded adapter, bitwise."""
    r, ids = ad["rank"], ad["pages"]
    per_a, per_b = D_IN // P, d_out // P
    got = pool[ids.astype(np.int64)].cpu().numpy().view(np.uint16)
    want = np.concatenate([ad["a_t"].reshape(r * per_a, P), ad["b"].reshape(r * per_b, P)]).view(np.uint16)
    assert np.array_equal(got, want), f"slot {ad['slot']}: page contents"
    pt = w.tensors[5].cpu().numpy()
    assert np.array_equal(pt[ad["pt_off"]:ad["pt_off"] + len(ids)], ids), f"slot {ad['slot']}: page table"
    s = ad["slot"]
    assert int(w.tensors[0][s]) == r and float(w.tensors[1][s]) == np.float32(ad["scale"])
    assert int(w.tensors[6][s]) == ad["pt_off"] and int(w.tensors[7][s]) == ad["pt_off"] + r * per_a


def _compute_and_check(w, rank, d_out, proj, label):
    """bgmv and sgmv on the loaded pool against the oracle on the same adapters."""
    import torch
    n = 100
    idx = np.random.default_rng(5).integers(-1, S, size=n).astype(np.int32)
    scale = wl.scale_for_rank(rank)
    store = wl.dense_store(CFG, proj, S, D_IN, d_out, rank, scale, r_max=R_MAX)
    x, y0 = wl.activations(CFG, proj, n, D_IN, d_out)
    y_ref, v_ref = oracle.bgmv(store, x, y0, idx, nthreads=16)
    for form in ("bgmv", "sgmv_rowmap"):
        dc = G.DeviceCase(x, y0, R_MAX)
        y, v = G.run_bgmv(w, dc, idx) if form == "bgmv" else G.run_sgmv(w, dc, idx=idx)
        G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), f"{label}-{form}")


def test_load_compute_unload_reload():
    import torch
    d_out = 1536
    rank = np.array([8, 16, 0, 64, 33, 1], dtype=np.int32)
    need = int(sum(B.lora_pool_pages_for(int(r), D_IN, d_out, P) for r in rank))
    num_pages = need + 300
    pool = torch.full((num_pages, P), float("nan"), dtype=torch.float16, device="cuda")
    rank_t = torch.zeros(S, dtype=torch.int32, device="cuda")
    scale_t = torch.zeros(S, dtype=torch.float32, device="cuda")
    w, cap = _target(d_out, num_pages, rank_t, scale_t, pool)
    st = _fragmented_pool(num_pages, 1)
    G.say(f"case pool-load {D_IN}->{d_out} P={P} pages={num_pages}")
    ads = [_adapter(w, cap, st, 0, s, int(r), d_out) for s, r in enumerate(rank) if r > 0]
    _load(ads)
    for ad in ads:
        _check_placed(w, pool, ad, d_out)
    assert int(rank_t[2]) == 0
    assert st.free == num_pages - need
    _compute_and_check(w, rank, d_out, 0, "pool")

    # unload slot 0, return its pages, load slot 2 (rank 8) into them
    G.say("case pool-unload-reload")
    gone = ads[0]
    _load([dict(w=w, slot=0, rank=0, scale=0.0)])
    st.release(gone["pages"])
    new = _adapter(w, cap, st, 0, 2, 8, d_out)
    assert sorted(new["pages"].tolist()) == sorted(gone["pages"].tolist())   # the freed pages, reused
    _load([new])
    _check_placed(w, pool, new, d_out)
    for ad in ads[1:]:
        _check_placed(w, pool, ad, d_out)                                       # the others untouched
    rank2 = rank.copy()
    rank2[0], rank2[2] = 0, 8
    _compute_and_check(w, rank2, d_out, 0, "pool-reloaded")


def test_one_call_two_projections_one_pool():
    """q-like and k-like targets sharing one pool and one rank/scale array."""
    import torch
    outs = (2048, 512)
    rank = np.array([16, 0, 32, 8, 64, 16], dtype=np.int32)
    need = sum(int(B.lora_pool_pages_for(int(r), D_IN, d, P)) for d in outs for r in rank)
    num_pages = need + 50
    pool = torch.full((num_pages, P), float("nan"), dtype=torch.float16, device="cuda")
    rank_t = torch.zeros(S, dtype=torch.int32, device="cuda")
    scale_t = torch.zeros(S, dtype=torch.float32, device="cuda")
    st = _fragmented_pool(num_pages, 2)
    targets = [_target(d, num_pages, rank_t, scale_t, pool) for d in outs]
    G.say(f"case pool-two-targets pages={num_pages}")
    ads = [_adapter(w, cap, st, p, s, int(r), d) for p, ((w, cap), d) in enumerate(zip(targets, outs))
           for s, r in enumerate(rank) if r > 0]
    _load(ads)
    assert st.free == num_pages - need
    for ad in ads:
        _check_placed(ad["w"], pool, ad, ad["b"].shape[1])
    for p, ((w, _), d) in enumerate(zip(targets, outs)):
        _compute_and_check(w, rank, d, p, f"pool-proj{p}")


@pytest.mark.parametrize("page_elems,d_in,d_out", [(56, 1288, 1064), (4096, 4096, 8192), (8, 64, 24)])
def test_page_sizes(page_elems, d_in, d_out):
    """Pages copied by 7 lanes (56 elements), by a whole workgroup in a loop (4096), and
    by one lane each (8); every placed adapter checked bitwise and through the kernels."""
    import torch
    rank = np.array([3, 0, 17, 64, 1, 8], dtype=np.int32)
    cap = R_MAX * (d_in // page_elems + d_out // page_elems)
    need = int(sum(B.lora_pool_pages_for(int(r), d_in, d_out, page_elems) for r in rank))
    num_pages = need + 7
    pool = torch.full((num_pages, page_elems), float("nan"), dtype=torch.float16, device="cuda")
    w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=R_MAX,
                  rank=torch.zeros(S, dtype=torch.int32, device="cuda"),
                  scale=torch.zeros(S, dtype=torch.float32, device="cuda"), pool=pool, page_elems=page_elems,
                  page_table=torch.full((S * cap,), -1, dtype=torch.int32, device="cuda"),
                  a_pt_off=torch.zeros(S, dtype=torch.int64, device="cuda"),
                  b_pt_off=torch.zeros(S, dtype=torch.int64, device="cuda"))
    st = _fragmented_pool(num_pages, page_elems)
    G.say(f"case pool-pages P={page_elems} {d_in}->{d_out}")
    ads = []
    for s, r in enumerate(rank):
        if r == 0:
            continue
        a_t, b = wl.slot_matrices(CFG, 9, s, int(r), d_in, d_out)
        ads.append(dict(w=w, slot=s, rank=int(r), scale=float(wl.scale_for_rank(int(r))), pt_off=s * cap, a_t=a_t,
                        b=b, pages=st.alloc(B.lora_pool_pages_for(int(r), d_in, d_out, page_elems))))
    _load(ads)
    for ad in ads:
        r, ids = ad["rank"], ad["pages"]
        got = pool[ids.astype(np.int64)].cpu().numpy().view(np.uint16)
        want = np.concatenate([ad["a_t"].reshape(-1, page_elems), ad["b"].reshape(-1, page_elems)]).view(np.uint16)
        assert np.array_equal(got, want), f"slot {ad['slot']}: page contents"
    n = 60
    idx = np.random.default_rng(page_elems).integers(-1, S, size=n).astype(np.int32)
    store = wl.dense_store(CFG, 9, S, d_in, d_out, rank, wl.scale_for_rank(rank), r_max=R_MAX)
    x, y0 = wl.activations(CFG, 9, n, d_in, d_out)
    y_ref, v_ref = oracle.bgmv(store, x, y0, idx, nthreads=16)
    dc = G.DeviceCase(x, y0, R_MAX)
    y, v = G.run_bgmv(w, dc, idx)
    G.check(dc, y, v, y_ref, v_ref, G.active_rows(idx, rank), f"pool-pages-{page_elems}")


def _pack_data_first(adapters):
    """A blob with each job's rank-rows before its page ids (valid for lora_pool_load, but
    not the direct route's layout, so it takes the staged route)."""
    import ctypes
    import torch
    n = len(adapters)
    off = int(B.lib().lora_pool_load_header_bytes(n))
    jobs = (B.CLoadJob * n)()
    parts = []
    for i, ad in enumerate(adapters):
        j = jobs[i]
        j.w = ctypes.addressof(ad["w"].c)
        j.slot, j.rank, j.scale, j.reserved = int(ad["slot"]), int(ad["rank"]), float(ad["scale"]), 0
        j.pt_off = int(ad["pt_off"])
        data = np.concatenate([ad["a_t"].ravel(), ad["b"].ravel()]).astype(np.float16).view(np.uint8)
        j.data_off = off
        parts.append((off, data))
        off = -(-(off + len(data)) // 16) * 16
        j.pages_off = off
        ids = np.ascontiguousarray(ad["pages"], np.int32).view(np.uint8)
        parts.append((off, ids))
        off = -(-(off + len(ids)) // 16) * 16
    blob = torch.zeros(off, dtype=torch.uint8, pin_memory=True)
    view = blob.numpy()
    for o, d in parts:
        view[o:o + len(d)] = d
    return blob, jobs


@pytest.mark.parametrize("layout", ["fresh", "runs", "data_first"])
def test_direct_and_staged_routes(layout):
    """fresh: a new free list hands out consecutive pages, so the call's rank-rows are one
    run per pool (the direct route: copies straight into the pool); runs: pages released
    as three ascending ranges, the middle one handed out first, come back as three runs
    (direct); data_first: the same pages
    from a blob whose rank-rows precede the page ids (the staged route).  Every placement
    checked bitwise and through the kernels."""
    import torch
    outs = (2048, 512)
    rank = np.array([16, 0, 32, 8, 64, 16], dtype=np.int32)
    need = sum(int(B.lora_pool_pages_for(int(r), D_IN, d, P)) for d in outs for r in rank)
    num_pages = need + 40
    pool = torch.full((num_pages, P), float("nan"), dtype=torch.float16, device="cuda")
    rank_t = torch.zeros(S, dtype=torch.int32, device="cuda")
    scale_t = torch.zeros(S, dtype=torch.float32, device="cuda")
    st = B.PoolState(num_pages)
    if layout == "runs":
        taken = st.alloc(num_pages)                     # 0 .. num_pages-1
        third = num_pages // 3
        st.release(taken[2 * third:])                   # handed out last
        st.release(taken[:third])
        st.release(taken[third:2 * third])              # handed out first
    targets = [_target(d, num_pages, rank_t, scale_t, pool) for d in outs]
    G.say(f"case pool-route-{layout} pages={num_pages}")
    ads = [_adapter(w, cap, st, p, s, int(r), d) for p, ((w, cap), d) in enumerate(zip(targets, outs))
           for s, r in enumerate(rank) if r > 0]
    ids = np.concatenate([ad["pages"] for ad in ads])
    breaks = int(np.count_nonzero(np.diff(ids) != 1))
    assert breaks == (0 if layout != "runs" else 2), breaks   # the runs the direct route copies
    if layout == "data_first":
        blob, jobs = _pack_data_first(ads)
        staging = torch.empty(blob.numel(), dtype=torch.uint8, device="cuda")
        B.lora_pool_load(jobs, blob, staging)
        torch.cuda.synchronize()
    else:
        _load(ads)
    for ad in ads:
        _check_placed(ad["w"], pool, ad, ad["b"].shape[1])
    for p, ((w, _), d) in enumerate(zip(targets, outs)):
        _compute_and_check(w, rank, d, p, f"pool-route-{layout}-proj{p}")
