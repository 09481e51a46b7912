"""The C-ABI library on the CPU: exports, host metadata, and every host-checked error path.

No test here launches a kernel: every call either is host-only (metadata builders,
validators) or is rejected by the host checks before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from segmented_gather_matmul_amd import workloads as wl
from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd import build as build_mod

HEADER = os.path.join(build_mod.INCLUDE, "lora_sgmv.h")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if build_mod.stale():
        build_mod.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 37 and set(names) == set(B.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", build_mod.LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (lora_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(B.lib(), n)
    assert B.lib().lora_abi_version() == 2


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert B.status_str(code) and B.status_str(code) != "unknown status"
    assert B.status_str(-99) == "unknown status"


# ------------------------------------------------------------------ metadata builder
def _random_idx(rng):
    S = int(rng.integers(1, 3000))
    n = int(rng.integers(0, 600))
    mode = rng.integers(0, 4)
    if mode == 0:
        idx = rng.integers(-1, S, size=n)
    elif mode == 1:
        idx = np.full(n, int(rng.integers(-1, S)))
    elif mode == 2:
        idx = rng.choice(np.arange(min(S, 5)), size=n) - 1
    else:
        idx = rng.permutation(max(n, 1))[:n] % S
    return idx.astype(np.int32), S


def test_build_segments_bit_exact_vs_python_reference():
    rng = np.random.default_rng(2024)
    for _ in range(200):
        idx, S = _random_idx(rng)
        got = B.lora_build_segments(idx, S)
        want = oracle.build_segments(idx, S)
        for g, w in zip(got[:3], want[:3]):
            assert g.dtype == np.int32 and np.array_equal(g, w)
        assert got[3] == want[3]


def test_build_segments_edge_cases():
    rm, sp, ss, na = B.lora_build_segments(np.zeros(0, np.int32), 4)
    assert na == 0 and sp.tolist() == [0] and len(ss) == 0
    rm, sp, ss, na = B.lora_build_segments(np.full(5, -1, np.int32), 4)
    assert na == 0 and sp.tolist() == [0]
    rm, sp, ss, na = B.lora_build_segments(np.array([3, 3, 0, 3], np.int32), 4)
    assert rm.tolist() == [2, 0, 1, 3] and sp.tolist() == [0, 1, 4] and ss.tolist() == [0, 3]


def test_build_segments_rejects_bad_slots():
    for bad in ([0, 4], [-2, 0]):
        with pytest.raises(B.LoraError) as e:
            B.lora_build_segments(np.array(bad, np.int32), 4)
        assert e.value.code == B.LORA_E_INDEX
    with pytest.raises(B.LoraError) as e:
        B.lora_build_segments(np.array([0], np.int32), 0)
    assert e.value.code == B.LORA_E_SHAPE


def test_build_tiles_valid_and_balanced():
    rng = np.random.default_rng(7)
    for _ in range(100):
        n_seg = int(rng.integers(0, 40))
        lens = rng.integers(0, 300, size=n_seg)
        start = int(rng.integers(0, 5))
        seg_ptr = np.concatenate([[start], start + np.cumsum(lens)]).astype(np.int32)
        seg_slot = rng.integers(-1, 50, size=n_seg).astype(np.int32)
        mtr = int(rng.choice([1, 7, 16, 64]))
        tiles = B.lora_build_tiles(seg_ptr, seg_slot, mtr)
        nprob, msgs = oracle.check_tiles(tiles, seg_ptr, seg_slot, mtr)
        assert nprob == 0, msgs[:5]
        assert len(tiles) <= B.lora_tiles_bound(int(lens.sum()), n_seg, mtr)
        for g in range(n_seg):                               # near-equal cut of each segment
            sizes = tiles[tiles[:, 3] == g][:, 2]
            if len(sizes):
                assert sizes.max() - sizes.min() <= 1 and len(sizes) == -(-lens[g] // mtr)


def test_build_tiles_errors():
    seg_ptr = np.array([0, 5, 3], np.int32)
    with pytest.raises(B.LoraError) as e:
        B.lora_build_tiles(seg_ptr, np.array([0, 1], np.int32), 4)
    assert e.value.code == B.LORA_E_SHAPE
    with pytest.raises(B.LoraError) as e:
        B.lora_build_tiles(np.array([0, 5], np.int32), np.array([0], np.int32), 65)
    assert e.value.code == B.LORA_E_SHAPE
    tiles = np.zeros((1, 4), np.int32)
    n = ctypes.c_int32()
    st = B.lib().lora_build_tiles(np.array([0, 100], np.int32).ctypes.data, np.array([0], np.int32).ctypes.data,
                                  1, 8, tiles.ctypes.data, 1, ctypes.byref(n))
    assert st == B.LORA_E_CAPACITY


# ------------------------------------------------------------------ launch-time host checks
FAKE = 0x7f0000000000  # 16-byte aligned stand-in for a device address; never dereferenced


def _desc(**kw):
    c = B.CWeights()
    c.layout, c.num_slots, c.d_in, c.d_out, c.r_max = 0, 4, 1024, 1024, 16
    c.rank = c.scale = c.a_t = c.b = FAKE
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _shrink(c, v=FAKE, ldv=16, x=FAKE, ldx=1024, n=8, idx=FAKE):
    return B.lib().lora_bgmv_shrink(None, v, ldv, x, ldx, idx, n, ctypes.byref(c))


def test_launch_argument_errors():
    L = B.lib()
    assert _shrink(_desc(rank=None)) == B.LORA_E_NULL
    assert _shrink(_desc(), x=None) == B.LORA_E_NULL
    assert _shrink(_desc(), idx=None) == B.LORA_E_NULL
    assert _shrink(_desc(d_in=1020)) == B.LORA_E_SHAPE
    assert _shrink(_desc(num_slots=0)) == B.LORA_E_SHAPE
    assert _shrink(_desc(r_max=0)) == B.LORA_E_SHAPE
    assert _shrink(_desc(r_max=65), ldv=68) == B.LORA_E_UNSUPPORTED
    assert _shrink(_desc(layout=3)) == B.LORA_E_SHAPE
    assert _shrink(_desc(a_t=FAKE + 2)) == B.LORA_E_ALIGN
    assert _shrink(_desc(), x=FAKE + 8) == B.LORA_E_ALIGN
    assert _shrink(_desc(), ldx=1028) == B.LORA_E_ALIGN
    assert _shrink(_desc(), ldx=512) == B.LORA_E_SHAPE
    assert "leading dimension" in B.last_error()
    assert _shrink(_desc(), ldv=8) == B.LORA_E_SHAPE
    assert _shrink(_desc(), ldv=18) == B.LORA_E_ALIGN
    assert _shrink(_desc(), n=-1) == B.LORA_E_SHAPE
    assert "n_rows" in B.last_error()
    # zero rows is a no-op that launches nothing
    assert _shrink(_desc(), n=0) == B.LORA_OK
    c = _desc()
    assert L.lora_bgmv_expand(None, FAKE, 1000, FAKE, 16, FAKE, 8, ctypes.byref(c)) == B.LORA_E_SHAPE
    assert L.lora_bgmv_expand(None, FAKE + 2, 1024, FAKE, 16, FAKE, 8, ctypes.byref(c)) == B.LORA_E_ALIGN
    assert L.lora_bgmv(None, None, 1024, FAKE, 1024, FAKE, 8, ctypes.byref(c), FAKE, 16) == B.LORA_E_NULL
    assert L.lora_bgmv(None, FAKE, 1024, FAKE, 1024, FAKE, 8, ctypes.byref(c), FAKE, 12) == B.LORA_E_SHAPE


def test_paged_descriptor_errors():
    kw = dict(layout=1, a_t=None, b=None, pool=FAKE, page_table=FAKE, a_pt_off=FAKE, b_pt_off=FAKE,
              num_pages=10, pt_entries=10)
    assert _shrink(_desc(**kw, page_elems=1000)) == B.LORA_E_SHAPE   # does not divide 1024
    assert _shrink(_desc(**kw, page_elems=4)) == B.LORA_E_SHAPE      # not a multiple of 8
    assert _shrink(_desc(**dict(kw, pool=None), page_elems=256)) == B.LORA_E_NULL
    assert _shrink(_desc(**dict(kw, num_pages=0), page_elems=256)) == B.LORA_E_SHAPE


def test_segment_descriptor_errors():
    L = B.lib()
    c = _desc()
    s = B.CSegments()
    s.n_tiles, s.tiles, s.row_map, s.n_pos, s.max_rows = 3, None, None, 0, 0
    assert L.lora_sgmv_shrink(None, FAKE, 16, FAKE, 1024, 8, ctypes.byref(c), ctypes.byref(s)) == B.LORA_E_NULL
    s.tiles = FAKE + 4
    assert L.lora_sgmv_expand(None, FAKE, 1024, FAKE, 16, 8, ctypes.byref(c), ctypes.byref(s)) == B.LORA_E_ALIGN
    assert L.lora_sgmv_shrink(None, FAKE, 16, FAKE, 1024, 8, ctypes.byref(c), None) == B.LORA_E_NULL
    s.tiles, s.max_rows = FAKE, 65
    assert L.lora_sgmv_shrink(None, FAKE, 16, FAKE, 1024, 8, ctypes.byref(c), ctypes.byref(s)) == B.LORA_E_SHAPE


# ------------------------------------------------------------------ host validators
def _host_weights(rank, layout=0, **kw):
    keep = {}
    c = _desc(layout=layout, num_slots=len(rank), r_max=16)
    keep["rank"] = np.ascontiguousarray(rank, np.int32)
    c.rank = keep["rank"].ctypes.data
    for k, v in kw.items():
        if isinstance(v, np.ndarray):
            keep[k] = v
            setattr(c, k, v.ctypes.data)
        else:
            setattr(c, k, v)
    return c, keep


def test_validate_weights_host():
    c, keep = _host_weights([16, 0, 8])
    assert B.lib().lora_validate_weights_host(ctypes.byref(c)) == B.LORA_OK
    c, keep = _host_weights([16, 17, 8])
    assert B.lib().lora_validate_weights_host(ctypes.byref(c)) == B.LORA_E_SHAPE
    P = 256
    pa = pb = 1024 // P
    rank = np.array([2, 1], np.int32)
    entries = int(rank.sum() * (pa + pb))
    pt = np.arange(entries, dtype=np.int32)
    a_off = np.array([0, 2 * (pa + pb)], np.int64)
    b_off = a_off + rank * pa
    kw = dict(a_t=None, b=None, pool=FAKE, page_elems=P, num_pages=entries, pt_entries=entries,
              page_table=pt, a_pt_off=a_off, b_pt_off=b_off.astype(np.int64))
    c, keep = _host_weights(rank, layout=1, **kw)
    assert B.lib().lora_validate_weights_host(ctypes.byref(c)) == B.LORA_OK
    bad = pt.copy()
    bad[3] = entries
    c, keep = _host_weights(rank, layout=1, **dict(kw, page_table=bad))
    assert B.lib().lora_validate_weights_host(ctypes.byref(c)) == B.LORA_E_INDEX
    c, keep = _host_weights(rank, layout=1, **dict(kw, pt_entries=entries - 1))
    assert B.lib().lora_validate_weights_host(ctypes.byref(c)) == B.LORA_E_INDEX


def test_validate_segments_host():
    idx = np.array([2, -1, 0, 2, 2, 1], np.int32)
    row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(idx, 3)
    tiles = B.lora_build_tiles(seg_ptr, seg_slot, 2)
    s = B.CSegments()
    s.n_tiles, s.tiles, s.row_map, s.n_pos = len(tiles), tiles.ctypes.data, row_map.ctypes.data, n_act
    s.max_rows = int(tiles[:, 2].max())
    assert B.lib().lora_validate_segments_host(ctypes.byref(s), 6, 3) == B.LORA_OK
    assert B.lib().lora_validate_segments_host(ctypes.byref(s), 6, 2) == B.LORA_E_INDEX   # slot 2 >= 2
    dup = row_map.copy()
    dup[1] = dup[0]
    s.row_map = dup.ctypes.data
    assert B.lib().lora_validate_segments_host(ctypes.byref(s), 6, 3) == B.LORA_E_INDEX
    s.row_map = row_map.ctypes.data
    over = tiles.copy()
    over[0, 2] = 65
    s.tiles = over.ctypes.data
    assert B.lib().lora_validate_segments_host(ctypes.byref(s), 6, 3) == B.LORA_E_SHAPE


def test_multi_projection_errors():
    L = B.lib()
    c1, c2 = _desc(), _desc(d_in=2048)
    arr = (B.CProj * 5)()
    for i in range(5):
        arr[i].w, arr[i].v, arr[i].ldv, arr[i].y, arr[i].ldy = ctypes.addressof(c1), FAKE, 16, FAKE, 1024
    assert L.lora_bgmv_shrink_multi(None, FAKE, 1024, FAKE, 8, 0, arr) == B.LORA_E_SHAPE
    assert L.lora_bgmv_shrink_multi(None, FAKE, 1024, FAKE, 8, 5, arr) == B.LORA_E_SHAPE
    assert L.lora_bgmv_shrink_multi(None, FAKE, 1024, FAKE, 8, 2, None) == B.LORA_E_NULL
    arr[1].w = ctypes.addressof(c2)
    assert L.lora_bgmv_shrink_multi(None, FAKE, 1024, FAKE, 8, 2, arr) == B.LORA_E_SHAPE     # d_in differs
    assert "share x" in B.last_error()
    c3 = _desc(layout=1, a_t=None, b=None, pool=FAKE, page_table=FAKE, a_pt_off=FAKE, b_pt_off=FAKE,
               num_pages=10, pt_entries=10, page_elems=256)
    arr[1].w = ctypes.addressof(c3)
    assert L.lora_bgmv_expand_multi(None, FAKE, 8, 2, arr) == B.LORA_E_UNSUPPORTED         # mixed layouts
    arr[1].w = ctypes.addressof(c1)
    arr[1].ldy = 1000
    assert L.lora_bgmv_expand_multi(None, FAKE, 8, 2, arr) == B.LORA_E_SHAPE
    arr[1].ldy = 1024
    assert L.lora_bgmv_expand_multi(None, FAKE, 0, 2, arr) == B.LORA_OK                     # no rows: no launch


def test_two_step_decode_errors():
    """lora_bgmv_multi checks what both steps need before launching anything."""
    L = B.lib()
    c1, c2 = _desc(), _desc(d_in=2048)
    arr = (B.CProj * 2)()
    for i in range(2):
        arr[i].w, arr[i].v, arr[i].ldv, arr[i].y, arr[i].ldy = ctypes.addressof(c1), FAKE, 16, FAKE, 1024
    call = lambda x=FAKE, ldx=1024, idx=FAKE, n=8, n_proj=2, a=arr: L.lora_bgmv_multi(None, x, ldx, idx, n, n_proj, a)
    assert call(idx=None) == B.LORA_E_NULL
    assert call(n_proj=0) == B.LORA_E_SHAPE
    assert call(a=None) == B.LORA_E_NULL
    assert call(n=-1) == B.LORA_E_SHAPE
    assert call(x=None) == B.LORA_E_NULL
    assert call(x=FAKE + 8) == B.LORA_E_ALIGN
    assert call(ldx=1000) == B.LORA_E_SHAPE
    arr[1].ldy = 1000                                   # y checked even though x is fine
    assert call() == B.LORA_E_SHAPE and "y" in B.last_error()
    arr[1].ldy = 1024
    arr[1].ldv = 12                                     # v leading dimension < r_max
    assert call() == B.LORA_E_SHAPE
    arr[1].ldv = 16
    arr[1].w = ctypes.addressof(c2)
    assert call() == B.LORA_E_SHAPE and "share x" in B.last_error()
    arr[1].w = ctypes.addressof(c1)
    assert call(n=0) == B.LORA_OK


def test_handoff_decode_errors():
    """lora_bgmv_multi_handoff checks lora_bgmv_multi's arguments, then the workspace,
    before launching anything."""
    L = B.lib()
    assert L.lora_handoff_bytes(0) == 0 and L.lora_handoff_bytes(-3) == 0
    assert L.lora_handoff_bytes(1) == 4 * 128 * 4 and L.lora_handoff_bytes(1000) == 1000 * 2048
    c1 = _desc()
    arr = (B.CProj * 2)()
    for i in range(2):
        arr[i].w, arr[i].v, arr[i].ldv, arr[i].y, arr[i].ldy = ctypes.addressof(c1), FAKE, 16, FAKE, 1024
    need = L.lora_handoff_bytes(8)
    call = lambda x=FAKE, idx=FAKE, n=8, n_proj=2, a=arr, work=FAKE, nbytes=need: \
        L.lora_bgmv_multi_handoff(None, x, 1024, idx, n, n_proj, a, work, nbytes)
    assert call(idx=None) == B.LORA_E_NULL
    assert call(n_proj=5) == B.LORA_E_SHAPE
    assert call(x=FAKE + 8) == B.LORA_E_ALIGN
    assert call(n=-1) == B.LORA_E_SHAPE
    assert call(work=None) == B.LORA_E_NULL and "workspace" in B.last_error()
    assert call(work=FAKE + 16) == B.LORA_E_ALIGN and "workspace" in B.last_error()
    assert call(nbytes=need - 1) == B.LORA_E_SHAPE and "workspace" in B.last_error()
    wide = _desc(d_out=65536 * 512)
    arr[1].w, arr[1].ldy = ctypes.addressof(wide), 65536 * 512
    assert call() == B.LORA_E_SHAPE and "too wide" in B.last_error()
    assert call(n=0, work=None, nbytes=0) == B.LORA_OK                 # no rows: nothing is read or launched
    assert L.lora_set_handoff_polls(0) == B.LORA_OK and L.lora_set_handoff_polls(-1) == B.LORA_OK
    # the segment form: its own segment checks, then the same workspace checks
    arr[1].w, arr[1].ldy = ctypes.addressof(c1), 1024
    seg = B.CSegments()
    seg.n_tiles, seg.tiles, seg.row_map, seg.n_pos, seg.max_rows = 4, FAKE, FAKE, 8, 2
    scall = lambda s_=seg, n=8, work=FAKE, nbytes=need: \
        L.lora_sgmv_multi_handoff(None, FAKE, 1024, n, ctypes.byref(s_) if s_ is not None else None, 2, arr, work,
                                  nbytes)
    assert scall(s_=None) == B.LORA_E_NULL
    assert scall(work=None) == B.LORA_E_NULL and "workspace" in B.last_error()
    assert scall(work=FAKE + 64) == B.LORA_E_ALIGN
    assert scall(nbytes=need - 4) == B.LORA_E_SHAPE
    seg.max_rows = 16                                                   # MFMA tiles: two launches, same checks
    assert scall(work=None) == B.LORA_E_NULL
    seg.max_rows = 65
    assert scall() == B.LORA_E_SHAPE
    seg.max_rows = 2
    assert scall(n=0, work=None) == B.LORA_OK


def test_set_plan_ranges():
    L = B.lib()
    assert L.lora_set_plan(-1, 0) == B.LORA_E_SHAPE
    assert L.lora_set_plan(65, 0) == B.LORA_E_SHAPE
    assert L.lora_set_plan(0, 3) == B.LORA_E_SHAPE
    assert L.lora_set_plan(0, -1) == B.LORA_E_SHAPE
    assert L.lora_set_plan(64, 4) == B.LORA_OK
    assert L.lora_set_plan(0, 0) == B.LORA_OK


def test_set_stream_weights_values():
    L = B.lib()
    assert L.lora_set_stream_weights(2) == B.LORA_E_SHAPE
    assert L.lora_set_stream_weights(-1) == B.LORA_E_SHAPE
    assert L.lora_set_stream_weights(1) == B.LORA_OK
    assert L.lora_set_stream_weights(0) == B.LORA_OK


def test_pick_tile_rows():
    assert B.lora_pick_tile_rows(np.array([0, 1, 4, 6, 8], np.int32)) == 2      # short segments
    assert B.lora_pick_tile_rows(np.array([0, 4, 9, 13, 16], np.int32)) == 2
    assert B.lora_pick_tile_rows(np.array([0, 4, 4, 8], np.int32)) == 2         # empty segment
    assert B.lora_pick_tile_rows(np.array([0, 127, 140], np.int32)) == 2        # longest 127 rows
    assert B.lora_pick_tile_rows(np.array([0, 5, 133], np.int32)) == 64         # one of 128 or more
    assert B.lora_pick_tile_rows(np.array([0, 128], np.int32)) == 64
    assert B.lora_pick_tile_rows(np.array([0], np.int32)) == 2                  # no segments


def test_pick_expand_tile_rows():
    """16-row expand tiles for decode batches whose 16-row tiles average >= 6 rows; else
    the general choice (2 for short segments, 64 for long ones)."""
    seg = wl.segments_from_lengths
    assert B.lora_pick_expand_tile_rows(seg([58])) == 16                        # identical mix
    assert B.lora_pick_expand_tile_rows(seg([30, 11, 9, 5, 1, 1, 1])) == 16     # skewed mix: 58 rows, 8 tiles
    assert B.lora_pick_expand_tile_rows(seg([6, 5, 5, 5, 4, 4, 4, 4, 3, 3, 3, 3, 2, 2, 1])) == 2  # uniform
    assert B.lora_pick_expand_tile_rows(seg([58, 31, 14, 11, 10, 8] + [1] * 92)) == 2   # paged pool mix
    assert B.lora_pick_expand_tile_rows(seg([7, 7, 7])) == 2                    # no tile reaches 8 rows
    assert B.lora_pick_expand_tile_rows(seg([5, 6, 1])) == 2                    # 12 rows in 3 tiles
    assert B.lora_pick_expand_tile_rows(seg([0, 12, 0])) == 16                  # empty segments ignored
    assert B.lora_pick_expand_tile_rows(seg([5, 200])) == 64                    # prefill: long segments
    assert B.lora_pick_expand_tile_rows(np.array([0], np.int32)) == 2           # no segments
    assert B.lora_pick_expand_tile_rows(np.array([0, 9], np.int32)) == 16


# ------------------------------------------------------------------ offsets form of the segment descriptor
def _offsets(seg_ptr, seg_slot, row_map=None, tile_rows=0):
    keep = [np.ascontiguousarray(seg_ptr, np.int32), np.ascontiguousarray(seg_slot, np.int32)]
    s = B.CSegments()
    s.n_seg, s.seg_ptr, s.seg_slot = len(keep[1]), keep[0].ctypes.data, keep[1].ctypes.data
    if row_map is not None:
        keep.append(np.ascontiguousarray(row_map, np.int32))
        s.row_map = keep[-1].ctypes.data
    s.tile_rows = tile_rows
    return s, keep


def test_offsets_descriptor_host_checks():
    """The pages' form (Punica digest, section 5.4: the SGMV call takes the segment offsets
    s with s[0] = 0 and s[-1] = the batch, and one adapter index per segment)."""
    L = B.lib()
    ok, keep = _offsets([0, 1, 4, 6, 8], [0, 1, 2, 3])
    assert L.lora_validate_segments_host(ctypes.byref(ok), 8, 4) == B.LORA_OK
    assert L.lora_validate_segments_host(ctypes.byref(ok), 7, 4) == B.LORA_E_INDEX     # s[-1] > rows
    assert L.lora_validate_segments_host(ctypes.byref(ok), 8, 3) == B.LORA_E_INDEX     # slot 3 >= 3
    dec, keep2 = _offsets([0, 4, 1, 8], [0, 1, 2])
    assert L.lora_validate_segments_host(ctypes.byref(dec), 8, 4) == B.LORA_E_SHAPE    # decreasing
    neg, keep3 = _offsets([-1, 4], [0])
    assert L.lora_validate_segments_host(ctypes.byref(neg), 8, 4) == B.LORA_E_SHAPE
    empty, keep4 = _offsets([0, 0, 3, 3, 3], [2, -1, 0, 1])                             # empty and -1 segments
    assert L.lora_validate_segments_host(ctypes.byref(empty), 3, 4) == B.LORA_OK
    rm, keep5 = _offsets([0, 2, 3], [1, 0], row_map=[5, 1, 5])
    assert L.lora_validate_segments_host(ctypes.byref(rm), 6, 2) == B.LORA_E_INDEX     # row 5 twice
    rm2, keep6 = _offsets([0, 2, 3], [1, 0], row_map=[5, 1, 6])
    assert L.lora_validate_segments_host(ctypes.byref(rm2), 6, 2) == B.LORA_E_INDEX    # row 6 >= 6
    assert L.lora_validate_segments_host(ctypes.byref(rm2), 7, 2) == B.LORA_OK
    tall, keep7 = _offsets([0, 8], [0], tile_rows=65)
    assert L.lora_validate_segments_host(ctypes.byref(tall), 8, 1) == B.LORA_E_SHAPE
    # the launching calls check the descriptor before anything else
    c = _desc()
    tall.tile_rows = 65
    assert L.lora_sgmv_shrink(None, FAKE, 16, FAKE, 1024, 8, ctypes.byref(c), ctypes.byref(tall)) == B.LORA_E_SHAPE
    nul, keep8 = _offsets([0, 8], [0])
    nul.seg_ptr = None
    assert L.lora_sgmv_expand(None, FAKE, 1024, FAKE, 16, 8, ctypes.byref(c), ctypes.byref(nul)) == B.LORA_E_NULL
    neg_seg = B.CSegments()
    neg_seg.n_seg = -1
    assert L.lora_sgmv_shrink(None, FAKE, 16, FAKE, 1024, 8, ctypes.byref(c), ctypes.byref(neg_seg)) == B.LORA_E_SHAPE
    # no segments, or no rows: nothing is read or launched
    none = B.CSegments()
    assert L.lora_sgmv_shrink(None, FAKE, 16, FAKE, 1024, 8, ctypes.byref(c), ctypes.byref(none)) == B.LORA_OK
    assert L.lora_sgmv_expand(None, FAKE, 1024, FAKE, 16, 0, ctypes.byref(c), ctypes.byref(ok)) == B.LORA_OK


def test_offsets_host_helper_rejects_bad_offsets():
    with pytest.raises(B.LoraError):
        B.segments_from_offsets(np.array([0, 3, 2], np.int32), np.array([0, 1], np.int32), device="cpu")
    segs = B.segments_from_offsets(np.array([0, 1, 4, 6, 8], np.int32), np.arange(4, dtype=np.int32), device="cpu")
    assert segs.is_offsets and segs.c.n_seg == 4 and segs.n_tiles == 0
    with pytest.raises(ValueError, match="GPU tensor"):
        segs.ref


def test_workspace_bytes():
    L = B.lib()
    out = ctypes.c_size_t(123)
    assert L.lora_sgmv_workspace_bytes(None, 32, 32, ctypes.byref(out)) == B.LORA_OK
    assert out.value == L.lora_handoff_bytes(32) > 0
    assert L.lora_sgmv_workspace_bytes(None, 0, 0, ctypes.byref(out)) == B.LORA_OK and out.value == 0
    assert L.lora_sgmv_workspace_bytes(None, -1, 0, ctypes.byref(out)) == B.LORA_E_SHAPE
    assert L.lora_sgmv_workspace_bytes(None, 1, -1, ctypes.byref(out)) == B.LORA_E_SHAPE
    assert L.lora_sgmv_workspace_bytes(None, 1, 1, None) == B.LORA_E_NULL
    assert B.lora_sgmv_workspace_bytes(8, 4) == L.lora_handoff_bytes(8)


def test_noalloc_handoff_rejects_more_rows_than_its_scratch():
    """The allocation-free hand-off form holds LORA_NOALLOC_MAX_ROWS rows; larger calls are
    rejected on the host before anything reaches the GPU."""
    L = B.lib()
    c1 = _desc()
    arr = (B.CProj * 1)()
    arr[0].w, arr[0].v, arr[0].ldv, arr[0].y, arr[0].ldy = ctypes.addressof(c1), FAKE, 16, FAKE, 1024
    n = B.NOALLOC_MAX_ROWS + 1
    assert L.lora_bgmv_multi_handoff_noalloc(None, FAKE, 1024, FAKE, n, 1, arr) == B.LORA_E_SHAPE
    assert "scratch" in B.last_error() and str(B.NOALLOC_MAX_ROWS) in B.last_error()
    assert L.lora_bgmv_multi_handoff_noalloc(None, FAKE, 1024, None, 8, 1, arr) == B.LORA_E_NULL
    assert L.lora_bgmv_multi_handoff_noalloc(None, FAKE, 1024, FAKE, 0, 1, arr) == B.LORA_OK   # nothing to do
