"""Thin ctypes binding of ``liblora_sgmv.so`` (argument marshalling only).

Functions carry the C names of ``include/lora_sgmv.h``.  Tensors are torch tensors on
the GPU (fp16 x / y / A / B, fp32 v / scale, int32 indices, int64 page-table
offsets); the binding passes their device pointers and torch's current HIP stream.
Every computation happens in the library's kernels.  If the library is missing, the
first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

LORA_OK = 0
LORA_E_NULL = -1
LORA_E_SHAPE = -2
LORA_E_ALIGN = -3
LORA_E_INDEX = -4
LORA_E_UNSUPPORTED = -5
LORA_E_HIP = -6
LORA_E_CAPACITY = -7
LAYOUT_DENSE, LAYOUT_PAGED = 0, 1
MAX_RANK = 64
MAX_TILE_ROWS = 64

EXPORTS = ["lora_build_segments", "lora_tiles_bound", "lora_build_tiles", "lora_validate_weights_host",
           "lora_validate_segments_host", "lora_sgmv_shrink", "lora_sgmv_expand",
           "lora_bgmv_shrink", "lora_bgmv_expand", "lora_bgmv", "lora_last_error", "lora_status_str",
           "lora_abi_version", "lora_set_launch_events", "lora_sgmv_shrink_multi", "lora_sgmv_expand_multi",
           "lora_bgmv_shrink_multi", "lora_bgmv_expand_multi", "lora_pick_tile_rows", "lora_bgmv_multi",
           "lora_set_plan", "lora_pool_state_bytes", "lora_pool_init", "lora_pool_alloc", "lora_pool_release",
           "lora_pool_free_count", "lora_pool_pages_for", "lora_pool_load_header_bytes", "lora_pool_load",
           "lora_handoff_bytes", "lora_bgmv_multi_handoff", "lora_sgmv_multi_handoff", "lora_set_handoff_polls"]
MAX_PROJ = 4


class LoraError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (status {code})")
        self.code = code


class CWeights(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("num_slots", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("d_out", ctypes.c_int32), ("r_max", ctypes.c_int32), ("rank", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("a_t", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("pool", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("page_elems", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("pt_entries", ctypes.c_int64),
                ("a_pt_off", ctypes.c_void_p), ("b_pt_off", ctypes.c_void_p)]


class CProj(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("v", ctypes.c_void_p), ("ldv", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("ldy", ctypes.c_int64)]


class CLoadJob(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("slot", ctypes.c_int32), ("rank", ctypes.c_int32), ("scale", ctypes.c_float),
                ("reserved", ctypes.c_int32), ("pt_off", ctypes.c_int64), ("data_off", ctypes.c_int64),
                ("pages_off", ctypes.c_int64)]


class CSegments(ctypes.Structure):
    _fields_ = [("n_tiles", ctypes.c_int32), ("tiles", ctypes.c_void_p), ("row_map", ctypes.c_void_p),
                ("n_pos", ctypes.c_int32), ("max_rows", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} is missing: build it with "
                               "`python -m segmented_gather_matmul_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(_build.LIB)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "lora_build_segments": [P, I32, I32, P, P, P, P, P],
            "lora_tiles_bound": [I32, I32, I32],
            "lora_build_tiles": [P, P, I32, I32, P, I32, P],
            "lora_validate_weights_host": [P],
            "lora_validate_segments_host": [P, I32, I32],
            "lora_sgmv_shrink": [P, P, I64, P, I64, I32, P, P],
            "lora_sgmv_expand": [P, P, I64, P, I64, I32, P, P],
            "lora_bgmv_shrink": [P, P, I64, P, I64, P, I32, P],
            "lora_bgmv_expand": [P, P, I64, P, I64, P, I32, P],
            "lora_bgmv": [P, P, I64, P, I64, P, I32, P, P, I64],
            "lora_status_str": [ctypes.c_int],
            "lora_last_error": [],
            "lora_abi_version": [],
            "lora_set_launch_events": [P, P],
            "lora_sgmv_shrink_multi": [P, P, I64, I32, P, I32, P],
            "lora_sgmv_expand_multi": [P, I32, P, I32, P],
            "lora_bgmv_shrink_multi": [P, P, I64, P, I32, I32, P],
            "lora_bgmv_expand_multi": [P, P, I32, I32, P],
            "lora_pick_tile_rows": [P, I32],
            "lora_bgmv_multi": [P, P, I64, P, I32, I32, P, I32],
            "lora_set_plan": [I32, I32],
            "lora_bgmv_multi_handoff": [P, P, I64, P, I32, I32, P, P, ctypes.c_size_t],
            "lora_set_handoff_polls": [I32],
            "lora_sgmv_multi_handoff": [P, P, I64, I32, P, I32, P, P, ctypes.c_size_t],
            "lora_pool_init": [P, ctypes.c_size_t, I64],
            "lora_pool_alloc": [P, I32, P],
            "lora_pool_release": [P, I32, P],
            "lora_pool_load": [P, I32, P, P, ctypes.c_size_t, P, ctypes.c_size_t],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.lora_tiles_bound.restype = ctypes.c_int32
        for name, args, res in (("lora_pool_state_bytes", [I64], ctypes.c_size_t),
                                ("lora_pool_free_count", [P], I64),
                                ("lora_pool_pages_for", [I32, I32, I32, I32], I64),
                                ("lora_pool_load_header_bytes", [I32], ctypes.c_size_t),
                                ("lora_handoff_bytes", [I32], ctypes.c_size_t)):
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        L.lora_pick_tile_rows.restype = ctypes.c_int32
        L.lora_last_error.restype = ctypes.c_char_p
        L.lora_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().lora_last_error().decode()


def status_str(code: int) -> str:
    return lib().lora_status_str(code).decode()


def _check(code: int):
    if code != LORA_OK:
        raise LoraError(code, last_error() or status_str(code))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ descriptors
class Weights:
    """lora_weights over device tensors (kept alive by this object)."""

    def __init__(self, *, num_slots, d_in, d_out, r_max, rank, scale, a_t=None, b=None, pool=None,
                 page_elems=0, page_table=None, a_pt_off=None, b_pt_off=None):
        self.tensors = [rank, scale, a_t, b, pool, page_table, a_pt_off, b_pt_off]
        c = CWeights()
        c.layout = LAYOUT_PAGED if pool is not None else LAYOUT_DENSE
        c.num_slots, c.d_in, c.d_out, c.r_max = int(num_slots), int(d_in), int(d_out), int(r_max)
        c.rank, c.scale = _ptr(rank), _ptr(scale)
        c.a_t, c.b, c.pool = _ptr(a_t), _ptr(b), _ptr(pool)
        c.num_pages = int(pool.shape[0]) if pool is not None else 0
        c.page_elems = int(page_elems)
        c.page_table = _ptr(page_table)
        c.pt_entries = int(page_table.numel() if hasattr(page_table, "numel") else
                           (len(page_table) if page_table is not None else 0))
        c.a_pt_off, c.b_pt_off = _ptr(a_pt_off), _ptr(b_pt_off)
        self.c = c
        self.num_slots, self.d_in, self.d_out, self.r_max = c.num_slots, c.d_in, c.d_out, c.r_max

    @property
    def ref(self):
        return ctypes.byref(self.c)


def weights_from_store(store, device="cuda"):
    """Device copy of a workloads.DenseStore / PagedStore as a Weights descriptor."""
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    common = dict(num_slots=store.num_slots, d_in=store.d_in, d_out=store.d_out, r_max=store.r_max,
                  rank=t(store.rank.astype(np.int32)), scale=t(store.scale.astype(np.float32)))
    if hasattr(store, "pool"):
        return Weights(**common, pool=t(store.pool), page_elems=store.page_elems,
                       page_table=t(store.page_table.astype(np.int32)),
                       a_pt_off=t(store.a_pt_off.astype(np.int64)), b_pt_off=t(store.b_pt_off.astype(np.int64)))
    return Weights(**common, a_t=t(store.a_t), b=t(store.b))


class Segments:
    """lora_segments over device tensors: the tile work-list and the row map."""

    def __init__(self, tiles, row_map, n_pos, max_rows=0):
        self.tiles, self.row_map = tiles, row_map
        c = CSegments()
        c.n_tiles = int(tiles.shape[0]) if tiles is not None else 0
        c.tiles = _ptr(tiles) if c.n_tiles else None
        c.row_map = _ptr(row_map)
        c.n_pos = int(n_pos)
        c.max_rows = int(max_rows)
        self.c = c
        self.n_tiles = c.n_tiles

    @property
    def ref(self):
        return ctypes.byref(self.c)


# ------------------------------------------------------------------ host metadata
def lora_build_segments(idx, num_slots):
    """Host: (row_map, seg_ptr, seg_slot, n_act) as int32 numpy arrays."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n = len(idx)
    cap = min(n, int(num_slots))
    row_map = np.empty(max(n, 1), dtype=np.int32)
    seg_ptr = np.empty(cap + 1, dtype=np.int32)
    seg_slot = np.empty(max(cap, 1), dtype=np.int32)
    n_seg, n_act = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().lora_build_segments(_ptr(idx) if n else None, n, int(num_slots), _ptr(row_map), _ptr(seg_ptr),
                                     _ptr(seg_slot), ctypes.byref(n_seg), ctypes.byref(n_act)))
    g = n_seg.value
    return row_map[:n_act.value].copy(), seg_ptr[:g + 1].copy(), seg_slot[:g].copy(), n_act.value


def lora_tiles_bound(n_pos, n_seg, max_tile_rows=MAX_TILE_ROWS):
    return int(lib().lora_tiles_bound(int(n_pos), int(n_seg), int(max_tile_rows)))


def lora_pick_tile_rows(seg_ptr):
    seg_ptr = np.ascontiguousarray(seg_ptr, dtype=np.int32)
    return int(lib().lora_pick_tile_rows(_ptr(seg_ptr), len(seg_ptr) - 1))


def lora_build_tiles(seg_ptr, seg_slot, max_tile_rows=None):
    """Host: tile work-list as int32 [n_tiles, 4] = (slot, pos0, nrows, seg).
    max_tile_rows None: the height lora_pick_tile_rows suggests for this batch."""
    seg_ptr = np.ascontiguousarray(seg_ptr, dtype=np.int32)
    seg_slot = np.ascontiguousarray(seg_slot, dtype=np.int32)
    n_seg = len(seg_slot)
    if max_tile_rows is None:
        max_tile_rows = lora_pick_tile_rows(seg_ptr)
    n_pos = int(seg_ptr[-1] - seg_ptr[0]) if n_seg else 0
    cap = max(lora_tiles_bound(n_pos, n_seg, max_tile_rows), 1)
    tiles = np.zeros((cap, 4), dtype=np.int32)
    n = ctypes.c_int32()
    _check(lib().lora_build_tiles(_ptr(seg_ptr), _ptr(seg_slot), n_seg, int(max_tile_rows), _ptr(tiles), cap,
                                  ctypes.byref(n)))
    return tiles[:n.value].copy()


def segments_to_device(tiles, row_map, n_pos, device="cuda"):
    """Device copies of a host tile list (and row map) as a Segments descriptor."""
    import torch
    tiles = np.ascontiguousarray(tiles, dtype=np.int32).reshape(-1, 4)
    t = torch.from_numpy(tiles).to(device)
    rm = None if row_map is None else torch.from_numpy(np.ascontiguousarray(row_map, dtype=np.int32)).to(device)
    return Segments(t, rm, n_pos, int(tiles[:, 2].max()) if len(tiles) else 0)


def lora_validate_weights_host(c_weights_host: CWeights):
    _check(lib().lora_validate_weights_host(ctypes.byref(c_weights_host)))


def lora_validate_segments_host(c_segments_host: CSegments, n_rows, num_slots):
    _check(lib().lora_validate_segments_host(ctypes.byref(c_segments_host), int(n_rows), int(num_slots)))


# ------------------------------------------------------------------ launches
def _ld(t):
    return int(t.stride(0))


def lora_sgmv_shrink(v, x, weights: Weights, segments: Segments, n_rows=None, stream=None):
    n_rows = x.shape[0] if n_rows is None else n_rows
    _check(lib().lora_sgmv_shrink(_stream(stream), _ptr(v), _ld(v), _ptr(x), _ld(x), int(n_rows), weights.ref,
                                  segments.ref))


def lora_sgmv_expand(y, v, weights: Weights, segments: Segments, n_rows=None, stream=None):
    n_rows = y.shape[0] if n_rows is None else n_rows
    _check(lib().lora_sgmv_expand(_stream(stream), _ptr(y), _ld(y), _ptr(v), _ld(v), int(n_rows), weights.ref,
                                  segments.ref))


def lora_bgmv_shrink(v, x, idx, weights: Weights, stream=None):
    _check(lib().lora_bgmv_shrink(_stream(stream), _ptr(v), _ld(v), _ptr(x), _ld(x), _ptr(idx), int(x.shape[0]),
                                  weights.ref))


def lora_bgmv_expand(y, v, idx, weights: Weights, stream=None):
    _check(lib().lora_bgmv_expand(_stream(stream), _ptr(y), _ld(y), _ptr(v), _ld(v), _ptr(idx), int(y.shape[0]),
                                  weights.ref))


def lora_bgmv(y, x, idx, weights: Weights, v, stream=None):
    _check(lib().lora_bgmv(_stream(stream), _ptr(y), _ld(y), _ptr(x), _ld(x), _ptr(idx), int(y.shape[0]),
                           weights.ref, _ptr(v), _ld(v)))


def lora_set_plan(shrink_rank_rows=0, rows_per_pass=0):
    """Fix (or, with 0, release) the rank-rows per VALU shrink workgroup and the rows per
    pass of the segment-form VALU kernels for this thread's later launches; results are
    bit-identical either way."""
    _check(lib().lora_set_plan(int(shrink_rank_rows), int(rows_per_pass)))


def lora_set_handoff_polls(polls=-1):
    """Polls an expand workgroup of the hand-off form makes before computing its v itself
    (0: always computes it; negative: the library's default), for this thread's later
    calls; results are bit-identical either way."""
    _check(lib().lora_set_handoff_polls(int(polls)))


def lora_set_launch_events(start_event, stop_event):
    """Attach raw hipEvent_t handles (ints) to this thread's next kernel launch."""
    _check(lib().lora_set_launch_events(start_event, stop_event))


# ------------------------------------------------------------------ several projections per launch
def proj_list(items):
    """items: sequence of (Weights, v, y_or_None).  Returns a ctypes lora_proj array."""
    arr = (CProj * len(items))()
    for i, (w, v, y) in enumerate(items):
        arr[i].w = ctypes.addressof(w.c)
        arr[i].v, arr[i].ldv = _ptr(v), _ld(v)
        arr[i].y, arr[i].ldy = (_ptr(y), _ld(y)) if y is not None else (None, 0)
    return arr


def lora_sgmv_shrink_multi(x, segments: Segments, items, n_rows=None, stream=None):
    n_rows = x.shape[0] if n_rows is None else n_rows
    arr = proj_list(items)
    _check(lib().lora_sgmv_shrink_multi(_stream(stream), _ptr(x), _ld(x), int(n_rows), segments.ref, len(items), arr))


def lora_sgmv_expand_multi(segments: Segments, items, n_rows, stream=None):
    arr = proj_list(items)
    _check(lib().lora_sgmv_expand_multi(_stream(stream), int(n_rows), segments.ref, len(items), arr))


def lora_bgmv_shrink_multi(x, idx, items, stream=None):
    arr = proj_list(items)
    _check(lib().lora_bgmv_shrink_multi(_stream(stream), _ptr(x), _ld(x), _ptr(idx), int(x.shape[0]), len(items), arr))


def lora_bgmv_expand_multi(idx, items, n_rows, stream=None):
    arr = proj_list(items)
    _check(lib().lora_bgmv_expand_multi(_stream(stream), _ptr(idx), int(n_rows), len(items), arr))


def handoff_workspace(n_rows, device="cuda"):
    """A zeroed workspace for lora_bgmv_multi_handoff calls of up to n_rows rows (the
    library leaves it zeroed after every call)."""
    import torch
    nbytes = int(lib().lora_handoff_bytes(int(n_rows)))
    return torch.zeros(max(nbytes, 256) // 4, dtype=torch.int32, device=device)


def lora_bgmv_multi_handoff(x, idx, items, work, stream=None):
    """Shrink and expand of the decode form in one launch, v handed from the shrink's
    workgroups to the expand's through `work` (handoff_workspace); the bits of the
    two-launch path."""
    arr = proj_list(items)
    _check(lib().lora_bgmv_multi_handoff(_stream(stream), _ptr(x), _ld(x), _ptr(idx), int(x.shape[0]), len(items),
                                         arr, _ptr(work), int(work.numel() * work.element_size())))


def lora_sgmv_multi_handoff(x, segs, items, n_rows, work, stream=None):
    """Shrink and expand of the segment form, in one launch with v handed off where the
    tiles are short and the weights dense (otherwise the two launches); the bits of the
    two calls."""
    arr = proj_list(items)
    _check(lib().lora_sgmv_multi_handoff(_stream(stream), _ptr(x), _ld(x), int(n_rows), segs.ref, len(items), arr,
                                         _ptr(work), int(work.numel() * work.element_size())))


def lora_bgmv_multi(x, idx, items, chunks=0, stream=None):
    """Shrink and expand of the decode form; chunks: 0 library's choice, -1 two launches,
    c >= 1 one launch with c 512-column chunks per workgroup."""
    arr = proj_list(items)
    _check(lib().lora_bgmv_multi(_stream(stream), _ptr(x), _ld(x), _ptr(idx), int(x.shape[0]), len(items), arr,
                                 int(chunks)))


# ------------------------------------------------------------------ adapter pool
class PoolState:
    """Host free-page list (lora_pool_*) in a numpy buffer owned by this object."""

    def __init__(self, num_pages):
        n = lib().lora_pool_state_bytes(int(num_pages))
        if n == 0:
            raise LoraError(LORA_E_SHAPE, f"num_pages = {num_pages}")
        self.buf = np.zeros(n, dtype=np.uint8)
        _check(lib().lora_pool_init(self.buf.ctypes.data, n, int(num_pages)))

    def alloc(self, n):
        out = np.zeros(int(n), dtype=np.int32)
        _check(lib().lora_pool_alloc(self.buf.ctypes.data, int(n), out.ctypes.data if n else None))
        return out

    def release(self, pages):
        pages = np.ascontiguousarray(pages, dtype=np.int32)
        _check(lib().lora_pool_release(self.buf.ctypes.data, len(pages), pages.ctypes.data if len(pages) else None))

    @property
    def free(self):
        return int(lib().lora_pool_free_count(self.buf.ctypes.data))


def lora_pool_pages_for(rank, d_in, d_out, page_elems):
    n = int(lib().lora_pool_pages_for(int(rank), int(d_in), int(d_out), int(page_elems)))
    if n < 0:
        _check(n)
    return n


def pack_adapters(adapters, pinned=True):
    """Blob for lora_pool_load.  adapters: sequence of dicts with keys w (Weights), slot,
    rank, scale, pt_off, a_t (fp16 [rank][d_in] numpy), b (fp16 [rank][d_out]), pages
    (int32 ids in page-table order); rank 0 entries unload.  Returns (blob uint8 tensor,
    page-locked when pinned, and the ctypes job array)."""
    import torch
    n = len(adapters)
    off = int(lib().lora_pool_load_header_bytes(n))
    jobs = (CLoadJob * n)()
    parts = []
    for i, ad in enumerate(adapters):
        j = jobs[i]
        j.w = ctypes.addressof(ad["w"].c)
        j.slot, j.rank, j.scale, j.reserved = int(ad["slot"]), int(ad["rank"]), float(ad["scale"]), 0
        j.pt_off = int(ad.get("pt_off", 0))
        if ad["rank"] == 0:
            continue
        data = np.concatenate([np.ascontiguousarray(ad["a_t"], np.float16).ravel(),
                               np.ascontiguousarray(ad["b"], np.float16).ravel()]).view(np.uint8)
        ids = np.ascontiguousarray(ad["pages"], np.int32).view(np.uint8)
        j.data_off = off
        parts.append((off, data))
        off = -(-(off + len(data)) // 16) * 16
        j.pages_off = off
        parts.append((off, ids))
        off = -(-(off + len(ids)) // 16) * 16
    blob = torch.zeros(max(off, 16), dtype=torch.uint8, pin_memory=pinned)
    view = blob.numpy()
    for o, d in parts:
        view[o:o + len(d)] = d
    return blob, jobs


def lora_pool_load(jobs, blob, staging, stream=None):
    _check(lib().lora_pool_load(_stream(stream), len(jobs), jobs, _ptr(blob), int(blob.numel()), _ptr(staging),
                                int(staging.numel())))
