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
           "lora_bgmv_shrink_multi", "lora_bgmv_expand_multi", "lora_pick_tile_rows", "lora_pick_expand_tile_rows",
           "lora_bgmv_multi",
           "lora_set_plan", "lora_set_stream_weights", "lora_pool_state_bytes", "lora_pool_init", "lora_pool_alloc", "lora_pool_release",
           "lora_pool_free_count", "lora_pool_pages_for", "lora_pool_load_header_bytes", "lora_pool_load",
           "lora_handoff_bytes", "lora_bgmv_multi_handoff", "lora_sgmv_multi_handoff", "lora_set_handoff_polls",
           "lora_sgmv_workspace_bytes", "lora_bgmv_multi_handoff_noalloc"]
NOALLOC_MAX_ROWS = 1024
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
    _fields_ = [("n_seg", ctypes.c_int32), ("seg_ptr", ctypes.c_void_p), ("seg_slot", ctypes.c_void_p),
                ("row_map", ctypes.c_void_p), ("tile_rows", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
                ("tiles", ctypes.c_void_p), ("n_pos", ctypes.c_int32), ("max_rows", ctypes.c_int32)]


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
            "lora_pick_expand_tile_rows": [P, I32],
            "lora_bgmv_multi": [P, P, I64, P, I32, I32, P],
            "lora_set_plan": [I32, I32],
            "lora_set_stream_weights": [I32],
            "lora_bgmv_multi_handoff": [P, P, I64, P, I32, I32, P, P, ctypes.c_size_t],
            "lora_set_handoff_polls": [I32],
            "lora_sgmv_multi_handoff": [P, P, I64, I32, P, I32, P, P, ctypes.c_size_t],
            "lora_pool_init": [P, ctypes.c_size_t, I64],
            "lora_pool_alloc": [P, I32, P],
            "lora_pool_release": [P, I32, P],
            "lora_pool_load": [P, I32, P, P, ctypes.c_size_t, P, ctypes.c_size_t],
            "lora_sgmv_workspace_bytes": [P, I32, I32, P],
            "lora_bgmv_multi_handoff_noalloc": [P, P, I64, P, I32, I32, P],
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
        L.lora_pick_expand_tile_rows.restype = ctypes.c_int32
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


# ------------------------------------------------------------------ argument checks
# The C ABI receives raw pointers and leading dimensions and cannot tell a host pointer
# or a too-short tensor from a valid one, so every tensor is checked here before any
# call: dtype, unit stride along the last dimension, enough rows and columns for what
# the kernels touch, and residence on the current GPU.  Violations raise ValueError.
def _torch_dtype(name):
    import torch
    return {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32, "i64": torch.int64,
            "u8": torch.uint8}[name]


def _on_gpu(t, what):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor (got device {t.device})")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")


def check_matrix(t, what, dtype, rows, cols, gpu=True):
    """t: 2-D tensor of `dtype` with unit column stride, >= rows rows and >= cols columns."""
    if t is None:
        raise ValueError(f"{what} is required")
    if not hasattr(t, "dtype") or t.dtype != _torch_dtype(dtype):
        raise ValueError(f"{what} must have dtype {dtype} (got {getattr(t, 'dtype', type(t).__name__)})")
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D (got {t.dim()}-D)")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{what} needs unit stride along its columns (stride {t.stride(1)})")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{what} is {tuple(t.shape)}, needs at least ({rows}, {cols})")
    if t.shape[0] > 1 and t.stride(0) < cols:
        raise ValueError(f"{what} has row stride {t.stride(0)} < {cols} columns")
    if gpu:
        _on_gpu(t, what)


def check_vector(t, what, dtype, n, gpu=True):
    """t: contiguous tensor of `dtype` with at least n elements."""
    if t is None:
        raise ValueError(f"{what} is required")
    if not hasattr(t, "dtype") or t.dtype != _torch_dtype(dtype):
        raise ValueError(f"{what} must have dtype {dtype} (got {getattr(t, 'dtype', type(t).__name__)})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{what} has {t.numel()} elements, needs at least {n}")
    if gpu:
        _on_gpu(t, what)


def _rows_arg(n_rows):
    n_rows = int(n_rows)
    if n_rows < 0:
        raise ValueError(f"n_rows = {n_rows}")
    return n_rows


# ------------------------------------------------------------------ descriptors
class Weights:
    """lora_weights over device tensors (kept alive by this object)."""

    def __init__(self, *, num_slots, d_in, d_out, r_max, rank, scale, a_t=None, b=None, pool=None,
                 page_elems=0, page_table=None, a_pt_off=None, b_pt_off=None):
        # dtypes and sizes here; residence on the current GPU at every launch (on_gpu)
        S = int(num_slots)
        check_vector(rank, "rank", "i32", S, gpu=False)
        check_vector(scale, "scale", "f32", S, gpu=False)
        if pool is None:
            for t, what, d in ((a_t, "a_t", d_in), (b, "b", d_out)):
                check_vector(t, what, "f16", S * int(r_max) * int(d), gpu=False)
        else:
            if pool.dim() != 2 or int(pool.shape[1]) != int(page_elems):
                raise ValueError(f"pool must be [num_pages, page_elems = {page_elems}] (got {tuple(pool.shape)})")
            check_vector(pool, "pool", "f16", 1, gpu=False)
            check_vector(page_table, "page_table", "i32", 1, gpu=False)
            check_vector(a_pt_off, "a_pt_off", "i64", S, gpu=False)
            check_vector(b_pt_off, "b_pt_off", "i64", S, gpu=False)
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

    def on_gpu(self):
        for t, what in zip(self.tensors, ("rank", "scale", "a_t", "b", "pool", "page_table", "a_pt_off",
                                           "b_pt_off")):
            if t is not None:
                _on_gpu(t, f"weights.{what}")

    @property
    def ref(self):
        self.on_gpu()
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
    """lora_segments over device tensors, in one of its two forms:

    * tile list (the precomputed fast path): Segments(tiles, row_map, n_pos, max_rows),
      tiles an int32 [n_tiles, 4] tensor from lora_build_tiles;
    * offsets (the pages' form): Segments.offsets(seg_ptr, seg_slot, row_map, tile_rows),
      the launch cuts the segments into tiles on the device."""

    def __init__(self, tiles, row_map, n_pos, max_rows=0):
        self.tiles, self.row_map = tiles, row_map
        self.seg_ptr = self.seg_slot = None
        c = CSegments()
        c.n_tiles = int(tiles.shape[0]) if tiles is not None else 0
        c.tiles = _ptr(tiles) if c.n_tiles else None
        if c.n_tiles and not c.tiles:
            raise ValueError("tiles is empty")
        c.row_map = _ptr(row_map)
        c.n_pos = int(n_pos)
        c.max_rows = int(max_rows)
        self.c = c
        self.n_tiles = c.n_tiles
        self.n_pos = c.n_pos

    @classmethod
    def offsets(cls, seg_ptr, seg_slot, row_map=None, tile_rows=0):
        """Offsets form: seg_ptr int32 [n_seg + 1] and seg_slot int32 [n_seg] device tensors
        (rows grouped by adapter; segments may be empty), row_map int32 device tensor or None,
        tile_rows 0 (library's choice) or 1..64."""
        self = cls.__new__(cls)
        n_seg = int(seg_slot.numel())
        check_vector(seg_ptr, "seg_ptr", "i32", n_seg + 1, gpu=False)
        check_vector(seg_slot, "seg_slot", "i32", n_seg, gpu=False)
        if row_map is not None:
            check_vector(row_map, "row_map", "i32", 0, gpu=False)
        self.tiles, self.row_map, self.seg_ptr, self.seg_slot = None, row_map, seg_ptr, seg_slot
        c = CSegments()
        c.n_seg, c.seg_ptr, c.seg_slot = n_seg, _ptr(seg_ptr), _ptr(seg_slot)
        c.row_map, c.tile_rows = _ptr(row_map), int(tile_rows)
        self.c = c
        self.n_tiles = 0
        self.n_pos = 0
        return self

    @property
    def is_offsets(self):
        return self.tiles is None and self.seg_ptr is not None

    @property
    def ref(self):
        if self.is_offsets:
            _gpu(seg_ptr=self.seg_ptr, seg_slot=self.seg_slot, row_map=self.row_map)
        else:
            if self.n_tiles:
                check_matrix(self.tiles, "tiles", "i32", self.n_tiles, 4)
            if self.row_map is not None:
                check_vector(self.row_map, "row_map", "i32", self.n_pos)
        return ctypes.byref(self.c)


def segments_from_offsets(seg_ptr, seg_slot, row_map=None, tile_rows=0, device="cuda", n_rows=None,
                          num_slots=None):
    """Device copies of host offsets (and row map) as an offsets-form Segments descriptor,
    after lora_validate_segments_host on the host copies (n_rows and num_slots default to
    the smallest values the arrays allow)."""
    import torch
    sp = np.ascontiguousarray(seg_ptr, dtype=np.int32)
    ss = np.ascontiguousarray(seg_slot, dtype=np.int32)
    rm = None if row_map is None else np.ascontiguousarray(row_map, dtype=np.int32)
    host = CSegments()
    host.n_seg, host.seg_ptr, host.seg_slot = len(ss), sp.ctypes.data, ss.ctypes.data
    host.row_map = rm.ctypes.data if rm is not None else None
    host.tile_rows = int(tile_rows)
    if n_rows is None:
        n_rows = max(int(sp[-1]), int(rm.max()) + 1 if rm is not None and len(rm) else 0)
    if num_slots is None:
        num_slots = max(int(ss.max()) + 1 if len(ss) else 1, 1)
    _check(lib().lora_validate_segments_host(ctypes.byref(host), int(n_rows), int(num_slots)))
    dev = lambda a: torch.from_numpy(a).to(device)
    return Segments.offsets(dev(sp), dev(ss), None if rm is None else dev(rm), tile_rows)


def lora_sgmv_workspace_bytes(n_rows, n_seg=0):
    """Device workspace bytes the calls on a batch need (the one-launch forms' hand-off
    buffer; the separate shrink and expand need none)."""
    out = ctypes.c_size_t()
    _check(lib().lora_sgmv_workspace_bytes(None, int(n_rows), int(n_seg), ctypes.byref(out)))
    return int(out.value)


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


def lora_pick_expand_tile_rows(seg_ptr):
    """Host: the tile height suited to the expand launches of this batch."""
    seg_ptr = np.ascontiguousarray(seg_ptr, dtype=np.int32)
    return int(lib().lora_pick_expand_tile_rows(_ptr(seg_ptr), len(seg_ptr) - 1))


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


def segments_to_device(tiles, row_map, n_pos, device="cuda", n_rows=None, num_slots=None):
    """Device copies of a host tile list (and row map) as a Segments descriptor.

    The host copies are checked first with lora_validate_segments_host: every position
    in at most one tile and every row at most once in the row map (the one-launch
    hand-off form counts each row's work items and relies on this), tiles inside the
    positions, slots inside [-1, num_slots).  n_rows and num_slots default to the
    smallest values the arrays allow."""
    import torch
    tiles = np.ascontiguousarray(tiles, dtype=np.int32).reshape(-1, 4)
    rm_h = None if row_map is None else np.ascontiguousarray(row_map, dtype=np.int32)
    host = CSegments()
    host.n_tiles = len(tiles)
    host.tiles = tiles.ctypes.data if len(tiles) else None
    host.row_map = rm_h.ctypes.data if rm_h is not None else None
    host.n_pos = int(n_pos)
    host.max_rows = int(tiles[:, 2].max()) if len(tiles) else 0
    if n_rows is None:
        n_rows = (int(rm_h.max()) + 1 if rm_h is not None and len(rm_h) else 0) if rm_h is not None else int(n_pos)
    if num_slots is None:
        num_slots = max(int(tiles[:, 0].max()) + 1 if len(tiles) else 1, 1)
    _check(lib().lora_validate_segments_host(ctypes.byref(host), int(n_rows), int(num_slots)))
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


# Shapes and dtypes of all arguments are checked first, residence on the GPU last
# (_gpu), so the first message names the first argument that is wrong in kind.
def _x(x, n_rows, d_in):
    check_matrix(x, "x", "f16", n_rows, d_in, gpu=False)


def _v(v, n_rows, w, what="v"):
    check_matrix(v, what, "f32", n_rows, w.r_max, gpu=False)


def _y(y, n_rows, w, what="y"):
    check_matrix(y, what, "f16", n_rows, w.d_out, gpu=False)


def _idx(idx, n_rows):
    check_vector(idx, "idx", "i32", n_rows, gpu=False)


def _gpu(**tensors):
    for what, t in tensors.items():
        if t is not None:
            _on_gpu(t, what)


def _segs(segments, n_rows):
    if not isinstance(segments, Segments):
        raise ValueError("segments must be a Segments descriptor")
    if not segments.is_offsets and segments.row_map is None and segments.n_pos > n_rows:
        raise ValueError(f"segments cover {segments.n_pos} positions without a row map, n_rows = {n_rows}")


def lora_sgmv_shrink(v, x, weights: Weights, segments: Segments, n_rows=None, stream=None):
    n_rows = _rows_arg(x.shape[0] if n_rows is None else n_rows)
    _x(x, n_rows, weights.d_in)
    _v(v, n_rows, weights)
    _segs(segments, n_rows)
    _gpu(v=v, x=x)
    _check(lib().lora_sgmv_shrink(_stream(stream), _ptr(v), _ld(v), _ptr(x), _ld(x), n_rows, weights.ref,
                                  segments.ref))


def lora_sgmv_expand(y, v, weights: Weights, segments: Segments, n_rows=None, stream=None):
    n_rows = _rows_arg(y.shape[0] if n_rows is None else n_rows)
    _y(y, n_rows, weights)
    _v(v, n_rows, weights)
    _segs(segments, n_rows)
    _gpu(y=y, v=v)
    _check(lib().lora_sgmv_expand(_stream(stream), _ptr(y), _ld(y), _ptr(v), _ld(v), n_rows, weights.ref,
                                  segments.ref))


def lora_bgmv_shrink(v, x, idx, weights: Weights, stream=None):
    n_rows = _rows_arg(x.shape[0])
    _x(x, n_rows, weights.d_in)
    _v(v, n_rows, weights)
    _idx(idx, n_rows)
    _gpu(v=v, x=x, idx=idx)
    _check(lib().lora_bgmv_shrink(_stream(stream), _ptr(v), _ld(v), _ptr(x), _ld(x), _ptr(idx), n_rows,
                                  weights.ref))


def lora_bgmv_expand(y, v, idx, weights: Weights, stream=None):
    n_rows = _rows_arg(y.shape[0])
    _y(y, n_rows, weights)
    _v(v, n_rows, weights)
    _idx(idx, n_rows)
    _gpu(y=y, v=v, idx=idx)
    _check(lib().lora_bgmv_expand(_stream(stream), _ptr(y), _ld(y), _ptr(v), _ld(v), _ptr(idx), n_rows,
                                  weights.ref))


def lora_bgmv(y, x, idx, weights: Weights, v, stream=None):
    n_rows = _rows_arg(y.shape[0])
    _x(x, n_rows, weights.d_in)
    _y(y, n_rows, weights)
    _v(v, n_rows, weights)
    _idx(idx, n_rows)
    _gpu(y=y, x=x, idx=idx, v=v)
    _check(lib().lora_bgmv(_stream(stream), _ptr(y), _ld(y), _ptr(x), _ld(x), _ptr(idx), n_rows,
                           weights.ref, _ptr(v), _ld(v)))


def lora_set_plan(shrink_rank_rows=0, rows_per_pass=0):
    """Fix (or, with 0, release) the rank-rows per VALU shrink workgroup and the rows per
    pass of the segment-form VALU kernels for this thread's later launches; results are
    bit-identical either way."""
    _check(lib().lora_set_plan(int(shrink_rank_rows), int(rows_per_pass)))


def lora_set_stream_weights(on: bool):
    """Per-thread hint: the later per-row calls' rows use distinct adapters, so dense
    weights are read with streaming loads (same bits; slower when adapters repeat)."""
    _check(lib().lora_set_stream_weights(1 if on else 0))


def lora_set_handoff_polls(polls=-1):
    """Polls an expand workgroup of the hand-off form makes before computing its v itself
    (0: always computes it; negative: the library's default), for this thread's later
    calls; results are bit-identical either way."""
    _check(lib().lora_set_handoff_polls(int(polls)))


def lora_set_launch_events(start_event, stop_event):
    """Attach raw hipEvent_t handles (ints) to this thread's next kernel launch."""
    _check(lib().lora_set_launch_events(start_event, stop_event))


# ------------------------------------------------------------------ several projections per launch
def proj_list(items, n_rows=None, expand=False):
    """items: sequence of (Weights, v, y_or_None).  Returns a ctypes lora_proj array.  With
    n_rows, each v (and, for an expand, each y) is checked to cover n_rows rows."""
    if not 1 <= len(items) <= MAX_PROJ:
        raise ValueError(f"{len(items)} projections (1..{MAX_PROJ} per launch)")
    arr = (CProj * len(items))()
    for i, (w, v, y) in enumerate(items):
        if n_rows is not None:
            _v(v, n_rows, w, f"v of projection {i}")
            if expand:
                _y(y, n_rows, w, f"y of projection {i}")
        w.on_gpu()
        _gpu(**{f"v of projection {i}": v, f"y of projection {i}": y if expand else None})
        arr[i].w = ctypes.addressof(w.c)
        arr[i].v, arr[i].ldv = _ptr(v), _ld(v)
        arr[i].y, arr[i].ldy = (_ptr(y), _ld(y)) if y is not None else (None, 0)
    return arr


def lora_sgmv_shrink_multi(x, segments: Segments, items, n_rows=None, stream=None):
    n_rows = _rows_arg(x.shape[0] if n_rows is None else n_rows)
    _x(x, n_rows, items[0][0].d_in)
    _segs(segments, n_rows)
    arr = proj_list(items, n_rows)
    _gpu(x=x)
    _check(lib().lora_sgmv_shrink_multi(_stream(stream), _ptr(x), _ld(x), n_rows, segments.ref, len(items), arr))


def lora_sgmv_expand_multi(segments: Segments, items, n_rows, stream=None):
    n_rows = _rows_arg(n_rows)
    _segs(segments, n_rows)
    arr = proj_list(items, n_rows, expand=True)
    _check(lib().lora_sgmv_expand_multi(_stream(stream), n_rows, segments.ref, len(items), arr))


def lora_bgmv_shrink_multi(x, idx, items, stream=None):
    n_rows = _rows_arg(x.shape[0])
    _x(x, n_rows, items[0][0].d_in)
    _idx(idx, n_rows)
    arr = proj_list(items, n_rows)
    _gpu(x=x, idx=idx)
    _check(lib().lora_bgmv_shrink_multi(_stream(stream), _ptr(x), _ld(x), _ptr(idx), n_rows, len(items), arr))


def lora_bgmv_expand_multi(idx, items, n_rows, stream=None):
    n_rows = _rows_arg(n_rows)
    _idx(idx, n_rows)
    arr = proj_list(items, n_rows, expand=True)
    _gpu(idx=idx)
    _check(lib().lora_bgmv_expand_multi(_stream(stream), _ptr(idx), n_rows, len(items), arr))


def handoff_workspace(n_rows, device="cuda"):
    """A zeroed workspace for lora_bgmv_multi_handoff calls of up to n_rows rows (the
    library leaves it zeroed after every call)."""
    import torch
    nbytes = int(lib().lora_handoff_bytes(int(n_rows)))
    return torch.zeros(max(nbytes, 256) // 4, dtype=torch.int32, device=device)


def _work(work):
    check_vector(work, "work", "i32", 1)
    return _ptr(work), int(work.numel() * work.element_size())


def lora_bgmv_multi_handoff(x, idx, items, work, stream=None):
    """Shrink and expand of the decode form in one launch, v handed from the shrink's
    workgroups to the expand's through `work` (handoff_workspace); the bits of the
    two-launch path."""
    n_rows = _rows_arg(x.shape[0])
    _x(x, n_rows, items[0][0].d_in)
    _idx(idx, n_rows)
    arr = proj_list(items, n_rows, expand=True)
    wp, wb = _work(work)
    _gpu(x=x, idx=idx)
    _check(lib().lora_bgmv_multi_handoff(_stream(stream), _ptr(x), _ld(x), _ptr(idx), n_rows, len(items), arr, wp,
                                         wb))


def lora_bgmv_multi_handoff_noalloc(x, idx, items, stream=None):
    """lora_bgmv_multi_handoff with the library's own hand-off scratch (at most
    NOALLOC_MAX_ROWS rows; no allocation in the call; calls that may overlap on one GPU
    race)."""
    n_rows = _rows_arg(x.shape[0])
    _x(x, n_rows, items[0][0].d_in)
    _idx(idx, n_rows)
    arr = proj_list(items, n_rows, expand=True)
    _gpu(x=x, idx=idx)
    _check(lib().lora_bgmv_multi_handoff_noalloc(_stream(stream), _ptr(x), _ld(x), _ptr(idx), n_rows, len(items),
                                                 arr))


def lora_sgmv_multi_handoff(x, segs, items, n_rows, work, stream=None):
    """Shrink and expand of the segment form, in one launch with v handed off where the
    tiles are short and the weights dense (otherwise the two launches); the bits of the
    two calls."""
    n_rows = _rows_arg(n_rows)
    _x(x, n_rows, items[0][0].d_in)
    _segs(segs, n_rows)
    arr = proj_list(items, n_rows, expand=True)
    wp, wb = _work(work)
    _gpu(x=x)
    _check(lib().lora_sgmv_multi_handoff(_stream(stream), _ptr(x), _ld(x), n_rows, segs.ref, len(items), arr, wp, wb))


def lora_bgmv_multi(x, idx, items, stream=None):
    """Shrink and expand of the decode form (two launches, arguments of both checked first)."""
    n_rows = _rows_arg(x.shape[0])
    _x(x, n_rows, items[0][0].d_in)
    _idx(idx, n_rows)
    arr = proj_list(items, n_rows, expand=True)
    _gpu(x=x, idx=idx)
    _check(lib().lora_bgmv_multi(_stream(stream), _ptr(x), _ld(x), _ptr(idx), n_rows, len(items), arr))


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
    # the job table, then every page-id list, then every job's rank-rows back to back (the
    # layout lora_pool_load's direct route takes: consecutive pages become one copy)
    datas = []
    for i, ad in enumerate(adapters):
        j = jobs[i]
        j.w = ctypes.addressof(ad["w"].c)
        j.slot, j.rank, j.scale, j.reserved = int(ad["slot"]), int(ad["rank"]), float(ad["scale"]), 0
        j.pt_off = int(ad.get("pt_off", 0))
        if ad["rank"] == 0:
            continue
        ids = np.ascontiguousarray(ad["pages"], np.int32).view(np.uint8)
        j.pages_off = off
        parts.append((off, ids))
        off = -(-(off + len(ids)) // 16) * 16
        datas.append((j, np.concatenate([np.ascontiguousarray(ad["a_t"], np.float16).ravel(),
                                         np.ascontiguousarray(ad["b"], np.float16).ravel()]).view(np.uint8)))
    for j, data in datas:
        j.data_off = off
        parts.append((off, data))
        off = -(-(off + len(data)) // 16) * 16
    blob = torch.zeros(max(off, 16), dtype=torch.uint8, pin_memory=pinned)
    view = blob.numpy()
    for o, d in parts:
        view[o:o + len(d)] = d
    return blob, jobs


def lora_pool_load(jobs, blob, staging, stream=None):
    """Place the packed adapters (pack_adapters) into their pools: blob is the host uint8
    tensor, staging a GPU uint8 tensor of at least blob's size."""
    check_vector(blob, "blob", "u8", 1, gpu=False)
    if blob.is_cuda:
        raise ValueError("blob must be host memory (page-locked for an asynchronous copy)")
    check_vector(staging, "staging", "u8", int(blob.numel()))
    for j in jobs:
        if not j.w:
            raise ValueError("load job without a target descriptor")
    _check(lib().lora_pool_load(_stream(stream), len(jobs), jobs, _ptr(blob), int(blob.numel()), _ptr(staging),
                                int(staging.numel())))
