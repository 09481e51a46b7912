"""Plain CPU oracle of the multi-LoRA add-on path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
imports or calls it, and it shares no code with them.

* ``sgmv`` / ``bgmv``: fp64 loop over rows (C, ``lora_oracle.c``), following the
  Punica operator definition (shrink v = xA, expand y += s.vB per segment or per
  row slot, rows with slot -1 skipped), reading dense or paged adapter storage
  through its own page-table walk.
* ``build_segments``: the per-batch metadata (rows grouped by adapter, as in Punica's
  batch layout construction), written as plain Python loops.
* ``check_tiles``: validity of a tile work-list (every active position in exactly one
  tile, each tile inside one segment).  Several tilings are correct, so only their
  validity is checked.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")


def lib_path(mutant: int = 0) -> str:
    name = "liblora_oracle.so" if mutant == 0 else f"liblora_oracle_mutant{mutant}.so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, out: str | None = None) -> str:
    """Compile the oracle with gcc (OpenMP for the multi-core timing mode)."""
    out = out or lib_path(mutant)
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", f"-DORACLE_MUTANT={int(mutant)}",
           _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Weights(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("num_slots", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("d_out", ctypes.c_int32), ("r_max", ctypes.c_int32),
                ("rank", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("a_t", ctypes.c_void_p), ("b", ctypes.c_void_p), ("pool", ctypes.c_void_p),
                ("page_elems", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("a_pt_off", ctypes.c_void_p), ("b_pt_off", ctypes.c_void_p)]


_libs: dict[int, ctypes.CDLL] = {}


def _load(mutant: int = 0) -> ctypes.CDLL:
    if mutant not in _libs:
        path = lib_path(mutant)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(mutant)
        lib = ctypes.CDLL(path)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_sgmv.argtypes = [P, I32, P, I64, P, I64, I32, P, P, P, P, P, I32]
        lib.oracle_bgmv.argtypes = [P, I32, P, I64, P, I64, P, P, P, I32]
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        _libs[mutant] = lib
    return _libs[mutant]


def _ptr(a):
    return None if a is None else a.ctypes.data


def _weights(store, keep):
    w = _Weights()
    w.num_slots, w.d_in, w.d_out, w.r_max = store.num_slots, store.d_in, store.d_out, store.r_max
    rank = np.ascontiguousarray(store.rank, dtype=np.int32)
    scale = np.ascontiguousarray(store.scale, dtype=np.float32)
    keep += [rank, scale]
    w.rank, w.scale = _ptr(rank), _ptr(scale)
    if hasattr(store, "pool"):
        w.layout = 1
        pool = np.ascontiguousarray(store.pool).view(np.uint16)
        pt = np.ascontiguousarray(store.page_table, dtype=np.int32)
        ao = np.ascontiguousarray(store.a_pt_off, dtype=np.int64)
        bo = np.ascontiguousarray(store.b_pt_off, dtype=np.int64)
        keep += [pool, pt, ao, bo]
        w.pool, w.page_elems, w.page_table = _ptr(pool), store.page_elems, _ptr(pt)
        w.a_pt_off, w.b_pt_off = _ptr(ao), _ptr(bo)
    else:
        w.layout = 0
        a_t = np.ascontiguousarray(store.a_t).view(np.uint16)
        b = np.ascontiguousarray(store.b).view(np.uint16)
        keep += [a_t, b]
        w.a_t, w.b = _ptr(a_t), _ptr(b)
    return w


def _rows(x, y0):
    x = np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)
    y0 = np.ascontiguousarray(y0, dtype=np.float16).view(np.uint16)
    return x, y0


def sgmv(store, x, y0, seg_ptr, seg_slot, row_map=None, nthreads=1, mutant=0):
    """Segment form.  Returns (y fp64 [n, d_out], v fp64 [n, r_max]; NaN where unwritten)."""
    keep = []
    w = _weights(store, keep)
    x, y0 = _rows(x, y0)
    n = x.shape[0]
    seg_ptr = np.ascontiguousarray(seg_ptr, dtype=np.int32)
    seg_slot = np.ascontiguousarray(seg_slot, dtype=np.int32)
    rm = None if row_map is None else np.ascontiguousarray(row_map, dtype=np.int32)
    y = np.empty((n, store.d_out), dtype=np.float64)
    v = np.full((n, store.r_max), np.nan, dtype=np.float64)
    _load(mutant).oracle_sgmv(ctypes.byref(w), n, _ptr(x), x.shape[1], _ptr(y0), y0.shape[1],
                              len(seg_slot), _ptr(seg_ptr), _ptr(seg_slot), _ptr(rm), _ptr(y), _ptr(v),
                              int(nthreads))
    return y, v


def bgmv(store, x, y0, idx, nthreads=1, mutant=0):
    """Per-row form.  Returns (y fp64 [n, d_out], v fp64 [n, r_max]; NaN where unwritten)."""
    keep = []
    w = _weights(store, keep)
    x, y0 = _rows(x, y0)
    n = x.shape[0]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    y = np.empty((n, store.d_out), dtype=np.float64)
    v = np.full((n, store.r_max), np.nan, dtype=np.float64)
    _load(mutant).oracle_bgmv(ctypes.byref(w), n, _ptr(x), x.shape[1], _ptr(y0), y0.shape[1],
                              _ptr(idx), _ptr(y), _ptr(v), int(nthreads))
    return y, v


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def build_segments(idx, num_slots):
    """Rows grouped by adapter (Punica batch layout construction).

    Returns (row_map, seg_ptr, seg_slot, n_act): segments in ascending slot order,
    rows inside a segment in ascending original index, rows with slot -1 left out.
    Raises ValueError for a slot outside [-1, num_slots).
    """
    idx = [int(s) for s in idx]
    for s in idx:
        if s < -1 or s >= num_slots:
            raise ValueError(f"slot {s} outside [-1, {num_slots})")
    buckets: dict[int, list[int]] = {}
    for row, s in enumerate(idx):
        if s >= 0:
            buckets.setdefault(s, []).append(row)
    row_map, seg_ptr, seg_slot = [], [0], []
    for s in sorted(buckets):
        row_map.extend(buckets[s])
        seg_ptr.append(len(row_map))
        seg_slot.append(s)
    return (np.array(row_map, dtype=np.int32), np.array(seg_ptr, dtype=np.int32),
            np.array(seg_slot, dtype=np.int32), len(row_map))


def check_tiles(tiles, seg_ptr, seg_slot, max_rows):
    """Validate a work-list of tiles (slot, pos0, nrows, seg) against the segments.

    Every position of every segment with slot >= 0 lies in exactly one tile; each tile
    lies inside one segment, carries that segment's slot and has 1..max_rows rows.
    Returns the number of problems found (0 = valid) and a list of messages.
    """
    problems = []
    seen = {}
    for t, (slot, pos0, nrows, seg) in enumerate(np.asarray(tiles).reshape(-1, 4).tolist()):
        if not (0 <= seg < len(seg_slot)):
            problems.append(f"tile {t}: segment {seg} out of range")
            continue
        if slot != seg_slot[seg]:
            problems.append(f"tile {t}: slot {slot} != segment slot {seg_slot[seg]}")
        if not (1 <= nrows <= max_rows):
            problems.append(f"tile {t}: {nrows} rows")
        if pos0 < seg_ptr[seg] or pos0 + nrows > seg_ptr[seg + 1]:
            problems.append(f"tile {t}: rows {pos0}..{pos0 + nrows} outside segment {seg}")
        for p in range(pos0, pos0 + nrows):
            seen[p] = seen.get(p, 0) + 1
    for g in range(len(seg_slot)):
        if seg_slot[g] < 0:
            continue
        for p in range(seg_ptr[g], seg_ptr[g + 1]):
            if seen.get(p, 0) != 1:
                problems.append(f"position {p} covered {seen.get(p, 0)} times")
    for p, c in seen.items():
        if not any(seg_ptr[g] <= p < seg_ptr[g + 1] and seg_slot[g] >= 0 for g in range(len(seg_slot))):
            problems.append(f"position {p} outside active segments")
    return len(problems), problems
