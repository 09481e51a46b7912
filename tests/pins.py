"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check returns None when it holds and a message when it fails, so the same
suite runs against the oracle (every check must hold) and against deliberately
broken builds of it (at least one check must fail).

Independent sources used:
  * exact rational arithmetic (fractions.Fraction) on tiny inputs: fp16 values and
    fp32 scales are dyadic rationals, so the add-on has an exact value;
  * numpy fp64 routines (einsum / matmul) at larger sizes;
  * the pages' identities: merged weight x(W + sAB) - xW = s(xA)B, an identical-adapter
    batch is one dense product, (xA)B = x(AB), rows without adapter are unchanged;
  * a closed form: all-ones x, A and B give y = y0 + s*r*d_in.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle
from segmented_gather_matmul_amd import workloads as wl


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def _dense_mats(store, s):
    r = int(store.rank[s])
    return store.a_t[s, :r].astype(np.float64), store.b[s, :r].astype(np.float64)


def exact_rows(x, y0, idx, rank, scale, mats):
    """Exact y for every row: y0 + scale * (x A) B in rational arithmetic."""
    n, d_out = y0.shape
    out = np.empty((n, d_out), dtype=np.float64)
    for i in range(n):
        s = int(idx[i])
        y0r = [Fraction(float(t)) for t in y0[i]]
        if s < 0 or int(rank[s]) == 0:
            out[i] = [float(t) for t in y0r]
            continue
        a_t, b = mats[s]
        xr = [Fraction(float(t)) for t in x[i]]
        v = [sum((xr[k] * Fraction(float(a_t[j][k])) for k in range(len(xr))), Fraction(0))
             for j in range(int(rank[s]))]
        sc = Fraction(float(np.float32(scale[s])))
        for c in range(d_out):
            acc = sum((v[j] * Fraction(float(b[j][c])) for j in range(len(v))), Fraction(0))
            out[i, c] = float(y0r[c] + sc * acc)
    return out


def _tiny_case(seed, n=7, d_in=48, d_out=40, num_slots=5, page_elems=8):
    rng = np.random.default_rng([99, seed])
    rank = np.array([3, 0, 4, 1, 2], dtype=np.int32)[:num_slots]
    scale = wl.scale_for_rank(rank)
    idx = rng.integers(-1, num_slots, size=n).astype(np.int32)
    idx[0], idx[1] = 2, -1
    x, y0 = wl.activations(90 + seed, 0, n, d_in, d_out)
    dense = wl.dense_store(90 + seed, 0, num_slots, d_in, d_out, rank, scale, r_max=4)
    paged = wl.paged_store(90 + seed, 0, num_slots, d_in, d_out, rank, scale, page_elems, spare_pages=3)
    mats = {s: wl.slot_matrices(90 + seed, 0, s, int(rank[s]), d_in, d_out) for s in range(num_slots)
            if rank[s] > 0}
    return x, y0, idx, rank, scale, dense, paged, mats


def check_exact_bgmv(mutant=0):
    for seed in range(3):
        x, y0, idx, rank, scale, dense, paged, mats = _tiny_case(seed)
        exact = exact_rows(x, y0, idx, rank, scale, mats)
        for store in (dense, paged):
            y, _ = oracle.bgmv(store, x, y0, idx, mutant=mutant)
            e = _rel(y, exact)
            if not e <= 1e-12:
                return f"bgmv vs exact rational (seed {seed}, {type(store).__name__}): rel err {e:.3g}"
    return None


def check_exact_sgmv(mutant=0):
    for seed in range(3):
        x, y0, idx, rank, scale, dense, paged, mats = _tiny_case(seed)
        row_map, seg_ptr, seg_slot, _ = oracle.build_segments(idx, len(rank))
        exact = exact_rows(x, y0, idx, rank, scale, mats)
        for store in (dense, paged):
            y, _ = oracle.sgmv(store, x, y0, seg_ptr, seg_slot, row_map, mutant=mutant)
            e = _rel(y, exact)
            if not e <= 1e-12:
                return f"sgmv vs exact rational (seed {seed}, {type(store).__name__}): rel err {e:.3g}"
    return None


def check_exact_v(mutant=0):
    """The shrink output v alone, exactly (the pages' v = xA)."""
    x, y0, idx, rank, scale, dense, paged, mats = _tiny_case(0)
    _, v = oracle.bgmv(dense, x, y0, idx, mutant=mutant)
    for i in range(len(idx)):
        s = int(idx[i])
        if s < 0 or rank[s] == 0:
            if not np.all(np.isnan(v[i])):
                return f"v row {i} written for a row without adapter"
            continue
        a_t, _ = mats[s]
        xr = [Fraction(float(t)) for t in x[i]]
        for j in range(4):
            want = 0.0 if j >= rank[s] else float(sum(xr[k] * Fraction(float(a_t[j][k])) for k in range(len(xr))))
            if abs(v[i, j] - want) > 1e-12 * max(abs(want), 1e-6):
                return f"v[{i},{j}] = {v[i, j]!r}, exact {want!r}"
    return None


def check_numpy_einsum(mutant=0):
    """Decode shape at full width against numpy fp64 einsum (a library routine)."""
    n, d_in, d_out, S = 6, 4096, 1024, 6
    rank = np.array([16, 8, 16, 4, 16, 2], dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    idx = np.array([0, 3, 5, -1, 1, 2], dtype=np.int32)
    x, y0 = wl.activations(77, 1, n, d_in, d_out)
    store = wl.dense_store(77, 1, S, d_in, d_out, rank, scale)
    y, _ = oracle.bgmv(store, x, y0, idx, mutant=mutant)
    want = y0.astype(np.float64)
    for i, s in enumerate(idx):
        if s < 0:
            continue
        a_t, b = _dense_mats(store, s)
        v = np.einsum("k,jk->j", x[i].astype(np.float64), a_t)
        want[i] += float(scale[s]) * np.einsum("j,jc->c", v, b)
    e = _rel(y - y0, want - y0)
    return None if e <= 1e-12 else f"vs numpy einsum: rel err of the add-on {e:.3g}"


def check_merged_identity(mutant=0):
    """x (W + s A B) - x W equals the unmerged add-on s (x A) B (zero base output)."""
    n, d_in, d_out, S = 5, 256, 192, 3
    rank = np.array([8, 16, 4], dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    idx = np.array([1, 0, 2, 1, -1], dtype=np.int32)
    x, _ = wl.activations(55, 0, n, d_in, d_out)
    y0 = np.zeros((n, d_out), dtype=np.float16)
    store = wl.dense_store(55, 0, S, d_in, d_out, rank, scale)
    W = np.random.default_rng(5).standard_normal((d_in, d_out))
    y, _ = oracle.bgmv(store, x, y0, idx, mutant=mutant)
    for i, s in enumerate(idx):
        xi = x[i].astype(np.float64)
        if s < 0:
            want = np.zeros(d_out)
        else:
            a_t, b = _dense_mats(store, s)
            merged = W + float(scale[s]) * (a_t.T @ b)
            want = xi @ merged - xi @ W
        if np.abs(y[i] - want).max() > 1e-9 * max(np.abs(xi @ W).max(), 1.0):
            return f"merged identity fails on row {i}"
    return None


def check_identical_is_gemm(mutant=0):
    """An all-one-adapter batch is one dense product Y0 + s X A B (with -1 rows untouched)."""
    n, d_in, d_out, S = 12, 512, 320, 4
    rank = np.full(S, 8, dtype=np.int32)
    scale = wl.scale_for_rank(rank)
    idx = np.zeros(n, dtype=np.int32)
    idx[[3, 7]] = -1
    x, y0 = wl.activations(66, 2, n, d_in, d_out)
    store = wl.dense_store(66, 2, S, d_in, d_out, rank, scale)
    a_t, b = _dense_mats(store, 0)
    want = y0.astype(np.float64)
    act = idx >= 0
    want[act] += float(scale[0]) * (x[act].astype(np.float64) @ a_t.T) @ b
    y, _ = oracle.bgmv(store, x, y0, idx, mutant=mutant)
    e = _rel(y - y0, want - y0)
    return None if e <= 1e-12 else f"identical batch vs one GEMM: rel err {e:.3g}"


def check_factorisation(mutant=0):
    """(x A) B equals x (A B), the un-factorised product."""
    n, d_in, d_out, S = 4, 384, 256, 2
    rank = np.array([16, 12], dtype=np.int32)
    scale = np.array([1.0, 0.25], dtype=np.float32)
    idx = np.array([0, 1, 1, 0], dtype=np.int32)
    x, y0 = wl.activations(44, 3, n, d_in, d_out)
    store = wl.dense_store(44, 3, S, d_in, d_out, rank, scale)
    y, _ = oracle.bgmv(store, x, y0, idx, mutant=mutant)
    for i, s in enumerate(idx):
        a_t, b = _dense_mats(store, s)
        want = y0[i].astype(np.float64) + float(scale[s]) * (x[i].astype(np.float64) @ (a_t.T @ b))
        if _rel(y[i] - y0[i], want - y0[i]) > 1e-12:
            return f"(xA)B != x(AB) on row {i}"
    return None


def check_ones_closed_form(mutant=0):
    """All-ones x, A and B: v_j = d_in and y = y0 + s * r * d_in."""
    n, d_in, d_out, S = 3, 64, 32, 2
    rank = np.array([4, 2], dtype=np.int32)
    scale = np.array([0.5, 2.0], dtype=np.float32)
    store = wl.dense_store(1, 0, S, d_in, d_out, rank, scale)
    for s in range(S):
        store.a_t[s, :rank[s]] = 1.0
        store.b[s, :rank[s]] = 1.0
    x = np.ones((n, d_in), dtype=np.float16)
    y0 = np.full((n, d_out), 0.25, dtype=np.float16)
    idx = np.array([0, 1, -1], dtype=np.int32)
    y, v = oracle.bgmv(store, x, y0, idx, mutant=mutant)
    for i, s in enumerate(idx):
        want = 0.25 + (float(scale[s]) * int(rank[s]) * d_in if s >= 0 else 0.0)
        if not np.all(y[i] == want):
            return f"ones closed form row {i}: {y[i][:3]} != {want}"
    return None


def check_noop_rows(mutant=0):
    """Rows with slot -1, rows of a rank-0 slot and empty segments leave y bit-identical."""
    x, y0, idx, rank, scale, dense, paged, mats = _tiny_case(1)
    y, _ = oracle.bgmv(dense, x, y0, idx, mutant=mutant)
    for i, s in enumerate(idx):
        if (s < 0 or rank[s] == 0) and not np.array_equal(y[i], y0[i].astype(np.float64)):
            return f"row {i} (slot {s}) changed"
    seg_ptr = np.array([0, 0, 2, 2], dtype=np.int32)   # empty, two rows of slot 2, empty
    seg_slot = np.array([0, 2, 4], dtype=np.int32)
    y, _ = oracle.sgmv(dense, x, y0, seg_ptr, seg_slot, mutant=mutant)
    if not np.array_equal(y[2:], y0[2:].astype(np.float64)):
        return "rows outside every segment changed"
    return None


CHECKS = [check_exact_bgmv, check_exact_sgmv, check_exact_v, check_numpy_einsum, check_merged_identity,
          check_identical_is_gemm, check_factorisation, check_ones_closed_form, check_noop_rows]


def failures(mutant=0):
    out = []
    for chk in CHECKS:
        msg = chk(mutant)
        if msg is not None:
            out.append(f"{chk.__name__}: {msg}")
    return out
