"""Seeded synthetic inputs for the multi-LoRA add-on (shrink v = x.A, expand y += s.v.B).

This module only *draws* inputs: row -> adapter-slot assignments, prompt lengths,
adapter ranks, the physical placement of adapter pages, and fp16 values.  It holds
none of the method's arithmetic, so both the plain CPU oracle and the HIP path can
consume the same inputs without sharing any computation.

Every draw comes from ``numpy.random.default_rng([cfg_id, stream, *keys])`` (PCG64),
so a single adapter slot or projection can be regenerated on its own.

Streams:
  0  assignment (idx, lengths, no-adapter rows, ranks)
  1  x (keys: projection)          2  base y (keys: projection)
  3  A^T of one slot (keys: projection, slot)
  4  B of one slot (keys: projection, slot)
  5  page placement (keys: projection)

Values are N(0, 1) * 0.02 rounded to fp16 (round-to-nearest-even, numpy astype),
the activation/weight distribution stated for the tiny SGMV workload and used for
all workloads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STD = 0.02
# fp16 quiet NaN: written into storage that a correct kernel must never read.
NAN16 = np.uint16(0x7E00)


def rng_for(cfg_id: int, stream: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng([int(cfg_id), int(stream), *[int(k) for k in keys]])


def normal16(rng: np.random.Generator, shape) -> np.ndarray:
    return (rng.standard_normal(shape) * STD).astype(np.float16)


# --------------------------------------------------------------------------- assignments
def assign_distinct(n: int) -> np.ndarray:
    """Row i uses slot i (every request its own adapter)."""
    return np.arange(n, dtype=np.int32)


def assign_identical(n: int, slot: int = 0) -> np.ndarray:
    return np.full(n, slot, dtype=np.int32)


def assign_uniform(rng: np.random.Generator, n: int, num_slots: int) -> np.ndarray:
    return rng.integers(0, num_slots, size=n).astype(np.int32)


def zipf_probs(num_slots: int, s: float) -> np.ndarray:
    """Finite Zipf law p_k proportional to k^-s, k = 1..num_slots; rank k is slot k-1."""
    k = np.arange(1, num_slots + 1, dtype=np.float64)
    p = k ** (-float(s))
    return p / p.sum()


def assign_zipf(rng: np.random.Generator, n: int, num_slots: int, s: float) -> np.ndarray:
    return rng.choice(num_slots, size=n, p=zipf_probs(num_slots, s)).astype(np.int32)


def mask_no_adapter(rng: np.random.Generator, idx: np.ndarray, frac: float) -> np.ndarray:
    """Set exactly round(frac*n) rows, chosen by a seeded permutation, to -1."""
    out = idx.copy()
    m = int(round(frac * len(idx)))
    if m:
        out[rng.permutation(len(idx))[:m]] = -1
    return out


def loguniform_lengths(rng: np.random.Generator, count: int, lo: int, hi: int) -> np.ndarray:
    """Prompt lengths drawn log-uniform in [lo, hi], rounded to the nearest integer."""
    u = rng.uniform(math.log(lo), math.log(hi), size=count)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


def segments_from_lengths(lengths) -> np.ndarray:
    """Offsets s_0 = 0 <= s_1 <= ... <= s_n of contiguous segments."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


# --------------------------------------------------------------------------- adapter storage
@dataclass
class DenseStore:
    """Slot-indexed adapters: a_t[s] is A[s] transposed ([r_max][d_in]), b[s] is [r_max][d_out].

    Rank-rows j >= rank[s] and slots never filled hold fp16 NaN, so any read of them
    by a kernel shows up in the result.
    """
    num_slots: int
    d_in: int
    d_out: int
    r_max: int
    rank: np.ndarray   # int32 [num_slots]
    scale: np.ndarray  # float32 [num_slots]
    a_t: np.ndarray    # float16 [num_slots, r_max, d_in]
    b: np.ndarray      # float16 [num_slots, r_max, d_out]


@dataclass
class PagedStore:
    """Adapters held as fixed-size pages in one pool.

    Each rank-row of A^T (d_in elements) and of B (d_out elements) is cut into
    d/P pages of P elements.  page_table[a_pt_off[s] + j*(d_in/P) + q] is the physical
    page that holds A^T[s][j][q*P:(q+1)*P]; likewise for B with b_pt_off.  Pages not
    owned by a filled slot hold fp16 NaN.
    """
    num_slots: int
    d_in: int
    d_out: int
    r_max: int
    page_elems: int
    rank: np.ndarray        # int32 [num_slots]
    scale: np.ndarray       # float32 [num_slots]
    pool: np.ndarray        # float16 [num_pages, page_elems]
    page_table: np.ndarray  # int32 [entries]
    a_pt_off: np.ndarray    # int64 [num_slots]
    b_pt_off: np.ndarray    # int64 [num_slots]


def slot_matrices(cfg_id: int, proj: int, slot: int, rank: int, d_in: int, d_out: int):
    """The fp16 A^T[slot] ([rank][d_in]) and B[slot] ([rank][d_out]) of one projection."""
    a_t = normal16(rng_for(cfg_id, 3, proj, slot), (rank, d_in))
    b = normal16(rng_for(cfg_id, 4, proj, slot), (rank, d_out))
    return a_t, b


def dense_store(cfg_id, proj, num_slots, d_in, d_out, rank, scale, r_max=None, fill=None) -> DenseStore:
    rank = np.asarray(rank, dtype=np.int32)
    if rank.ndim == 0:
        rank = np.full(num_slots, int(rank), dtype=np.int32)
    scale = np.asarray(scale, dtype=np.float32)
    if scale.ndim == 0:
        scale = np.full(num_slots, float(scale), dtype=np.float32)
    r_max = int(rank.max()) if r_max is None else int(r_max)
    a_t = np.full((num_slots, r_max, d_in), NAN16, dtype=np.uint16).view(np.float16)
    b = np.full((num_slots, r_max, d_out), NAN16, dtype=np.uint16).view(np.float16)
    slots = range(num_slots) if fill is None else sorted(set(int(s) for s in fill if s >= 0))
    for s in slots:
        r = int(rank[s])
        if r:
            a_t[s, :r], b[s, :r] = slot_matrices(cfg_id, proj, s, r, d_in, d_out)
    return DenseStore(num_slots, d_in, d_out, r_max, rank, scale, a_t, b)


def page_placement(cfg_id, proj, rank, d_in, d_out, page_elems, spare_pages=0):
    """Page table and per-slot offsets with pages scattered by a seeded permutation."""
    if d_in % page_elems or d_out % page_elems:
        raise ValueError("page_elems must divide d_in and d_out")
    rank = np.asarray(rank, dtype=np.int64)
    pa, pb = d_in // page_elems, d_out // page_elems
    per_slot = rank * (pa + pb)
    a_pt_off = np.concatenate([[0], np.cumsum(per_slot)[:-1]]).astype(np.int64)
    b_pt_off = (a_pt_off + rank * pa).astype(np.int64)
    entries = int(per_slot.sum())
    num_pages = entries + int(spare_pages)
    perm = rng_for(cfg_id, 5, proj).permutation(num_pages)[:entries].astype(np.int32)
    return perm, a_pt_off, b_pt_off, num_pages


def paged_store(cfg_id, proj, num_slots, d_in, d_out, rank, scale, page_elems,
                fill=None, spare_pages=0) -> PagedStore:
    rank = np.asarray(rank, dtype=np.int32)
    if rank.ndim == 0:
        rank = np.full(num_slots, int(rank), dtype=np.int32)
    scale = np.asarray(scale, dtype=np.float32)
    if scale.ndim == 0:
        scale = np.full(num_slots, float(scale), dtype=np.float32)
    pt, a_off, b_off, num_pages = page_placement(cfg_id, proj, rank, d_in, d_out, page_elems, spare_pages)
    pool = np.full((num_pages, page_elems), NAN16, dtype=np.uint16).view(np.float16)
    pa, pb = d_in // page_elems, d_out // page_elems
    slots = range(num_slots) if fill is None else sorted(set(int(s) for s in fill if s >= 0))
    for s in slots:
        r = int(rank[s])
        if not r:
            continue
        a_t, b = slot_matrices(cfg_id, proj, s, r, d_in, d_out)
        ia = pt[a_off[s]: a_off[s] + r * pa]
        ib = pt[b_off[s]: b_off[s] + r * pb]
        pool[ia] = a_t.reshape(r * pa, page_elems)
        pool[ib] = b.reshape(r * pb, page_elems)
    return PagedStore(num_slots, d_in, d_out, int(rank.max()), page_elems, rank, scale,
                      pool, pt, a_off, b_off)


# --------------------------------------------------------------------------- workloads
# Projection shapes (d_in, d_out) of one transformer layer; index = projection id.
LLAMA2_7B = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
             "gate": (4096, 11008), "up": (4096, 11008), "down": (11008, 4096)}
LLAMA2_13B = {"q": (5120, 5120), "k": (5120, 5120), "v": (5120, 5120), "o": (5120, 5120),
              "gate": (5120, 13824), "up": (5120, 13824), "down": (13824, 5120)}
# 70B with grouped-query attention: k/v project 8192 -> 1024.
LLAMA2_70B = {"q": (8192, 8192), "k": (8192, 1024), "v": (8192, 1024), "o": (8192, 8192),
              "gate": (8192, 28672), "up": (8192, 28672), "down": (28672, 8192)}
# One GPU's shard of 70B under 8-way tensor parallelism: q/k/v/gate/up split by output
# columns, o/down by input rows (their partial products join the base output's sum).
LLAMA2_70B_TP8 = {"q": (8192, 1024), "k": (8192, 128), "v": (8192, 128), "o": (1024, 8192),
                  "gate": (8192, 3584), "up": (8192, 3584), "down": (3584, 8192)}
PROJ_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


@dataclass
class Batch:
    """Row structure of one batch: either per-row slots (idx) or contiguous segments."""
    n: int
    idx: np.ndarray                      # int32 [n], -1 = no adapter (always present)
    seg_ptr: np.ndarray | None = None    # int32 [n_seg+1] when the batch is given as segments
    seg_slot: np.ndarray | None = None   # int32 [n_seg]
    info: dict = field(default_factory=dict)


def batch_tiny_sgmv() -> Batch:
    """8 rows in 4 contiguous segments of sizes [1, 3, 2, 2], slots 0..3."""
    seg_ptr = segments_from_lengths([1, 3, 2, 2])
    seg_slot = np.arange(4, dtype=np.int32)
    idx = np.repeat(seg_slot, np.diff(seg_ptr)).astype(np.int32)
    return Batch(8, idx, seg_ptr, seg_slot)


def batch_decode_distinct(n=32) -> Batch:
    return Batch(n, assign_distinct(n))


def batch_decode_mix(popularity: str, n=64, num_slots=16, none_frac=0.1, zipf_s=1.5, cfg_id=3) -> Batch:
    rng = rng_for(cfg_id, 0, {"uniform": 0, "skewed": 1, "identical": 2}[popularity])
    if popularity == "uniform":
        idx = assign_uniform(rng, n, num_slots)
    elif popularity == "skewed":
        idx = assign_zipf(rng, n, num_slots, zipf_s)
    elif popularity == "identical":
        idx = assign_identical(n)
    else:
        raise ValueError(popularity)
    return Batch(n, mask_no_adapter(rng, idx, none_frac), info={"popularity": popularity})


def batch_prefill(count=16, lo=64, hi=2048, cfg_id=4) -> Batch:
    lengths = loguniform_lengths(rng_for(cfg_id, 0), count, lo, hi)
    seg_ptr = segments_from_lengths(lengths)
    seg_slot = np.arange(count, dtype=np.int32)
    idx = np.repeat(seg_slot, lengths).astype(np.int32)
    return Batch(int(seg_ptr[-1]), idx, seg_ptr, seg_slot, info={"lengths": lengths})


def paged_ranks(num_slots=2000, choices=(8, 16, 32, 64), cfg_id=5) -> np.ndarray:
    return rng_for(cfg_id, 0, 1).choice(np.asarray(choices), size=num_slots).astype(np.int32)


def batch_paged_zipf(n=256, num_slots=2000, zipf_s=1.2, cfg_id=5) -> Batch:
    return Batch(n, assign_zipf(rng_for(cfg_id, 0, 2), n, num_slots, zipf_s))


def activations(cfg_id: int, proj: int, n: int, d_in: int, d_out: int):
    """x [n, d_in] and base y [n, d_out], both fp16 N(0, 0.02)."""
    return normal16(rng_for(cfg_id, 1, proj), (n, d_in)), normal16(rng_for(cfg_id, 2, proj), (n, d_out))


def scale_for_rank(rank, alpha: float = 32.0) -> np.ndarray:
    """scale = alpha / r per slot (alpha = 32); rank-0 slots get scale 0."""
    r = np.asarray(rank, dtype=np.float64)
    return np.where(r > 0, alpha / np.maximum(r, 1), 0.0).astype(np.float32)
