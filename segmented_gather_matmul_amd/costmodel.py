"""Algorithmic cost of the multi-LoRA add-on: bytes and flops per launch, and the
pages' own counting formulas.

Nothing here runs the method; these are the counts a roofline is priced with.

Per adapted projection with n_act active rows, d_in -> d_out, distinct slots D
(each read once), rank r_s per slot, v held in fp32 with row stride r_max:

  shrink bytes = 2 * sum_{s in D} r_s*d_in  + 2*n_act*d_in  + 4*n_act*r_max
                 (A^T once per distinct slot, x read, v written)
  expand bytes = 2 * sum_{s in D} r_s*d_out + 4*n_act*d_out + 4*n_act*r_max
                 (B once per distinct slot, y read + written, v read)
  flops        = 2 * sum_{active rows} r_row * (d_in + d_out)

A launch that serves several projections sharing one x (q/k/v, gate/up) reads x
once; bench.py counts it once per launch.  Nothing the method avoids is counted
(no padding to r_max, no gathered weight copies, no merged d_in x d_out matrix).
"""
from __future__ import annotations

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
FP32_VECTOR_PEAK_TFLOPS = 157.3


def _distinct_ranks(idx, rank):
    idx = np.asarray(idx)
    slots = np.unique(idx[idx >= 0])
    r = np.asarray(rank)[slots] if len(slots) else np.zeros(0, dtype=np.int64)
    return slots, r[r > 0].astype(np.int64)


def _active_ranks(idx, rank):
    idx = np.asarray(idx)
    act = idx[idx >= 0]
    r = np.asarray(rank)[act].astype(np.int64) if len(act) else np.zeros(0, dtype=np.int64)
    return r[r > 0]


def active_rows(idx, rank):
    """Rows with an adapter slot of rank > 0."""
    return len(_active_ranks(idx, rank))


def shrink_bytes(idx, rank, d_in, r_max):
    _, rd = _distinct_ranks(idx, rank)
    n_act = len(_active_ranks(idx, rank))
    return int(2 * rd.sum() * d_in + 2 * n_act * d_in + 4 * n_act * r_max)


def expand_bytes(idx, rank, d_out, r_max):
    _, rd = _distinct_ranks(idx, rank)
    n_act = len(_active_ranks(idx, rank))
    return int(2 * rd.sum() * d_out + 4 * n_act * d_out + 4 * n_act * r_max)


def op_bytes(idx, rank, d_in, d_out, r_max):
    return shrink_bytes(idx, rank, d_in, r_max) + expand_bytes(idx, rank, d_out, r_max)


def shrink_flops(idx, rank, d_in):
    return int(2 * _active_ranks(idx, rank).sum() * d_in)


def expand_flops(idx, rank, d_out):
    return int(2 * _active_ranks(idx, rank).sum() * d_out)


def op_flops(idx, rank, d_in, d_out):
    return shrink_flops(idx, rank, d_in) + expand_flops(idx, rank, d_out)


# ------------------------------------------------------------------ the pages' own formulas
def lora_pair_params(d_in, d_out, r):
    """Parameters of one A (d_in x r) plus B (r x d_out) pair: r * (d_in + d_out)."""
    return int(r) * (int(d_in) + int(d_out))


def adapter_params(shapes, r, layers):
    """Parameters of an adapter over `layers` layers, one A/B pair per listed projection."""
    return int(layers) * sum(lora_pair_params(di, do, r) for di, do in shapes)


def op_flops_per_token(d_in, d_out, r):
    """Operations of the factorised product (x A) B for one token: 2 r (d_in + d_out)."""
    return 2 * int(r) * (int(d_in) + int(d_out))


def punica_intensity(s_n, n, h_i, h_o):
    """Punica's roofline intensity: FLOP / I/O with 2 flops per MAC and 2-byte elements.

    I = s_n*h_i*h_o*2 / ((s_n*(h_i + h_o) + n*h_i*h_o) * 2).  It counts inputs,
    outputs and the n distinct weight matrices once; it does not count the read of
    the output that the in-place add performs.
    """
    return (s_n * h_i * h_o * 2) / ((s_n * (h_i + h_o) + n * h_i * h_o) * 2)


def gather_bmm_extra_elems(s_n, h_i, h_o):
    """Extra elements Gather-BMM moves over SGMV: it writes s_n weight copies and reads them back."""
    return 2 * int(s_n) * int(h_i) * int(h_o)


def decode_extra_bytes(distinct, adapter_bytes):
    """Decode byte model: extra traffic per step = distinct adapters x adapter bytes."""
    return int(distinct) * float(adapter_bytes)


def slora_pages_per_adapter(layers, matrices_per_layer, r):
    """S-LoRA unified paging: every adapted matrix pair uses r pages for A and r for B."""
    return int(layers) * int(matrices_per_layer) * 2 * int(r)


def layer_bytes_flops(shapes, idx, rank, r_max):
    """Sum over the projections of one layer: (bytes, flops)."""
    b = sum(op_bytes(idx, rank, di, do, r_max) for di, do in shapes)
    f = sum(op_flops(idx, rank, di, do) for di, do in shapes)
    return b, f
