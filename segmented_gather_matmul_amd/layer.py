"""Decode step of a Llama-2 decoder layer with LoRA add-ons on all seven projections.

The backbone (RMSNorm, the dense projections, attention over a key/value cache, SiLU
gating, residual adds) runs in PyTorch on the GPU; every LoRA add-on runs in this
library's kernels, in place on the backbone's fp16 outputs.  Each layer has seven
add-ons (q, k, v, o, gate, up, down), and one metadata build per batch serves all of
them in every layer: the device row -> slot ids of the per-row form, or the tile
work-list and row map of the segment form built once on the host from those ids
(Punica paper digest, 5.2-5.3: seven add-ons per layer, one segment tensor per batch).

q/k/v come from one backbone GEMM against a [h, 3h] weight and gate/up from one against
[h, 2f]; their add-ons land in column slices of that output through the row-stride
argument (ldy = 3h or 2f).  q/k/v share one call over three projections (same x), and
gate/up another, so a layer makes four add-on calls, each one launch (in the segment
form, for tiles of fewer than 8 rows).  Optionally each shrink runs on a second stream
while the backbone GEMM of the same input runs, so only the expands stay on the layer's
critical path.

Left out of the step on purpose: rotary position embedding (elementwise on q and k) and
sampling.  The current token's k and v are written into the last position of the cache,
so attention spans `seq_len` positions including it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import binding as B

PROJS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class LlamaShape:
    name: str
    hidden: int
    ffn: int
    heads: int
    head_dim: int = 128
    eps: float = 1e-5


LLAMA2_7B = LlamaShape("llama2-7b", 4096, 11008, 32)
LLAMA2_13B = LlamaShape("llama2-13b", 5120, 13824, 40)
SHAPES = {"7b": LLAMA2_7B, "13b": LLAMA2_13B}


def proj_dims(shape: LlamaShape) -> dict:
    """(d_in, d_out) of each adapted projection."""
    h, f = shape.hidden, shape.ffn
    return {"q": (h, h), "k": (h, h), "v": (h, h), "o": (h, h), "gate": (h, f), "up": (h, f), "down": (f, h)}


def backbone_bytes(shape: LlamaShape) -> int:
    """fp16 bytes of one layer's backbone weights (projections and the two norm vectors)."""
    h, f = shape.hidden, shape.ffn
    return 2 * (4 * h * h + 3 * h * f + 2 * h)


class BatchMeta:
    """Per-batch metadata shared by every add-on of every layer.

    form "bgmv": the row -> slot ids on the device (-1 = no adapter), read by the per-row
    kernels.  form "sgmv": in addition the segments the host builder makes from the same
    ids (rows grouped by slot through a row map) and their tile work-list, copied to the
    device once."""

    def __init__(self, idx, num_slots, form="bgmv", device="cuda"):
        import torch
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        if form not in ("bgmv", "sgmv"):
            raise ValueError(f"unknown form {form!r}")
        self.n, self.form, self.num_slots = len(idx), form, int(num_slots)
        self.idx = torch.from_numpy(idx).to(device)
        self.segs = None
        if form == "sgmv":
            row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(idx, num_slots)
            tiles = B.lora_build_tiles(seg_ptr, seg_slot)
            self.segs = B.segments_to_device(tiles, row_map, n_act, device)


class KVCache:
    """One layer's cache for n sequences of seq_len positions: keys stored transposed
    ([n, heads, head_dim, seq_len]) so both attention products read contiguous operands,
    values as [n, heads, seq_len, head_dim]."""

    def __init__(self, k_t, v):
        self.k_t, self.v = k_t, v
        self.n, self.heads, self.head_dim, self.seq_len = k_t.shape

    @classmethod
    def random(cls, shape: LlamaShape, n, seq_len, gen, device="cuda"):
        import torch
        kt = torch.randn((n, shape.heads, shape.head_dim, seq_len), generator=gen, device=device).half()
        v = torch.randn((n, shape.heads, seq_len, shape.head_dim), generator=gen, device=device).half()
        return cls(kt, v)


class LoraDecoderLayer:
    """One decoder layer: backbone weights and the seven projections' adapter stores.

    backbone: dict of fp16 device tensors w_qkv [h, 3h], w_o [h, h], w_gu [h, 2f],
    w_d [f, h] (all applied as x @ W), norm1 [h], norm2 [h].
    adapters: proj -> (a_t [S, r_max, d_in], b [S, r_max, d_out]) fp16 device tensors.
    rank (int32 [S]) and scale (fp32 [S]) are the slots' ranks and scales, shared by the
    seven projections.  max_rows bounds the batch (it sizes the v buffers).  Each add-on call
    hands v from the shrink's workgroups to the expand's in one launch (handoff, through a
    workspace the layer owns; the segment form does so for tiles of fewer than 8 rows);
    with handoff False, each call makes a shrink and an expand launch.  overlap:
    each shrink runs on a second stream (default priority) concurrently with the backbone
    GEMM of its projections, the expand after that GEMM.  The results are the same bits
    in every case."""

    def __init__(self, shape: LlamaShape, backbone: dict, adapters: dict, rank, scale, max_rows, overlap=False,
                 handoff=True):
        import torch
        self.shape = shape
        self.side = torch.cuda.Stream(device=rank.device) if overlap else None
        self.work = B.handoff_workspace(max_rows, rank.device) if handoff and not overlap else None
        self.bb = backbone
        num_slots, r_max = adapters["q"][0].shape[:2]
        self.num_slots, self.r_max = int(num_slots), int(r_max)
        dims = proj_dims(shape)
        self.w = {}
        for p in PROJS:
            a_t, b = adapters[p]
            d_in, d_out = dims[p]
            if tuple(a_t.shape) != (num_slots, r_max, d_in) or tuple(b.shape) != (num_slots, r_max, d_out):
                raise ValueError(f"{p}: adapter shapes {tuple(a_t.shape)}, {tuple(b.shape)}")
            self.w[p] = B.Weights(num_slots=self.num_slots, d_in=d_in, d_out=d_out, r_max=self.r_max, rank=rank,
                                  scale=scale, a_t=a_t, b=b)
        ldv = -(-self.r_max // 4) * 4
        self.v = {p: torch.empty((max_rows, ldv), dtype=torch.float32, device=rank.device) for p in PROJS}
        self.max_rows = int(max_rows)

    def _items(self, names, outs, n):
        return [(self.w[p], self.v[p][:n], y) for p, y in zip(names, outs)]

    def _shrink(self, meta: BatchMeta, x, names):
        items = self._items(names, [None] * len(names), x.shape[0])
        if meta.form == "bgmv":
            B.lora_bgmv_shrink_multi(x, meta.idx, items)
        else:
            B.lora_sgmv_shrink_multi(x, meta.segs, items)

    def _expand(self, meta: BatchMeta, names, outs, n):
        items = self._items(names, outs, n)
        if meta.form == "bgmv":
            B.lora_bgmv_expand_multi(meta.idx, items, n)
        else:
            B.lora_sgmv_expand_multi(meta.segs, items, n)

    def _project(self, meta: BatchMeta | None, x, w, names, widths):
        """x @ w, then the add-ons of the projections `names` (all reading x) on the column
        slices of the product (`widths` wide).  With overlap, the shrink runs on a second
        stream while the backbone GEMM runs, and the expand follows the GEMM."""
        import torch
        n = x.shape[0]
        side = self.side if meta is not None and self.side is not None else None
        if side is not None:
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                self._shrink(meta, x, names)
        y = torch.mm(x, w)
        outs, c = [], 0
        for wd in widths:
            outs.append(y[:, c:c + wd])
            c += wd
        if side is not None:
            cur.wait_stream(side)
            self._expand(meta, names, outs, n)
        elif meta is not None:
            items = self._items(names, outs, n)
            if meta.form == "bgmv" and self.work is not None:
                B.lora_bgmv_multi_handoff(x, meta.idx, items, self.work)
            elif meta.form == "bgmv":
                B.lora_bgmv_multi(x, meta.idx, items)
            elif self.work is not None:
                B.lora_sgmv_multi_handoff(x, meta.segs, items, n, self.work)
            else:
                B.lora_sgmv_shrink_multi(x, meta.segs, items)
                B.lora_sgmv_expand_multi(meta.segs, items, n)
        return outs

    def forward(self, hidden, cache: KVCache, meta: BatchMeta | None, trace: dict | None = None):
        """hidden [n, h] fp16 -> [n, h] fp16.  meta None runs the backbone alone.  trace, if
        given, receives copies of the seven projections' outputs after their add-ons."""
        import torch
        import torch.nn.functional as F
        s, bb = self.shape, self.bb
        h, f, H, dh = s.hidden, s.ffn, s.heads, s.head_dim
        n = hidden.shape[0]
        if n > self.max_rows or cache.n != n or cache.heads != H or cache.head_dim != dh:
            raise ValueError(f"batch of {n} rows does not fit this layer or cache")
        if meta is not None and meta.n != n:
            raise ValueError(f"metadata for {meta.n} rows, batch of {n}")

        a = F.rms_norm(hidden, (h,), bb["norm1"], s.eps)
        q, k, v = self._project(meta, a, bb["w_qkv"], ("q", "k", "v"), (h, h, h))
        cache.k_t[:, :, :, -1] = k.view(n, H, dh)
        cache.v[:, :, -1, :] = v.view(n, H, dh)
        S = cache.seq_len
        scores = torch.bmm(q.reshape(n * H, 1, dh), cache.k_t.view(n * H, dh, S))
        probs = torch.softmax(scores.float() * (1.0 / math.sqrt(dh)), dim=-1).half()
        attn = torch.bmm(probs, cache.v.view(n * H, S, dh)).view(n, h)
        (o,) = self._project(meta, attn, bb["w_o"], ("o",), (h,))
        h1 = hidden + o
        a2 = F.rms_norm(h1, (h,), bb["norm2"], s.eps)
        g, u = self._project(meta, a2, bb["w_gu"], ("gate", "up"), (f, f))
        act = F.silu(g) * u
        (d,) = self._project(meta, act, bb["w_d"], ("down",), (h,))
        if trace is not None:
            for name, t in zip(PROJS, (q, k, v, o, g, u, d)):
                trace[name] = t.clone()
        return h1 + d


def random_layer(shape: LlamaShape, num_slots, rank, max_rows, gen, device="cuda", overlap=False, handoff=True):
    """A layer with N(0, 0.02) fp16 backbone and adapter weights drawn on the device, every
    slot of rank `rank` with scale 32 / rank."""
    import torch

    def rnd(*sh):
        return (torch.randn(sh, generator=gen, device=device) * 0.02).half()

    h, f = shape.hidden, shape.ffn
    bb = dict(w_qkv=rnd(h, 3 * h), w_o=rnd(h, h), w_gu=rnd(h, 2 * f), w_d=rnd(f, h),
              norm1=torch.ones(h, dtype=torch.float16, device=device),
              norm2=torch.ones(h, dtype=torch.float16, device=device))
    ads = {p: (rnd(num_slots, rank, di), rnd(num_slots, rank, do)) for p, (di, do) in proj_dims(shape).items()}
    rank_t = torch.full((num_slots,), rank, dtype=torch.int32, device=device)
    scale_t = torch.full((num_slots,), 32.0 / rank, dtype=torch.float32, device=device)
    return LoraDecoderLayer(shape, bb, ads, rank_t, scale_t, max_rows, overlap=overlap, handoff=handoff)
