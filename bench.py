#!/usr/bin/env python3
"""Benchmark of the multi-LoRA add-on (SGMV/BGMV shrink + expand) on one MI355X.

Default workload: Llama-2-7B decode, batch 32, every row its own rank-16 adapter
(32 slots, scale 2.0), all 7 adapted projections of all 32 layers
(q/k/v/o 4096->4096, gate/up 4096->11008, down 11008->4096).  One step = one decode
step's LoRA work for the whole model: 32 x 7 x (shrink + expand) launches in the
per-row-slot (BGMV) form, captured once in a HIP graph and replayed.  Each layer has
its own adapter weights (2.6 GB in total), so every step reads them from HBM rather
than from the 256 MB Infinity Cache.  Inputs are seeded synthetic fp16 N(0, 0.02),
generated on the GPU before the timed region.

Prints one JSON line: metric, value (algorithmic GB/s of the whole step), us_per_layer,
TFLOP/s, the roofline of the dominant kernel (durations from HIP events attached to
every launch of that kernel, on its stream), and the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGMV shrink+expand µs/layer, GB/s & TFLOP/s vs roofline at bs=32 decode"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workloads
def workload_spec(name, rows=None):
    from segmented_gather_matmul_amd import workloads as wl
    if rows is not None and name != "decode_distinct_7b":
        raise SystemExit("--rows applies to decode_distinct_7b only")
    if name == "decode_distinct_7b":
        n = 32 if rows is None else int(rows)
        S = max(32, n)
        b = wl.batch_decode_distinct(n)
        return dict(cfg_id=2, shapes=wl.LLAMA2_7B, layers=32, num_slots=S, rank=np.full(S, 16, np.int32),
                    scale=np.full(S, 2.0, np.float32), batch=b, form="bgmv", layout="dense",
                    model="Llama-2-7B", popularity="distinct")
    if name.startswith("decode_") and name.endswith("_13b"):
        pop = name.split("_")[1]
        b = wl.batch_decode_mix(pop)
        return dict(cfg_id=3, shapes=wl.LLAMA2_13B, layers=40, num_slots=16, rank=np.full(16, 64, np.int32),
                    scale=np.full(16, 0.5, np.float32), batch=b, form="sgmv", layout="dense",
                    model="Llama-2-13B", popularity=pop)
    if name == "prefill_7b":
        b = wl.batch_prefill()
        return dict(cfg_id=4, shapes=wl.LLAMA2_7B, layers=4, num_slots=16, rank=np.full(16, 16, np.int32),
                    scale=np.full(16, 2.0, np.float32), batch=b, form="sgmv_contiguous", layout="dense",
                    model="Llama-2-7B", popularity="distinct")
    if name in ("paged_70b", "paged_70b_tp8", "paged_70b_tp8_slora"):
        rank = wl.paged_ranks(2000)
        b = wl.batch_paged_zipf(256, 2000)
        tp8 = "tp8" in name
        slora = name.endswith("slora")
        spec = dict(cfg_id=5, shapes=wl.LLAMA2_70B_TP8 if tp8 else wl.LLAMA2_70B, layers=2, num_slots=2000,
                    rank=rank, scale=wl.scale_for_rank(rank), batch=b, form="sgmv", layout="paged",
                    page_elems=128 if tp8 else 1024, model="Llama-2-70B, one GPU of 8-way TP" if tp8 else "Llama-2-70B",
                    popularity="zipf1.2")
        if slora:
            # A of the column-parallel projections split by rank columns over the 8 GPUs
            # (S-LoRA's partition): this GPU's shrink covers ceil(r / 8) rank-rows of the
            # full-width input; the expand still reads all r (after the all-gather of v,
            # which one GPU leaves out) into its d_out / 8 columns
            spec["shrink_rank"] = {p: (rank + 7) // 8 for p in ("q", "k", "v", "gate", "up")}
            spec["model"] = "Llama-2-70B, one GPU of 8-way TP, A split by rank columns"
        return spec
    raise SystemExit(f"unknown workload {name}")


class Op:
    """One adapted projection of one layer: its weights, activations and launch metadata."""


# Projections of a layer that read the same input (one x tensor, one launch when grouped).
INPUT_GROUPS = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def make_ops(spec, layers, device, tile_rows=None, expand_tile_rows=None):
    """Per layer: one x per input group, one y, v and weight descriptor per projection.
    With expand_tile_rows the expand launches get a tile list of their own (the shrink
    keeps tile_rows): the tile height is a launch shape, the results do not depend on it
    beyond the tolerance."""
    import torch
    from segmented_gather_matmul_amd import binding as B
    b = spec["batch"]
    n, S, rank = b.n, spec["num_slots"], spec["rank"]
    r_max = int(rank.max())
    idx_d = torch.from_numpy(b.idx.astype(np.int32)).to(device)
    segs = segs_e = None
    if spec["form"].startswith("sgmv") or spec["form"] == "mixed":
        if spec["form"] in ("sgmv", "mixed"):
            row_map, seg_ptr, seg_slot, n_act = B.lora_build_segments(b.idx, S)
            n_pos = n_act
        else:
            row_map, seg_ptr, seg_slot, n_pos = None, b.seg_ptr, b.seg_slot, n
        segs = B.segments_to_device(B.lora_build_tiles(seg_ptr, seg_slot, tile_rows), row_map, n_pos, device)
        segs_e = segs
        if expand_tile_rows is None and tile_rows is None:
            expand_tile_rows = B.lora_pick_expand_tile_rows(seg_ptr)
        if expand_tile_rows and expand_tile_rows != (tile_rows or B.lora_pick_tile_rows(seg_ptr)):
            segs_e = B.segments_to_device(B.lora_build_tiles(seg_ptr, seg_slot, expand_tile_rows), row_map, n_pos,
                                          device)
        spec["expand_tile_rows"] = int(expand_tile_rows or tile_rows or B.lora_pick_tile_rows(seg_ptr))
    rank_d = torch.from_numpy(rank.astype(np.int32)).to(device)
    scale_d = torch.from_numpy(spec["scale"].astype(np.float32)).to(device)
    gen = torch.Generator(device=device)
    names = list(spec["shapes"])
    ldv = max(4, -(-r_max // 4) * 4)
    groups = []
    for layer in range(layers):
        for grp in INPUT_GROUPS:
            gen.manual_seed(spec["cfg_id"] * 1_000_003 + layer * 101 + 50 + names.index(grp[0]))
            d_in = spec["shapes"][grp[0]][0]
            x = (torch.randn(n, d_in, generator=gen, device=device, dtype=torch.float32) * 0.02).half()
            ops = []
            for pname in grp:
                d_in_p, d_out = spec["shapes"][pname]
                assert d_in_p == d_in
                pid = names.index(pname)
                gen.manual_seed(spec["cfg_id"] * 1_000_003 + layer * 101 + pid)

                def rnd(*shape):
                    return (torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * 0.02).half()

                op = Op()
                op.layer, op.proj, op.d_in, op.d_out = layer, pname, d_in, d_out
                op.x = x
                op.y = rnd(n, d_out)
                if spec["layout"] == "dense":
                    op.w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=r_max, rank=rank_d, scale=scale_d,
                                     a_t=rnd(S, r_max, d_in), b=rnd(S, r_max, d_out))
                else:
                    from segmented_gather_matmul_amd import workloads as wl
                    P = spec["page_elems"]
                    pt, a_off, b_off, num_pages = wl.page_placement(spec["cfg_id"], layer * 7 + pid, rank, d_in,
                                                                    d_out, P)
                    pool = torch.empty((num_pages, P), dtype=torch.float16, device=device)
                    for c0 in range(0, num_pages, 1 << 20):
                        c1 = min(num_pages, c0 + (1 << 20))
                        pool[c0:c1] = rnd(c1 - c0, P)
                    op.w = B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=r_max, rank=rank_d,
                                     scale=scale_d, pool=pool, page_elems=P,
                                     page_table=torch.from_numpy(pt).to(device),
                                     a_pt_off=torch.from_numpy(a_off).to(device),
                                     b_pt_off=torch.from_numpy(b_off).to(device))
                op.ws, op.shrink_rank = op.w, None
                if pname in spec.get("shrink_rank", {}):
                    # this GPU's rank-column shard of A: its own pages (each shard rank-row
                    # carries one page of B that no kernel reads, as the descriptor wants both)
                    from segmented_gather_matmul_amd import workloads as wl
                    P = spec["page_elems"]
                    rs = spec["shrink_rank"][pname]
                    pt, a_off, b_off, num_pages = wl.page_placement(spec["cfg_id"], 100 + layer * 7 + pid, rs, d_in,
                                                                    P, P)
                    pool_s = rnd(num_pages, P)
                    op.ws = B.Weights(num_slots=S, d_in=d_in, d_out=P, r_max=int(rs.max()),
                                      rank=torch.from_numpy(rs.astype(np.int32)).to(device), scale=scale_d,
                                      pool=pool_s, page_elems=P, page_table=torch.from_numpy(pt).to(device),
                                      a_pt_off=torch.from_numpy(a_off).to(device),
                                      b_pt_off=torch.from_numpy(b_off).to(device))
                    op.shrink_rank = rs
                op.v = torch.zeros((n, ldv), dtype=torch.float32, device=device)
                op.idx, op.segs, op.segs_e = idx_d, segs, segs_e
                op.expand_per_row = spec["form"] == "mixed"
                ops.append(op)
            groups.append(ops)
    return groups


def launch_unit(kind, ops):
    """One launch over `ops` (projections sharing x): kind is "shrink", "expand" or
    "handoff" (both steps in one launch, v handed from the shrink's workgroups to the
    expand's)."""
    from segmented_gather_matmul_amd import binding as B
    op0 = ops[0]
    items = [(op.ws if kind == "shrink" else op.w, op.v, op.y) for op in ops]
    n = op0.x.shape[0]
    if kind == "handoff" and op0.segs is None:
        B.lora_bgmv_multi_handoff(op0.x, op0.idx, items, op0.work)
    elif kind == "handoff":
        B.lora_sgmv_multi_handoff(op0.x, op0.segs, items, n, op0.work)
    elif op0.segs is None:
        if kind == "shrink":
            B.lora_bgmv_shrink_multi(op0.x, op0.idx, items)
        else:
            B.lora_bgmv_expand_multi(op0.idx, items, n)
    elif kind == "shrink":
        B.lora_sgmv_shrink_multi(op0.x, op0.segs, items)
    elif op0.expand_per_row:
        B.lora_bgmv_expand_multi(op0.idx, items, n)
    else:
        B.lora_sgmv_expand_multi(op0.segs_e, items, n)


def launches(groups, grouped, handoff=False):
    """(kind, ops) of every launch of one step, in order.  With handoff each unit of the
    per-row or segment form is one hand-off launch."""
    out = []
    for ops in groups:
        units = [ops] if grouped else [[op] for op in ops]
        for u in units:
            if handoff and any(op.shrink_rank is not None for op in u):
                raise SystemExit("the one-launch forms read one weight descriptor; this workload's shrink has its own")
            if handoff and not u[0].expand_per_row:
                out.append(("handoff", u))
            else:
                out += [("shrink", u), ("expand", u)]
    return out


def step(plan):
    for kind, ops in plan:
        launch_unit(kind, ops)


# ------------------------------------------------------------------ HIP events (raw handles)
class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def kernel_durations(plan, steps):
    """Duration of every launch, from event pairs attached to the launches themselves
    (hipExtLaunchKernel records start and stop on the launch stream)."""
    from segmented_gather_matmul_amd import binding as B
    import torch
    ev = HipEvents()
    recs = []
    for _ in range(steps):
        for kind, u in plan:
            e0, e1 = ev.create(), ev.create()
            B.lora_set_launch_events(e0, e1)
            launch_unit(kind, u)
            recs.append((kind, u, e0, e1))
    torch.cuda.synchronize()
    out = {}
    for k, u, e0, e1 in recs:
        out.setdefault(k, []).append((u, ev.elapsed_ms(e0, e1)))
        ev.destroy(e0)
        ev.destroy(e1)
    return out


def reference_floors(plan, spec, steps):
    """Context for the roofline, timed like the step (graph replay, events around the
    replays): the same number of launches (a) doing nothing (an empty spin kernel) and
    (b) each a plain device copy moving the bytes of the launch it stands for (half
    read, half written; distinct buffers, so the copies stream from HBM as the step
    does)."""
    import torch
    sizes = [unit_counts(spec, u)[f"{k}_bytes"] for k, u in plan]
    bufs = [(torch.empty(b // 4 + 1, dtype=torch.float16, device="cuda"),
             torch.empty(b // 4 + 1, dtype=torch.float16, device="cuda")) for b in sizes]
    out = {"launches": len(plan)}
    for name, body in (("empty", lambda: [torch.cuda._sleep(0) for _ in plan]),
                       ("copy", lambda: [d.copy_(s_) for s_, d in bufs])):
        body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[f"{name}_ms_per_step"] = round(e0.elapsed_time(e1) / steps, 5)
        del g
    moved = sum(2 * (b // 4 + 1) * 2 for b in sizes)
    out["copy_bytes_per_step"] = moved
    out["copy_gbs"] = round(moved / (out["copy_ms_per_step"] * 1e-3) / 1e9, 1)
    out["copy_frac_of_peak"] = round(out["copy_gbs"] / 8000.0, 4)
    del bufs
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ accounting
def unit_counts(spec, ops):
    """Algorithmic bytes/flops of one launch over `ops` (projections sharing one x):
    the shared x is read once; each projection adds its adapters, v and y traffic."""
    from segmented_gather_matmul_amd import costmodel as cm
    idx, rank, r_max = spec["batch"].idx, spec["rank"], int(spec["rank"].max())
    n_act = int(cm.active_rows(idx, rank))
    x_bytes = 2 * n_act * ops[0].d_in
    srank = [rank if getattr(o, "shrink_rank", None) is None else o.shrink_rank for o in ops]
    sb = x_bytes + sum(cm.shrink_bytes(idx, sr, o.d_in, int(sr.max())) - x_bytes for o, sr in zip(ops, srank))
    eb = sum(cm.expand_bytes(idx, rank, o.d_out, r_max) for o in ops)
    sf = sum(cm.shrink_flops(idx, sr, o.d_in) for o, sr in zip(ops, srank))
    ef = sum(cm.expand_flops(idx, rank, o.d_out) for o in ops)
    return dict(shrink_bytes=sb, expand_bytes=eb, shrink_flops=sf, expand_flops=ef,
                handoff_bytes=sb + eb, handoff_flops=sf + ef)


def kernel_source_sha():
    p = os.path.join(ROOT, "segmented_gather_matmul_amd", "csrc", "lora_kernels.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profile(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernels."""
    p = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo, as lscpu reports it), its logical CPU
    count and the CPUs this process may run on."""
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    return dict(model=model, cpu_count=os.cpu_count(), available=len(os.sched_getaffinity(0)))


def cpu_baseline(spec, groups, budget_s=10.0):
    """The CPU oracle, as it is, on the same step: whole layers in order, repeated until
    about budget_s seconds of oracle time have run (inputs copied to host beforehand),
    once with OpenMP over all the CPUs this process may use and once on one core."""
    import oracle
    from segmented_gather_matmul_amd import workloads as wl
    if spec["layout"] != "dense":
        return None
    cpu = host_cpu()
    cores = cpu["available"]
    b = spec["batch"]
    S, rank, scale = spec["num_slots"], spec["rank"], spec["scale"]
    r_max = int(rank.max())
    host = []
    for ops in groups:
        x = ops[0].x.cpu().numpy()
        c = unit_counts(spec, ops)
        stores = [(wl.DenseStore(S, op.d_in, op.d_out, r_max, rank, scale, op.w.tensors[2].cpu().numpy(),
                                 op.w.tensors[3].cpu().numpy()), op.y.cpu().numpy()) for op in ops]
        host.append((ops[0].layer, x, stores, c["shrink_bytes"] + c["expand_bytes"]))
    if spec["form"] != "bgmv":
        rm, sp, ss, _ = oracle.build_segments(b.idx, S)
    n_layers = len(set(h[0] for h in host))

    def timed(threads, budget):
        t_total, bytes_total, layers_done = 0.0, 0, 0
        while t_total < budget:
            for lay in range(n_layers):
                for _, x, stores, nbytes in (h for h in host if h[0] == lay):
                    t0 = time.perf_counter()
                    for store, y0 in stores:
                        if spec["form"] == "bgmv":
                            oracle.bgmv(store, x, y0, b.idx, nthreads=threads)
                        else:
                            oracle.sgmv(store, x, y0, sp, ss, rm, nthreads=threads)
                    t_total += time.perf_counter() - t0
                    bytes_total += nbytes
                layers_done += 1
                if t_total >= budget:
                    break
        return t_total, bytes_total, layers_done

    t_total, bytes_total, layers_done = timed(cores, budget_s)
    t1, b1, l1 = timed(1, budget_s / 2)
    rows = b.n
    return dict(value=round(bytes_total / t_total / 1e9, 4), unit="GB/s", cores=cores, kind="oracle",
                us_per_layer=round(1e6 * t_total / layers_done, 1), cpu_model=cpu["model"],
                cpu_count=cpu["cpu_count"], cpus_available=cores,
                sample=f"{layers_done} layer passes over the {n_layers} layers x {len(spec['shapes'])} projections "
                       f"of the step ({rows} rows each), fp64 C loops with OpenMP over rows on all {cores} available "
                       f"CPUs (at most {rows} busy, one per row), {t_total:.1f} s",
                single_core=dict(value=round(b1 / t1 / 1e9, 4), unit="GB/s", cores=1,
                                 us_per_layer=round(1e6 * t1 / l1, 1),
                                 sample=f"{l1} layer passes, one thread, {t1:.1f} s"))


# ------------------------------------------------------------------ operator sweep
def sweep_assign(pop, n, seed):
    """Row -> adapter of the pages' popularity sweep, rows grouped by adapter (segment order):
    distinct (one adapter per row), uniform (ceil(sqrt n) adapters, uniform draw), skewed
    (Zipf s = 1.5 over n adapters), identical (one adapter)."""
    from segmented_gather_matmul_amd import workloads as wl
    rng = wl.rng_for(6, 0, seed)
    if pop == "distinct":
        idx = wl.assign_distinct(n)
    elif pop == "identical":
        idx = wl.assign_identical(n)
    elif pop == "uniform":
        idx = wl.assign_uniform(rng, n, int(np.ceil(np.sqrt(n))))
    else:
        idx = wl.assign_zipf(rng, n, n, 1.5)
    return np.sort(idx).astype(np.int32)


def operator_sweep(args):
    """One LoRA operator (shrink + expand, h -> r -> h) per configuration, timed for six
    implementations on the same inputs: this library's segment form (one shrink and one
    expand launch over contiguous segments) and per-row form, each also in its one-launch
    hand-off form, a loop over adapters (two fp16 GEMMs and an add per segment) and
    Gather-BMM (per-row copies of A and B, then two batched products).  Each implementation's L layers (distinct weights, so the adapters
    stream from HBM) are captured in one graph and replayed; the result is us per operator.
    The last two are plain PyTorch, timing context only."""
    import torch
    from segmented_gather_matmul_amd import binding as B
    h, L, K = args.sweep_h, args.sweep_layers or 16, args.steps
    ns = [int(v) for v in (args.sweep_batches or "1,2,4,8,16,32,64").split(",")]
    rs = [int(v) for v in args.sweep_ranks.split(",")]
    pops = args.sweep_pops.split(",")
    dev = "cuda"
    gen = torch.Generator(device=dev)
    results = []
    for r in rs:
        for pop in pops:
            for n in ns:
                idx = sweep_assign(pop, n, n * 100 + r)
                S = int(idx.max()) + 1
                seg_slot, counts = np.unique(idx, return_counts=True)
                seg_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
                seg_slot = seg_slot.astype(np.int32)
                tiles = B.lora_build_tiles(seg_ptr, seg_slot)
                segs = B.segments_to_device(tiles, None, n, dev)
                idx_d = torch.from_numpy(idx).to(dev)
                idx_l = idx_d.long()
                scale = 32.0 / r
                rank_d = torch.full((S,), r, dtype=torch.int32, device=dev)
                scale_d = torch.full((S,), scale, dtype=torch.float32, device=dev)
                gen.manual_seed(n * 7919 + r * 31 + len(pop))
                rnd = lambda *sh: (torch.randn(*sh, generator=gen, device=dev, dtype=torch.float32) * 0.02).half()
                layers = []
                for _ in range(L):
                    a_t, b = rnd(S, r, h), rnd(S, r, h)
                    lay = dict(x=rnd(n, h), y=rnd(n, h), a_t=a_t, b=b, a=a_t.transpose(1, 2).contiguous(),
                               v=torch.zeros((n, max(4, -(-r // 4) * 4)), dtype=torch.float32, device=dev))
                    lay["w"] = B.Weights(num_slots=S, d_in=h, d_out=h, r_max=r, rank=rank_d, scale=scale_d, a_t=a_t,
                                         b=b)
                    layers.append(lay)

                def ours_sgmv(lay, y):
                    B.lora_sgmv_shrink(lay["v"], lay["x"], lay["w"], segs)
                    B.lora_sgmv_expand(y, lay["v"], lay["w"], segs)

                def ours_bgmv(lay, y):
                    B.lora_bgmv(y, lay["x"], idx_d, lay["w"], lay["v"])

                work = B.handoff_workspace(n, dev)

                def ours_sgmv_handoff(lay, y):
                    B.lora_sgmv_multi_handoff(lay["x"], segs, [(lay["w"], lay["v"], y)], n, work)

                def ours_bgmv_handoff(lay, y):
                    B.lora_bgmv_multi_handoff(lay["x"], idx_d, [(lay["w"], lay["v"], y)], work)

                def loop(lay, y):
                    for g in range(len(seg_slot)):
                        a0, a1, s_ = int(seg_ptr[g]), int(seg_ptr[g + 1]), int(seg_slot[g])
                        y[a0:a1].add_((lay["x"][a0:a1] @ lay["a"][s_]) @ lay["b"][s_], alpha=scale)

                def gather_bmm(lay, y):
                    ag = lay["a"].index_select(0, idx_l).contiguous()
                    bg = lay["b"].index_select(0, idx_l).contiguous()
                    vv = torch.bmm(lay["x"].unsqueeze(1), ag)
                    y.add_(torch.bmm(vv, bg).squeeze(1), alpha=scale)

                impls = dict(ours_sgmv=ours_sgmv, ours_bgmv=ours_bgmv, ours_sgmv_handoff=ours_sgmv_handoff,
                             ours_bgmv_handoff=ours_bgmv_handoff, loop=loop, gather_bmm=gather_bmm)
                rec = dict(h=h, r=r, popularity=pop, n=n, adapters=len(seg_slot))
                # the same result from each, on a fresh copy of layer 0's y
                outs = {}
                for name, fn in impls.items():
                    y = layers[0]["y"].clone()
                    fn(layers[0], y)
                    outs[name] = y.float()
                torch.cuda.synchronize()
                ref = outs["gather_bmm"]
                rec["max_abs_vs_gather_bmm"] = {k: float((v - ref).abs().max()) for k, v in outs.items()}
                for name, fn in impls.items():
                    fn(layers[0], layers[0]["y"])
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for lay in layers:
                            fn(lay, lay["y"])
                    for _ in range(3):
                        g.replay()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(K):
                        g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    rec[f"{name}_us"] = round(1e3 * e0.elapsed_time(e1) / (K * L), 3)
                    del g
                log(f"[sweep] r={r} {pop} n={n}: " + " ".join(f"{k}={rec[k + '_us']}" for k in impls))
                results.append(rec)
                del layers
                torch.cuda.empty_cache()
    print(json.dumps({"sweep": "operator", "h": h, "layers": L, "steps": K, "results": results}), flush=True)


# ------------------------------------------------------------------ adapter loading
def load_sweep(args):
    """Loading adapters into one paged pool (lora_pool_load: one host-to-device copy of a
    page-locked blob, one scatter kernel on a small fixed grid).  A Llama-2-7B adapter set (32 layers x 7
    projections, rank 16, 256-element pages) per model; `--sweep-batches` models per call.
    Reported next to a plain host-to-device copy of the same blob (the link's rate) and to
    the 7B decode step's time with and without a load running on a side stream."""
    import torch
    from segmented_gather_matmul_amd import binding as B
    from segmented_gather_matmul_amd import workloads as wl
    dev, P, r = "cuda", 256, 16
    shapes = wl.LLAMA2_7B
    layers = 32
    out = {"sweep": "load", "model": "Llama-2-7B", "rank": r, "page_elems": P, "layers": layers, "results": []}
    # the decode step, to see what a concurrent load costs it
    spec = workload_spec("decode_distinct_7b")
    groups = make_ops(spec, spec["layers"], dev)
    work = B.handoff_workspace(spec["batch"].n, dev)   # the bench default: one hand-off launch per unit
    for ops in groups:
        for op in ops:
            op.work = work
    plan = launches(groups, True, handoff=True)
    step(plan)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(plan)
    side = torch.cuda.Stream()
    for models in [int(v) for v in (args.sweep_batches or "1,2,4").split(",")]:
        per_model_pages = layers * sum(r * (di // P + do // P) for di, do in shapes.values())
        num_pages = models * per_model_pages
        pool = torch.empty((num_pages, P), dtype=torch.float16, device=dev)
        rank_t = torch.zeros(models, dtype=torch.int32, device=dev)
        scale_t = torch.zeros(models, dtype=torch.float32, device=dev)
        st = B.PoolState(num_pages)
        targets = []
        for layer in range(layers):
            for name, (di, do) in shapes.items():
                cap = r * (di // P + do // P)
                w = B.Weights(num_slots=models, d_in=di, d_out=do, r_max=r, rank=rank_t, scale=scale_t, pool=pool,
                              page_elems=P, page_table=torch.zeros(models * cap, dtype=torch.int32, device=dev),
                              a_pt_off=torch.zeros(models, dtype=torch.int64, device=dev),
                              b_pt_off=torch.zeros(models, dtype=torch.int64, device=dev))
                targets.append((w, cap, di, do))
        rng = np.random.default_rng(models)
        ads = []
        for m in range(models):
            for w, cap, di, do in targets:
                ads.append(dict(w=w, slot=m, rank=r, scale=2.0, pt_off=m * cap,
                                a_t=(rng.standard_normal((r, di), dtype=np.float32) * 0.02).astype(np.float16),
                                b=(rng.standard_normal((r, do), dtype=np.float32) * 0.02).astype(np.float16),
                                pages=st.alloc(r * (di // P + do // P))))
        blob, jobs = B.pack_adapters(ads, pinned=True)
        staging = torch.empty(blob.numel(), dtype=torch.uint8, device=dev)
        weight_bytes = sum(2 * r * (di + do) for _, _, di, do in targets) * models

        def timed(fn, reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(side):
                fn()
                e0.record(side)
                for _ in range(reps):
                    fn()
                e1.record(side)
            side.synchronize()
            return e0.elapsed_time(e1) / reps

        load_ms = timed(lambda: B.lora_pool_load(jobs, blob, staging, stream=side), 5)
        copy_ms = timed(lambda: staging.copy_(blob, non_blocking=True), 5)
        # decode step alone, then with loads running on the side stream meanwhile
        reps = 20
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / reps
        def step_during(fn, per_ms):
            """Decode step time while `fn` runs back to back on the side stream.  The side
            work is queued first (twice what the replays take, since some of it runs while
            the host is still queueing) and the timed window opens after it, so that the
            host's own time in `fn` (argument checks, the job table) is not counted as a
            slower decode step."""
            with torch.cuda.stream(side):
                for _ in range(max(2, int(2 * reps * step_ms / max(per_ms, 1e-3)) + 1)):
                    fn()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            side.synchronize()
            return e0.elapsed_time(e1) / reps

        step_ms_loaded = step_during(lambda: B.lora_pool_load(jobs, blob, staging, stream=side), load_ms)
        step_ms_copies = step_during(lambda: staging.copy_(blob, non_blocking=True), copy_ms)
        # the same copies, each followed by a trivial kernel on the side stream (a 4 KiB fill)
        tiny = torch.empty(1024, dtype=torch.int32, device=dev)
        step_ms_copies_kernel = step_during(lambda: (staging.copy_(blob, non_blocking=True), tiny.fill_(1)), copy_ms)

        def step_paced(fn, every):
            """Decode step time in a host loop that keeps at most two steps queued (it waits
            for step i-1 once step i is queued) and issues `fn` on the side stream after
            every `every`-th step, so loads start as the decode reaches them and never queue
            behind one another (fn=None: the same loop without loads)."""
            evs = [torch.cuda.Event() for _ in range(reps)]
            e0.record()
            for i in range(reps):
                g.replay()
                evs[i].record()
                if i >= 1:
                    evs[i - 1].synchronize()
                if fn is not None and i % every == 0:
                    with torch.cuda.stream(side):
                        fn()
            e1.record()
            torch.cuda.synchronize()
            side.synchronize()
            return e0.elapsed_time(e1) / reps

        every = int(np.ceil(load_ms / step_ms)) + 1
        step_ms_paced_alone = step_paced(None, every)
        step_ms_paced = step_paced(lambda: B.lora_pool_load(jobs, blob, staging, stream=side), every)
        rec = dict(models=models, jobs=len(jobs), weight_bytes=weight_bytes, blob_bytes=int(blob.numel()),
                   load_ms=round(load_ms, 4), load_gbs=round(weight_bytes / (load_ms * 1e-3) / 1e9, 2),
                   ms_per_model=round(load_ms / models, 4), h2d_copy_ms=round(copy_ms, 4),
                   h2d_copy_gbs=round(blob.numel() / (copy_ms * 1e-3) / 1e9, 2),
                   decode_step_ms=round(step_ms, 4), decode_step_ms_during_loads=round(step_ms_loaded, 4),
                   decode_step_ms_during_copies=round(step_ms_copies, 4),
                   decode_step_ms_during_copies_and_fills=round(step_ms_copies_kernel, 4),
                   paced_every_steps=every, decode_step_ms_paced_alone=round(step_ms_paced_alone, 4),
                   decode_step_ms_paced_loads=round(step_ms_paced, 4),
                   paced_load_gbs=round(weight_bytes / (every * step_ms_paced * 1e-3) / 1e9, 2))
        log(f"[load] {rec}")
        out["results"].append(rec)
        del pool, staging, blob, targets, ads
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ serving with an adapter cache
def serve_sweep(args):
    """The 7B decode step (32 rows, 32 distinct rank-16 adapters, every layer and projection
    adapted) served from an AdapterCache over a paged pool: each step's adapters are made
    resident (normally already, by the prefetch), the compute stream waits for any of their
    loads still in flight, the step's graph replays with the step's slots, and the adapters
    of the step `--serve-lookahead` steps ahead are prefetched (their copies on the side
    stream) as soon as it is queued, keeping those of the steps in between.  The host loop
    keeps at most two steps queued (it waits for step i-1 once step i and the prefetch are
    queued).  Every `every` steps `turn` new adapters enter the batch (and `turn` leave),
    each an 80 MB load; turn 0 is the same loop with every adapter resident."""
    import torch
    from segmented_gather_matmul_amd import binding as B
    from segmented_gather_matmul_amd import workloads as wl
    from segmented_gather_matmul_amd.adapters import AdapterCache, HostAdapter, PagedModel
    dev, P, r, n, layers = "cuda", 256, 16, 32, 32
    names = list(wl.LLAMA2_7B)
    shapes = [wl.LLAMA2_7B[p] for _ in range(layers) for p in names]
    universe, slots = 40, 36
    per_adapter = sum(B.lora_pool_pages_for(r, di, do, P) for di, do in shapes)
    model = PagedModel(shapes, slots, r, P, slots * per_adapter, dev)
    rng = np.random.default_rng(7)
    tmpl = {}
    for di, do in set(shapes):
        tmpl[(di, do)] = ((rng.standard_normal((r, di)) * 0.02).astype(np.float16),
                          (rng.standard_normal((r, do)) * 0.02).astype(np.float16))
    store = {k: HostAdapter(model, r, 2.0, [tmpl[sh][0] for sh in shapes], [tmpl[sh][1] for sh in shapes])
             for k in range(universe)}
    weight_bytes = 2 * r * sum(di + do for di, do in shapes)
    # the step: per layer, shrink + expand per input group, per-row form, one idx for all
    idx_d = torch.full((n,), -1, dtype=torch.int32, device=dev)
    # page-locked slots per step, a ring: a step's copy may still be queued when the host
    # writes the next step's
    idx_ring = [torch.full((n,), -1, dtype=torch.int32, pin_memory=True) for _ in range(4)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    units = []
    for layer in range(layers):
        for grp in INPUT_GROUPS:
            d_in = wl.LLAMA2_7B[grp[0]][0]
            x = (torch.randn(n, d_in, generator=gen, device=dev) * 0.02).half()
            items = []
            for pname in grp:
                w = model.targets[layer * len(names) + names.index(pname)]
                y = (torch.randn(n, w.d_out, generator=gen, device=dev) * 0.02).half()
                v = torch.zeros((n, r), dtype=torch.float32, device=dev)
                items.append((w, v, y))
            units.append((x, items))

    def step():
        for x, items in units:
            B.lora_bgmv_shrink_multi(x, idx_d, items)
            B.lora_bgmv_expand_multi(idx_d, items, n)

    def batch(i, turn, every):
        # turn new adapters every `every` steps, spread over the steps (turn > every: one
        # or two new adapters at each step)
        base = (i * turn) // every
        return [(base + j) % universe for j in range(n)]

    cache = AdapterCache(model, store, max_side=args.serve_side_streams)
    first, ready = cache.ensure(batch(0, 0, 1))
    torch.cuda.synchronize()
    idx_d.copy_(torch.from_numpy(first))
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    cur = torch.cuda.current_stream()
    out = {"sweep": "serve", "model": "Llama-2-7B", "rows": n, "rank": r, "layers": layers, "page_elems": P,
           "side_streams": args.serve_side_streams,
           "universe": universe, "slots": slots, "adapter_bytes": weight_bytes, "results": []}
    reps = args.steps
    configs = [tuple(int(v) for v in c.split(":")) for c in args.serve_configs.split(",")]
    L = max(1, args.serve_lookahead)
    out["lookahead_steps"] = L
    for turn, every in configs:
        late0 = cache.late
        evs = [torch.cuda.Event() for _ in range(reps + 8)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_pf = t_wait = 0.0
        for i in range(reps + 8):
            if i == 8:
                e0.record(cur)
                l8 = cache.loads
            keys = batch(i, turn, every)
            keep = [k for j in range(1, L) for k in batch(i + j, turn, every)]
            sl, ready = cache.ensure(keys, keep)
            for e in ready:
                cur.wait_event(e)
            idx_h = idx_ring[i % len(idx_ring)]
            idx_h.copy_(torch.from_numpy(sl))
            idx_d.copy_(idx_h, non_blocking=True)
            g.replay()
            cache.mark_used(keys, cur)
            evs[i].record(cur)
            # step i+L's adapters as soon as this step is queued: issued after the host
            # waited for step i-1 instead, a load started well into step i and step i+1
            # waited for it (1 load every 2 steps: +36 % instead of +8 %)
            t0 = time.perf_counter()
            cache.prefetch(batch(i + L, turn, every), keep)
            t1 = time.perf_counter()
            if i >= 1:
                evs[i - 1].synchronize()
            if i >= 8:
                t_pf += t1 - t0
                t_wait += time.perf_counter() - t1
        e1.record(cur)
        torch.cuda.synchronize()
        for side in cache.sides:
            side.synchronize()
        ms = e0.elapsed_time(e1) / reps
        loads = cache.loads - l8
        rec = dict(turn=turn, every=every, step_ms=round(ms, 4), loads=loads,
                   loads_per_step=round(loads / reps, 3),
                   load_gbs_over_loop=round(loads * weight_bytes / (reps * ms * 1e-3) / 1e9, 2),
                   host_prefetch_ms_per_step=round(1e3 * t_pf / reps, 4),
                   host_wait_ms_per_step=round(1e3 * t_wait / reps, 4),
                   late_batches=cache.late - late0)
        log(f"[serve] {rec}")
        out["results"].append(rec)
    # reference: the same loop with every adapter resident and, each k-th step, a plain
    # host-to-device copy of one adapter's bytes on the side stream into scratch memory
    hsrc = torch.empty(weight_bytes, dtype=torch.uint8, pin_memory=True)
    dscratch = torch.empty(weight_bytes, dtype=torch.uint8, device=dev)
    for every in ((2, 1) if args.serve_copies else ()):
        keys = batch(0, 0, 1)
        evs = [torch.cuda.Event() for _ in range(reps + 8)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(reps + 8):
            if i == 8:
                e0.record(cur)
            g.replay()
            evs[i].record(cur)
            if i % every == 0:
                with torch.cuda.stream(cache.side):
                    dscratch.copy_(hsrc, non_blocking=True)
            if i >= 1:
                evs[i - 1].synchronize()
        e1.record(cur)
        torch.cuda.synchronize()
        cache.side.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rec = dict(turn=0, every=every, plain_copies=True, step_ms=round(ms, 4),
                   copy_gbs_over_loop=round(weight_bytes / every / (ms * 1e-3) / 1e9, 2))
        log(f"[serve] {rec}")
        out["results"].append(rec)
    base = out["results"][0]["step_ms"]
    for rec in out["results"]:
        rec["vs_resident"] = round(rec["step_ms"] / base - 1, 4)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ decoder layer
def layer_sweep(args):
    """Decode step of whole Llama-2 decoder layers (RMSNorm, fused q/k/v GEMM, attention
    over a key/value cache of `seq_len` positions, o GEMM, fused gate/up GEMM, SiLU
    gating, down GEMM, residual adds; PyTorch on the GPU) with the seven LoRA add-ons of
    each layer through this library, one metadata build per batch shared by all of them,
    against the same layers without add-ons.  Each mix runs twice: add-ons after each
    GEMM on one stream, and with each shrink on a second stream overlapping its GEMM
    ("+overlap", same bits).  The layers are chained (each feeds the next), have distinct
    weights and caches so nothing stays cached between layers, are captured in one graph
    and replayed; the result is us per layer.  Rank 16, 32 resident adapters, the
    popularity mixes of the operator sweep."""
    import torch
    from segmented_gather_matmul_amd import costmodel as cm
    from segmented_gather_matmul_amd import layer as LY
    ns = [int(v) for v in (args.sweep_batches or "1,2,4,8,16,32").split(",")]
    seqs = [int(v) for v in args.sweep_seqs.split(",")]
    pops = args.sweep_pops.split(",")
    variants = ["none"] + [p + sfx for p in pops for sfx in ("", "+overlap")]
    L, K, r, slots = args.sweep_layers or 4, args.steps, 16, 32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    side = torch.cuda.Stream()
    out = {"sweep": "layer", "form": args.layer_form, "rank": r,
           "resident_adapters": slots, "layers": L, "steps": K, "results": []}
    for model in args.sweep_models.split(","):
        shape = LY.SHAPES[model]
        log(f"[layer] {shape.name}: drawing {L} layers")
        layers = [LY.random_layer(shape, slots, r, max(ns), gen) for _ in range(L)]
        dims = LY.proj_dims(shape)
        for seq in seqs:
            for n in ns:
                caches = [LY.KVCache.random(shape, n, seq, gen) for _ in range(L)]
                hidden = torch.randn((n, shape.hidden), generator=gen, device="cuda").half()
                rec = dict(model=shape.name, seq_len=seq, n=n)
                metas = {}
                for var in variants:
                    pop, overlap = var.split("+")[0], var.endswith("+overlap")
                    build_us = 0.0
                    if pop == "none":
                        meta, idx = None, None
                    elif pop in metas:
                        meta, idx, build_us = metas[pop]
                    else:
                        idx = sweep_assign(pop, n, n * 100 + r)
                        t0 = time.perf_counter()
                        meta = LY.BatchMeta(idx, slots, args.layer_form)
                        torch.cuda.synchronize()
                        build_us = 1e6 * (time.perf_counter() - t0)
                        metas[pop] = (meta, idx, build_us)
                    for lay in layers:
                        lay.side = side if overlap else None

                    def run():
                        x = hidden
                        for lay, c in zip(layers, caches):
                            x = lay.forward(x, c, meta)
                        return x

                    eager = run().clone()
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        res = run()
                    g.replay()
                    torch.cuda.synchronize()
                    same = bool(torch.equal(res, eager))
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(K):
                        g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    us = 1e3 * e0.elapsed_time(e1) / (K * L)
                    del g, res
                    lora_b = 0 if idx is None else sum(cm.op_bytes(idx, np.full(slots, r), di, do, r)
                                                       for di, do in dims.values())
                    layer_b = LY.backbone_bytes(shape) + 2 * 2 * n * seq * shape.hidden + lora_b
                    rec[var] = dict(us=round(us, 2), lora_bytes=lora_b, gbs=round(layer_b / (us * 1e-6) / 1e9, 1),
                                    graph_equals_eager=same)
                    if pop != "none":
                        rec[var]["meta_build_us"] = round(build_us, 1)
                        rec[var]["overhead_vs_none"] = round(us / rec["none"]["us"] - 1.0, 4)
                if any(not rec[v]["graph_equals_eager"] for v in variants):
                    raise SystemExit(f"graph replay differs from the eager run at {shape.name} seq={seq} n={n}")
                log(f"[layer] {shape.name} seq={seq} n={n}: " + " ".join(f"{v}={rec[v]['us']}" for v in variants))
                out["results"].append(rec)
                del caches
                torch.cuda.empty_cache()
        for lay in layers:
            lay.side = None
        del layers
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_distinct_7b")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--rows", type=int, default=None,
                    help="decode_distinct_7b with this many rows (each its own adapter) instead of 32")
    ap.add_argument("--kernel-steps", type=int, default=5, help="steps of the per-launch event pass")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-group", action="store_true", help="one launch per projection (14 per layer)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile-rows", type=int, default=None,
                    help="tile height for the segment form (default: lora_pick_tile_rows)")
    ap.add_argument("--expand-tile-rows", type=int, default=None,
                    help="segment form: a tile height of its own for the expand launches")
    ap.add_argument("--form", choices=["bgmv", "sgmv", "mixed"], default=None,
                    help="per-row slots (bgmv), rows grouped by adapter (sgmv), or the segment-form shrink with "
                         "the per-row expand (mixed); default: the workload's own")
    ap.add_argument("--handoff", choices=["auto", "on", "off"], default="auto",
                    help="per-row and segment forms: one launch per unit with v handed from the shrink's "
                         "workgroups to the expand's (auto: the per-row form with dense weights, where it measures "
                         "faster than two launches)")
    ap.add_argument("--stream-weights", choices=["auto", "on", "off"], default="auto",
                    help="lora_set_stream_weights: auto = on for the per-row form with dense weights when "
                         "the batch's active rows use distinct adapters")
    ap.add_argument("--no-floors", action="store_true", help="skip the empty-launch and copy reference steps")
    ap.add_argument("--plan", default="0,0", metavar="JW,NR",
                    help="fix rank-rows per VALU shrink workgroup and rows per pass of the segment-form VALU "
                         "kernels (0 = library's choice; results are bit-identical either way)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (byte-counter calibration)")
    ap.add_argument("--sweep", choices=["operator", "load", "layer", "serve"], default=None,
                    help="instead of the step: 'operator' times one LoRA operator across batch sizes, popularity "
                         "and ranks against a loop over adapters and Gather-BMM; 'load' times placing 7B adapter "
                         "sets into a paged pool (--sweep-batches = models per call); 'layer' times whole "
                         "decoder layers with and without the seven add-ons; 'serve' serves the 7B decode step "
                         "from an adapter cache with new adapters prefetched while steps run")
    ap.add_argument("--serve-configs", default="0:1,1:8,1:4,1:2,1:1,9:8,5:4", metavar="TURN:EVERY,...",
                    help="serve sweep: new adapters per change and steps between changes, one loop each")
    ap.add_argument("--serve-copies", type=int, default=1, help="serve sweep: also the plain-copy reference loops")
    ap.add_argument("--serve-lookahead", type=int, default=3,
                    help="serve sweep: the host prefetches the adapters of the batch this many steps ahead")
    ap.add_argument("--serve-side-streams", type=int, default=4,
                    help="serve sweep: most side streams the cache spreads its loads over")
    ap.add_argument("--sweep-h", type=int, default=4096)
    ap.add_argument("--sweep-layers", type=int, default=None, help="layers per graph (operator 16, layer 4)")
    ap.add_argument("--sweep-batches", default=None,
                    help="batch sizes (operator 1..64, layer 1..32) or models per load call (load 1,2,4)")
    ap.add_argument("--sweep-ranks", default="8,16,32,64")
    ap.add_argument("--sweep-pops", default="distinct,uniform,skewed,identical")
    ap.add_argument("--sweep-models", default="7b,13b", help="layer sweep: Llama-2 shapes")
    ap.add_argument("--sweep-seqs", default="512,2048", help="layer sweep: cache lengths")
    ap.add_argument("--layer-form", choices=["bgmv", "sgmv"], default="bgmv",
                    help="layer sweep: add-ons in the per-row or the segment form")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(a batch shards across GPUs by rows without any exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    from segmented_gather_matmul_amd import binding as B
    from segmented_gather_matmul_amd import costmodel as cm
    B.lib()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    if args.sweep == "operator":
        operator_sweep(args)
        return
    if args.sweep == "load":
        load_sweep(args)
        return
    if args.sweep == "layer":
        layer_sweep(args)
        return
    if args.sweep == "serve":
        serve_sweep(args)
        return
    device = "cuda"
    grouped = not args.no_group
    spec = workload_spec(args.workload, args.rows)
    if args.form and args.form != spec["form"].split("_")[0]:
        if spec["form"] == "sgmv_contiguous":
            raise SystemExit("the prefill workload is given as contiguous segments")
        spec["form"] = args.form
    layers = args.layers or spec["layers"]
    B.lora_set_plan(*(int(v) for v in args.plan.split(",")))
    log(f"[bench] workload={args.workload} layers={layers} grouped={grouped} building inputs")
    groups = make_ops(spec, layers, device, args.tile_rows, args.expand_tile_rows)
    torch.cuda.synchronize()
    counts = [unit_counts(spec, ops) for ops in groups]
    step_bytes = sum(c["shrink_bytes"] + c["expand_bytes"] for c in counts)
    step_flops = sum(c["shrink_flops"] + c["expand_flops"] for c in counts)
    decode_form = spec["form"] in ("bgmv", "sgmv")
    if args.handoff == "on" and not decode_form:
        raise SystemExit("--handoff on needs the per-row or segment form (--form bgmv or sgmv)")
    # the library's hand-off form where it measures faster: the per-row form with dense
    # weights (the segment form's two launches are as fast or faster since its expand runs
    # the planned tile in one pass)
    handoff = args.handoff == "on" or (args.handoff == "auto" and spec["form"] == "bgmv" and spec["layout"] == "dense")
    if handoff:
        work = B.handoff_workspace(spec["batch"].n, device)
        for ops in groups:
            for op in ops:
                op.work = work
    # the caller's hint that each row of the per-row form uses its own adapter (dense
    # weights then stream through the caches): on where the batch's active rows carry
    # distinct adapters, as the host that built the batch knows
    act = spec["batch"].idx[spec["batch"].idx >= 0]
    distinct = len(np.unique(act)) == len(act)
    stream_w = args.stream_weights == "on" or (args.stream_weights == "auto" and spec["form"] == "bgmv"
                                               and spec["layout"] == "dense" and distinct)
    B.lora_set_stream_weights(stream_w)
    plan = launches(groups, grouped, handoff)
    n_launch = len(plan)

    log(f"[bench] {n_launch} launches/step, {step_bytes / 1e6:.1f} MB algorithmic per step; warmup {args.warmup}")
    stream = torch.cuda.current_stream()
    if args.no_graph:
        run = lambda: step(plan)
    else:
        step(plan)  # first eager pass (loads kernels)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(plan)
        run = g.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.4f} ms/step (wall {wall_ms:.4f})")

    log(f"[bench] per-launch event pass: {args.kernel_steps} steps")
    kd = kernel_durations(plan, args.kernel_steps)
    per_kernel, totals = {}, {}
    for k in kd:
        recs = kd[k]
        us = np.array([1e3 * t for _, t in recs])
        kb = sum(unit_counts(spec, u)[f"{k}_bytes"] for u, _ in recs)
        kf = sum(unit_counts(spec, u)[f"{k}_flops"] for u, _ in recs)
        totals[k] = float(us.sum())
        per_kernel[k] = dict(launches_per_step=len(recs) // args.kernel_steps, avg_us=round(float(us.mean()), 3),
                             p10_us=round(float(np.percentile(us, 10)), 3),
                             p90_us=round(float(np.percentile(us, 90)), 3), bytes_per_launch=round(kb / len(recs)),
                             gbs=round(kb / (totals[k] * 1e-6) / 1e9, 1),
                             tflops=round(kf / (totals[k] * 1e-6) / 1e12, 3))
    by_shape = {}
    for k in kd:
        for u, t in kd[k]:
            key = f"{k} {'+'.join(o.proj for o in u)} {u[0].d_in}->{'/'.join(str(o.d_out) for o in u)}"
            rec = by_shape.setdefault(key, [0, 0.0, unit_counts(spec, u)[f"{k}_bytes"]])
            rec[0] += 1
            rec[1] += 1e3 * t
    by_shape = {key: dict(avg_us=round(t / n, 3), gbs=round(nb / (t / n * 1e-6) / 1e9, 1))
                for key, (n, t, nb) in by_shape.items()}
    dom = max(per_kernel, key=lambda k: totals[k])
    pk = per_kernel[dom]
    kernel_name = {"shrink": "lora_shrink_kernel", "expand": "lora_expand_kernel",
                   "handoff": "lora_handoff_kernel"}[dom]
    traffic = None if args.rows is not None else traffic_from_profile(args.workload, dom)
    roofline = dict(bound="hbm", achieved=pk["gbs"], peak=cm.HBM_PEAK_GBS, unit="GB/s",
                    frac=round(pk["gbs"] / cm.HBM_PEAK_GBS, 4), traffic=traffic, kernel=kernel_name,
                    avg_launch_us=pk["avg_us"], algorithmic_bytes_per_launch=pk["bytes_per_launch"])

    floors = None
    if not args.no_floors:
        log("[bench] reference steps: empty launches, plain copies of the same bytes")
        floors = reference_floors(plan, spec, min(args.steps, 20))
        floors["step_vs_copy"] = round(floors["copy_ms_per_step"] / ms, 4)  # our speed as a fraction of the copies

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(spec, groups, args.cpu_budget)

    gbs = step_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,0.02) fp16, generated on the GPU)",
        "config": {"workload": args.workload, "model_shapes": spec["model"], "layers": layers,
                   "projections": list(spec["shapes"]), "batch_rows": spec["batch"].n,
                   "num_slots": spec["num_slots"], "rank": sorted(set(int(r) for r in spec["rank"])),
                   "popularity": spec["popularity"], "form": spec["form"], "layout": spec["layout"],
                   "grouped": grouped, "launches_per_step": n_launch, "tile_rows": args.tile_rows,
                   "expand_tile_rows": spec.get("expand_tile_rows"),
                   "handoff": handoff,
                   "stream_weights": bool(stream_w),
                   "plan": args.plan,
                   "graph": not args.no_graph,
                   "parallelism": "none"},
        "us_per_layer": round(1e3 * ms / layers, 3),
        "tflops": round(step_flops / (ms * 1e-3) / 1e12, 4),
        "step_bytes": step_bytes,
        "step_flops": step_flops,
        "hbm_frac_step": round(gbs / cm.HBM_PEAK_GBS, 4),
        "wall_ms_per_step": round(wall_ms, 5),
        "kernels": per_kernel,
        "launch_shapes": by_shape,
        "roofline": roofline,
        "floors": floors,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def reap_children():
    """End any child process still running (the bench starts none that should outlive it)."""
    try:
        import psutil
    except ImportError:
        return
    kids = psutil.Process().children(recursive=True)
    for k in kids:
        try:
            k.terminate()
        except psutil.Error:
            pass
    psutil.wait_procs(kids, timeout=5)


if __name__ == "__main__":
    try:
        main()
    finally:
        reap_children()
