"""CPU reference of the decoder-layer decode step that segmented_gather_matmul_amd.layer
runs on the GPU, for checking the integration of the seven LoRA add-ons.

Every add-on is the fp64 oracle (per-row form) rounded once to fp16; the backbone is
numpy fp64 with an fp16 rounding wherever the GPU step stores an fp16 tensor (norm
outputs, GEMM outputs, attention scores, probabilities and output, the SiLU, the gate
product, residual sums).  Test infrastructure only."""
import math

import numpy as np

import oracle

F16, F64 = np.float16, np.float64
PROJS = ("q", "k", "v", "o", "gate", "up", "down")


def rms_norm(x16, w16, eps):
    x = x16.astype(F64)
    return (x / np.sqrt((x * x).mean(-1, keepdims=True) + eps) * w16.astype(F64)).astype(F16)


def mm16(a16, w16):
    return (a16.astype(F64) @ w16.astype(F64)).astype(F16)


def silu16(g16):
    g = g16.astype(F64)
    return (g / (1.0 + np.exp(-g))).astype(F16)


def lora16(store, x16, y16, idx):
    y_ref, _ = oracle.bgmv(store, x16, y16, idx, nthreads=8)
    return y_ref.astype(F16)


def layer_step(dims, bb, stores, hidden, k_t, v_cache, idx, drop=()):
    """dims = (h, f, heads, head_dim, eps); bb: fp16 numpy backbone weights (keys as in the
    GPU layer); stores: proj -> oracle store; k_t/v_cache: fp16 caches, updated in place at
    the last position; drop: projections whose add-on is left out (to show what a check
    against this reference detects).  Returns the seven projections' outputs and 'out'."""
    h, f, H, dh, eps = dims
    n = hidden.shape[0]
    outs = {}

    def add(p, x, y):
        outs[p] = y if p in drop else lora16(stores[p], x, y, idx)
        return outs[p]

    a = rms_norm(hidden, bb["norm1"], eps)
    qkv = mm16(a, bb["w_qkv"])
    q, k, v = (add(p, a, np.ascontiguousarray(qkv[:, i * h:(i + 1) * h])) for i, p in enumerate(("q", "k", "v")))
    k_t[:, :, :, -1] = k.reshape(n, H, dh)
    v_cache[:, :, -1, :] = v.reshape(n, H, dh)
    scores = (q.astype(F64).reshape(n, H, 1, dh) @ k_t.astype(F64)).astype(F16)
    z = scores.astype(F64) / math.sqrt(dh)
    z = np.exp(z - z.max(-1, keepdims=True))
    probs = (z / z.sum(-1, keepdims=True)).astype(F16)
    attn = (probs.astype(F64) @ v_cache.astype(F64)).astype(F16).reshape(n, h)
    o = add("o", attn, mm16(attn, bb["w_o"]))
    h1 = (hidden.astype(F64) + o.astype(F64)).astype(F16)
    a2 = rms_norm(h1, bb["norm2"], eps)
    gu = mm16(a2, bb["w_gu"])
    g = add("gate", a2, np.ascontiguousarray(gu[:, :f]))
    u = add("up", a2, np.ascontiguousarray(gu[:, f:]))
    act = (silu16(g).astype(F64) * u.astype(F64)).astype(F16)
    d = add("down", act, mm16(act, bb["w_d"]))
    outs["out"] = (h1.astype(F64) + d.astype(F64)).astype(F16)
    return outs


def rel_fro(got, want):
    g, w = got.astype(F64), want.astype(F64)
    return float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300))


# ------------------------------------------------------------------ seeded cases
CASES = {
    # name: (hidden, ffn, heads, seq_len, rows, slot ranks, r_max, cfg id)
    "tiny": (512, 1376, 4, 40, 13, (16, 0, 8, 64, 3), 64, 40),
    "7b": (4096, 11008, 32, 64, 4, (16, 16, 16, 16), 16, 41),
}


def make_case(name):
    """Seeded inputs of one layer step: backbone weights, adapter stores, hidden state,
    caches and row -> slot ids (drawn with the shared workload generators)."""
    from segmented_gather_matmul_amd import workloads as wl
    h, f, H, seq, n, ranks, r_max, cfg = CASES[name]
    dh = h // H
    rank = np.asarray(ranks, dtype=np.int32)
    S = len(rank)
    scale = wl.scale_for_rank(rank)
    dims = {"q": (h, h), "k": (h, h), "v": (h, h), "o": (h, h), "gate": (h, f), "up": (h, f), "down": (f, h)}
    stores = {p: wl.dense_store(cfg, wl.PROJ_IDS[p], S, di, do, rank, scale, r_max=r_max)
              for p, (di, do) in dims.items()}
    w = lambda k, shape: wl.normal16(wl.rng_for(cfg, 7, k), shape)
    bb = dict(w_qkv=w(0, (h, 3 * h)), w_o=w(1, (h, h)), w_gu=w(2, (h, 2 * f)), w_d=w(3, (f, h)),
              norm1=(1.0 + 5.0 * w(4, (h,)).astype(F64)).astype(F16),
              norm2=(1.0 + 5.0 * w(5, (h,)).astype(F64)).astype(F16))
    unit = lambda k, shape: wl.rng_for(cfg, 8, k).standard_normal(shape).astype(F16)
    hidden = unit(0, (n, h))
    k_t, v_cache = unit(1, (n, H, dh, seq)), unit(2, (n, H, seq, dh))
    idx = wl.rng_for(cfg, 0).integers(-1, S, size=n).astype(np.int32)
    return dict(dims=(h, f, H, dh, 1e-5), bb=bb, stores=stores, hidden=hidden, k_t=k_t, v_cache=v_cache, idx=idx,
                rank=rank, scale=scale)


def reference(case, drop=()):
    return layer_step(case["dims"], case["bb"], case["stores"], case["hidden"], case["k_t"].copy(),
                      case["v_cache"].copy(), case["idx"], drop)
