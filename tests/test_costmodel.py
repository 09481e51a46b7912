"""The byte/flop counters against the pages' worked numbers (tests/golden)."""
import json
import os

import numpy as np
import pytest

from segmented_gather_matmul_amd import costmodel as cm
from segmented_gather_matmul_amd import workloads as wl

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")))
E = {e["name"]: e for e in GOLD["entries"]}


def _llama3_8b_shapes(proj=("q", "k", "v", "o", "gate", "up", "down")):
    g = GOLD["llama3_8b_shapes"]
    h, kv = g["hidden"], g["kv_heads"] * g["head_dim"]
    all7 = {"q": (h, h), "k": (h, kv), "v": (h, kv), "o": (h, h),
            "gate": (h, g["mlp"]), "up": (h, g["mlp"]), "down": (g["mlp"], h)}
    return [all7[p] for p in proj], g["layers"]


def _near(got, entry):
    return abs(got - entry["value"]) <= entry["rel_tol"] * abs(entry["value"])


def test_adapter_memory_worked_example():
    shapes, L = _llama3_8b_shapes()
    p16 = cm.adapter_params(shapes, 16, L)
    assert _near(2 * p16, E["llama3_8b_r16_all7_bytes"])
    assert _near(2 * p16, E["llama3_8b_r16_all7_ops_per_token"])  # 2 ops per parameter
    assert _near(2 * cm.adapter_params(shapes, 64, L), E["llama3_8b_r64_all7_bytes"])
    assert _near(16 * 2 * p16, E["sixteen_r16_bytes"])
    assert _near(16 * 2 * cm.adapter_params(shapes, 64, L), E["sixteen_r64_bytes"])
    qv, _ = _llama3_8b_shapes(("q", "v"))
    pqv = cm.adapter_params(qv, 16, L)
    assert pqv == E["llama3_8b_r16_qv_params"]["value"]
    assert _near(2 * pqv, E["llama3_8b_r16_qv_bytes"])


def test_decode_byte_model_table():
    e = E["decode_extra_gb"]
    for distinct, gb, pct in e["rows"]:
        extra = cm.decode_extra_bytes(distinct, e["adapter_bytes"])
        assert round(extra / 1e9, 2) == pytest.approx(gb)
        assert round(100 * extra / e["base_bytes"], 1) == pytest.approx(pct)


def test_slora_counts():
    h, r, L = 4096, 16, 32
    params = cm.adapter_params([(h, h)] * 4, r, L)
    assert _near(params, E["slora_llama7b_r16_params"])
    assert _near(2 * params, E["slora_llama7b_r16_bytes"])
    assert cm.slora_pages_per_adapter(L, 4, r) == E["slora_pages_per_adapter"]["value"]
    assert h * 2 == E["slora_page_bytes"]["value"]
    assert _near(2 * 32 * h * h, E["slora_base_flops_b32"])
    # Printed adapter FLOPs are twice the formula's value: keep the formula.
    e = E["slora_adapter_flops_b32_printed"]
    got = 32 * cm.op_flops_per_token(h, h, r)
    assert got == e["correct"] and got * 2 == pytest.approx(e["value"], rel=0.002)


def test_punica_intensity_properties():
    e = E["punica_expand_intensity_identical_bs64"]
    i_id = cm.punica_intensity(e["s_n"], e["n"], e["h_i"], e["h_o"])
    assert i_id == pytest.approx(64 * 16 * 4096 / (64 * 4112 + 16 * 4096))
    # Distinct (n = s_n): constant in batch size.  Identical (n = 1): grows with batch size.
    d = [cm.punica_intensity(s, s, 16, 4096) for s in (1, 8, 64)]
    assert max(d) - min(d) < 1e-12
    ident = [cm.punica_intensity(s, 1, 16, 4096) for s in (1, 8, 64)]
    assert ident[0] < ident[1] < ident[2]


def test_gather_bmm_extra_io():
    assert cm.gather_bmm_extra_elems(64, 4096, 16) == 2 * 64 * 4096 * 16


def test_counter_matches_byte_formula_for_distinct_decode():
    idx = wl.assign_distinct(32)
    rank = np.full(32, 16, dtype=np.int32)
    b = cm.op_bytes(idx, rank, 4096, 4096, 16)
    assert b == 2 * 32 * 16 * 8192 + 2 * 32 * 4096 + 4 * 32 * 4096 + 8 * 32 * 16
    assert cm.op_flops(idx, rank, 4096, 4096) == 32 * cm.op_flops_per_token(4096, 4096, 16)
    # each distinct adapter counted once, however many rows use it
    same = np.zeros(32, dtype=np.int32)
    assert cm.op_bytes(same, rank, 4096, 4096, 16) == (2 * 16 * 8192 + 2 * 32 * 4096 + 4 * 32 * 4096
                                                      + 8 * 32 * 16)
    # rows without adapter and rank-0 slots cost nothing
    rank0 = rank.copy()
    rank0[3] = 0
    idx2 = idx.copy()
    idx2[5] = -1
    assert cm.op_flops(idx2, rank0, 4096, 4096) == 30 * cm.op_flops_per_token(4096, 4096, 16)
