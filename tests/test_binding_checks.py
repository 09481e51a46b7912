"""The Python binding rejects tensors the C ABI cannot check (CPU, no GPU needed).

The library receives raw pointers and leading dimensions, so a host tensor, a wrong
dtype, a transposed view or a tensor with too few rows or columns would reach the
kernels as an out-of-bounds access.  The binding checks every tensor before the call
and raises ValueError; host tile lists with a position in two tiles or a row twice in
the row map are rejected before they are copied to the device."""
import numpy as np
import pytest
import torch

from segmented_gather_matmul_amd import binding as B


def _weights(S=2, d_in=16, d_out=24, r_max=4):
    return B.Weights(num_slots=S, d_in=d_in, d_out=d_out, r_max=r_max, rank=torch.full((S,), r_max, dtype=torch.int32),
                     scale=torch.ones(S, dtype=torch.float32), a_t=torch.zeros(S * r_max * d_in, dtype=torch.float16),
                     b=torch.zeros(S * r_max * d_out, dtype=torch.float16))


def _args(n=3, d_in=16, d_out=24, r_max=4):
    x = torch.zeros((n, d_in), dtype=torch.float16)
    y = torch.zeros((n, d_out), dtype=torch.float16)
    v = torch.zeros((n, r_max), dtype=torch.float32)
    idx = torch.zeros(n, dtype=torch.int32)
    return x, y, v, idx


def test_weights_reject_wrong_dtypes_and_sizes():
    S, r = 2, 4
    ok = dict(num_slots=S, d_in=16, d_out=24, r_max=r, rank=torch.zeros(S, dtype=torch.int32),
              scale=torch.ones(S, dtype=torch.float32), a_t=torch.zeros(S * r * 16, dtype=torch.float16),
              b=torch.zeros(S * r * 24, dtype=torch.float16))
    B.Weights(**ok)
    for key, bad, msg in (("rank", torch.zeros(S, dtype=torch.int64), "dtype"),
                          ("scale", torch.ones(S, dtype=torch.float16), "dtype"),
                          ("rank", torch.zeros(S - 1, dtype=torch.int32), "elements"),
                          ("a_t", torch.zeros(S * r * 16 - 1, dtype=torch.float16), "elements"),
                          ("b", torch.zeros((S * r * 24, 2), dtype=torch.float16)[:, 0], "contiguous")):
        with pytest.raises(ValueError, match=msg):
            B.Weights(**{**ok, key: bad})


@pytest.mark.parametrize("case", ["x_dtype", "x_transposed", "x_rows", "y_cols", "v_cols", "v_dtype", "idx_dtype",
                                  "idx_short", "x_host", "w_host"])
def test_launch_arguments_are_checked_before_the_call(case):
    w = _weights()
    x, y, v, idx = _args()
    expect = {"x_dtype": "dtype", "x_transposed": "stride", "x_rows": "at least", "y_cols": "at least",
              "v_cols": "at least", "v_dtype": "dtype", "idx_dtype": "dtype", "idx_short": "elements",
              "x_host": "GPU tensor", "w_host": "GPU tensor"}[case]
    if case == "x_dtype":
        x = x.float()
    elif case == "x_transposed":
        x = torch.zeros((16, 3), dtype=torch.float16).t()
    elif case == "x_rows":
        x = x[:2]
    elif case == "y_cols":
        y = y[:, :23]
    elif case == "v_cols":
        v = v[:, :3]
    elif case == "v_dtype":
        v = v.half()
    elif case == "idx_dtype":
        idx = idx.long()
    elif case == "idx_short":
        idx = idx[:2]
    with pytest.raises(ValueError, match=expect):
        if case == "w_host":
            B.proj_list([(w, v, y)], 3, expand=True)
        else:
            B.lora_bgmv(y, x, idx, w, v)
    if case in ("x_dtype", "x_transposed", "v_cols", "v_dtype", "idx_dtype", "idx_short", "x_host"):
        with pytest.raises(ValueError, match=expect):
            B.lora_bgmv_shrink(v, x, idx, w)


def test_segment_lists_with_reused_positions_or_rows_are_rejected():
    tiles = np.array([[0, 0, 2, 0], [1, 1, 2, 1]], dtype=np.int32)   # position 1 in two tiles
    with pytest.raises(B.LoraError) as e:
        B.segments_to_device(tiles, None, 4, device="cpu")
    assert e.value.code == B.LORA_E_INDEX
    tiles = np.array([[0, 0, 2, 0], [1, 2, 2, 1]], dtype=np.int32)
    with pytest.raises(B.LoraError) as e:
        B.segments_to_device(tiles, np.array([3, 0, 3, 1], dtype=np.int32), 4, device="cpu")  # row 3 twice
    assert e.value.code == B.LORA_E_INDEX
    segs = B.segments_to_device(tiles, np.array([3, 0, 2, 1], dtype=np.int32), 4, device="cpu")
    assert segs.n_tiles == 2
    with pytest.raises(ValueError, match="GPU tensor"):
        segs.ref


def test_pool_load_needs_host_blob_and_large_enough_staging():
    blob = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="elements"):
        B.lora_pool_load([], blob, torch.zeros(32, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dtype"):
        B.lora_pool_load([], blob.float(), torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.lora_pool_load([], blob, torch.zeros(64, dtype=torch.uint8))
