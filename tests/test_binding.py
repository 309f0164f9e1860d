"""The Python binding's own checks, on the CPU: host tensors are refused before any call
reaches the library (their addresses given to a kernel would fault the GPU), and wrong
dtypes or shapes raise ValueError."""
import pytest
import torch

import combine_moe_layout_amd as moe

T, K, E, G, H = 8, 2, 8, 2, 64


def test_host_tensors_are_refused():
    idx = torch.zeros((T, K), dtype=torch.int32)
    w = torch.full((T, K), 0.5)
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        moe.moe_layout(idx, E, G)
    L = moe.Layout.empty(T, K, E, G, device="cpu")
    with pytest.raises(ValueError, match="GPU tensors"):
        moe.moe_dispatch(L, x, w, idx, "expert")
    with pytest.raises(ValueError, match="GPU tensors"):
        moe.moe_combine(L, x, w, "expert")
    with pytest.raises(ValueError, match="GPU tensors"):
        moe.moe_layout_dispatch(idx, E, G, x, w, "expert", out_layout=L)


def test_wrong_dtype_or_shape_raises():
    with pytest.raises(ValueError):
        moe.moe_layout(torch.zeros((T, K), dtype=torch.int64), E, G)
    with pytest.raises(ValueError):
        moe.moe_layout(torch.zeros((T * K,), dtype=torch.int32), E, G)
    L = moe.Layout.empty(T, K, E, G, device="cpu")
    idx = torch.zeros((T, K), dtype=torch.int32)
    with pytest.raises(ValueError):
        moe.moe_dispatch(L, torch.zeros((T, H), dtype=torch.float32), torch.zeros((T, K)), idx)
    with pytest.raises(ValueError):
        moe.moe_dispatch(L, torch.zeros((T, H), dtype=torch.bfloat16), torch.zeros((T, K + 1)), idx)
    with pytest.raises(ValueError):
        moe.moe_combine(L, torch.zeros((T, H), dtype=torch.float16), torch.zeros((T, K)))
    with pytest.raises(ValueError):
        moe.moe_layout(torch.zeros((T, K), dtype=torch.int32), E, G, out=moe.Layout.empty(T, K + 1, E, G, "cpu"))


def test_out_buffers_and_layout_arrays_are_checked():
    """Caller-supplied buffers the library would write past are refused by name: the C
    ABI sees only pointers and row counts."""
    L = moe.Layout.empty(T, K, E, G, device="cpu")
    idx = torch.zeros((T, K), dtype=torch.int32)
    w = torch.full((T, K), 0.5)
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    D = moe.alloc_dispatch(L, H, "expert", "bf16", device="cpu")
    cap = D.recv_x.shape[0]
    with pytest.raises(ValueError, match="recv_topk_idx"):          # arrays that disagree
        moe.Dispatched(D.recv_x, None, torch.zeros((cap, K + 1)), D.recv_topk_idx)
    bad = moe.Dispatched(D.recv_x, None, torch.zeros((cap, K + 1)), torch.zeros((cap, K + 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="recv_topk_w"):             # another K than the layout's
        moe.moe_dispatch(L, x, w, idx, "expert", out=bad)
    with pytest.raises(ValueError, match="recv_x"):
        moe.moe_dispatch(L, x, w, idx, "expert", "fp8", out=D)          # bf16 rows for FP8
    with pytest.raises(ValueError, match="one row per token"):
        moe.moe_dispatch(L, torch.zeros((T + 1, H), dtype=torch.bfloat16), w, idx, "expert")
    with pytest.raises(ValueError, match="out"):
        moe.moe_combine(L, x, w, "expert", out=torch.zeros((T, H - 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="topk_w"):
        moe.moe_combine(L, x, w.t(), "expert")                          # strided
    q = torch.zeros((T, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scale"):
        moe.moe_fp8_dequant(L, q, torch.zeros((T, 2)))
    with pytest.raises(ValueError, match="scale"):
        moe.moe_cast_transpose_fp8(L, torch.zeros((T * K, H), dtype=torch.bfloat16), torch.zeros(E + 1))
    short = moe.Layout.empty(T, K, E, G, device="cpu")
    short.slot_e = short.slot_e[:-1]
    with pytest.raises(ValueError, match="Layout.slot_e"):
        moe.moe_dispatch(short, x, w, idx, "expert")
    with pytest.raises(ValueError, match="nbytes"):
        moe.moe_ref_copy(torch.zeros(16, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8))
