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
