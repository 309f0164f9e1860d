"""The no-allocation entry point, moe_layout_dispatch_noalloc (the library's own
fixed layout workspace), through the C ABI against moe_layout_dispatch with a
workspace the caller allocates: every layout array and receive array equal bit for
bit, rows past the layout's count untouched, on two calls in a row with the second
input smaller, for the three forms the call takes (one launch for the smallest
batches; count kernel + placing dispatch with the offsets in its workgroup 0; and
with a finalize launch in between for more than 16 tiles), bf16 and FP8, both
receive layouts. The call itself allocates nothing through torch either."""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

CANARY = -12345
PAIRS = [
    # (T, H, E, G, K, mode, dtype) for the first call, then the smaller second call
    ((4096, 7168, 256, 8, 8, "expert", "bf16"), (1000, 2048, 64, 8, 6, "group", "bf16")),
    ((2048, 1024, 128, 8, 8, "expert", "fp8"), (300, 512, 16, 4, 4, "group", "fp8")),
    ((5000, 512, 64, 8, 8, "group", "bf16"), (64, 256, 8, 8, 2, "expert", "bf16")),
    # top-k above 8 (moe_layout + moe_dispatch inside the call, on the library's workspace) and
    # FP8 rows longer than 8192 (the row-sized form, also layout + dispatch inside)
    ((3000, 1024, 64, 8, 12, "group", "bf16"), (700, 16384, 128, 8, 8, "expert", "fp8")),
]
FIELDS = ("expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask", "slot_e",
          "slot_g", "slot_tg", "status")


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_layout_amd as m
    return m


def _inputs(case, seed):
    T, H, E, G, K, mode, dtype = case
    d = si.make_inputs(T, H, E, K, seed=seed)
    idx = d["topk_idx"].copy()
    if T > 100:
        idx[T // 3, 0] = E + 2                       # an invalid entry
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(idx).cuda(), x, torch.from_numpy(d["topk_w"]).cuda()


def _fresh(moe, case):
    T, H, E, G, K, mode, dtype = case
    L = moe.Layout.empty(T, K, E, G)
    D = moe.alloc_dispatch(L, H, mode, dtype)
    if dtype == "bf16":
        D.recv_x.view(torch.int16).fill_(CANARY)
    else:
        D.recv_x.fill_(0xA5)
        D.recv_scale.fill_(-1.5)
    D.recv_topk_w.fill_(-3.0)
    D.recv_topk_idx.fill_(-77)
    return L, D


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a[0]}-{a[6]}-then-{b[0]}-{b[6]}" for a, b in PAIRS])
def test_noalloc_equals_workspace_call(moe, first, second):
    for n, case in enumerate((first, second)):
        T, H, E, G, K, mode, dtype = case
        idx, x, w = _inputs(case, seed=100 + T + n)
        L1, D1 = _fresh(moe, case)
        moe.moe_layout_dispatch(idx, E, G, x, w, mode, dtype, out_layout=L1, out=D1)
        L2, D2 = _fresh(moe, case)
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        moe.moe_layout_dispatch_noalloc(idx, E, G, x, w, mode, dtype, out_layout=L2, out=D2)
        after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        torch.cuda.synchronize()
        assert after == before, "the no-allocation call allocated through torch"
        for f in FIELDS:
            assert torch.equal(getattr(L1, f), getattr(L2, f)), (case, f)
        R, P = int(L1.expert_offset[E].item()), int(L1.group_offset[G].item())
        assert int(L2.status.item()) & moe.STATUS_ERRORS == moe.STATUS_BAD_INDEX if T > 100 else True
        assert torch.equal(L1.recv_src_e[:R], L2.recv_src_e[:R]), case
        assert torch.equal(L1.recv_src_g[:P], L2.recv_src_g[:P]), case
        rows = R if mode == "expert" else P
        a1, a2 = (D1.recv_x.view(torch.int16), D2.recv_x.view(torch.int16)) if dtype == "bf16" else (D1.recv_x, D2.recv_x)
        assert torch.equal(a1, a2), (case, "rows")              # the canary tails too
        if dtype == "fp8":
            assert torch.equal(D1.recv_scale.view(torch.int32), D2.recv_scale.view(torch.int32)), case
            assert bool((D2.recv_x[rows:] == 0xA5).all())
        else:
            assert bool((D2.recv_x.view(torch.int16)[rows:] == CANARY).all())
        assert torch.equal(D1.recv_topk_w.view(torch.int32), D2.recv_topk_w.view(torch.int32)), case
        assert torch.equal(D1.recv_topk_idx, D2.recv_topk_idx), case
        print(f"{case}: {rows} rows equal, status {int(L2.status.item())}", flush=True)


def test_noalloc_no_tokens(moe):
    """T = 0: the call zeroes the counts, offsets and status, as moe_layout_dispatch does."""
    L = moe.Layout.empty(0, 8, 256, 8)
    L.expert_offset.fill_(7)
    L.group_count.fill_(7)
    L.status.fill_(5)
    D = moe.alloc_dispatch(L, 1024, "expert", "bf16")
    idx = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    x = torch.zeros((0, 1024), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    moe.moe_layout_dispatch_noalloc(idx, 256, 8, x, w, "expert", "bf16", out_layout=L, out=D)
    torch.cuda.synchronize()
    assert int(L.expert_offset.abs().sum().item()) == 0 and int(L.group_count.abs().sum().item()) == 0
    assert int(L.status.item()) == 0
