"""Random batches through moe_layout_dispatch, the one call of layout and dispatch:
40 routing problems of 300-16384 tokens (the count kernel and a dispatch whose
workgroups place their own tokens, with the offsets from its workgroup 0 up to 16
tiles and from a finalize workgroup above; FP8 with the placing dispatch up to 3072
tokens, the layout and the plain dispatch above), top-k 1-8, both receive layouts,
bf16 and FP8, with repeated and out-of-range entries. Every layout array, receive
row (FP8: codes and scales), weight and index row is compared with the oracle, bit
for bit; rows past the receive count keep their canary."""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

NAMES = ("expert_count", "expert_offset", "group_count", "group_offset", "slot_e", "slot_g", "slot_tg")
CANARY16 = np.int16(-12345)


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_layout_amd as moe
    import oracle
    return moe, oracle


def test_random_fused_calls(libs):
    moe, orc = libs
    rng = np.random.default_rng(20261204)
    for rnd in range(40):
        G = int(rng.choice([1, 4, 8, 32]))
        E = G * int(rng.choice([1, 2, 8, 16])) if G < 32 else 32 * int(rng.choice([1, 4, 8]))
        K = min(int(rng.integers(1, 9)), E)
        T = int(rng.integers(300, 16385))
        fp8 = bool(rng.random() < 0.35)
        H = 128 * int(rng.integers(1, 9)) if fp8 else 8 * int(rng.integers(1, 129))
        mode = "group" if rnd % 2 else "expert"
        d = si.make_inputs(T, H, E, K, seed=4000 + rnd, routing="zipf" if rnd % 3 == 0 else "uniform")
        idx = d["topk_idx"].copy()
        if K > 1 and rnd % 2 == 0:
            n = int(rng.integers(1, 20))
            ts, k1 = rng.integers(0, T, n), rng.integers(1, K, n)
            idx[ts, k1] = idx[ts, (rng.random(n) * k1).astype(np.int64)]
        if rnd % 5 == 0:
            n = int(rng.integers(1, 10))
            idx[rng.integers(0, T, n), rng.integers(0, K, n)] = rng.choice([-1, E, E + 3], n)
        what = f"round {rnd}: T={T} H={H} E={E} G={G} K={K} {mode} {'fp8' if fp8 else 'bf16'}"
        print(what, flush=True)
        dt = "fp8" if fp8 else "bf16"
        L = moe.Layout.empty(T, K, E, G)
        D = moe.alloc_dispatch(L, H, mode, dt)
        if fp8:
            D.recv_x.fill_(0xA5)
        else:
            D.recv_x.view(torch.int16).fill_(int(CANARY16))
        x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).cuda().view(torch.bfloat16)
        L, D = moe.moe_layout_dispatch(torch.from_numpy(idx).cuda(), E, G, x,
                                       torch.from_numpy(d["topk_w"]).cuda(), mode, dt, out_layout=L, out=D)
        torch.cuda.synchronize()
        Lo = orc.layout(idx, E, G)
        assert int(L.status.item()) & ~moe.STATUS_SYNC_FALLBACK == Lo["status"], what
        for n in NAMES:
            np.testing.assert_array_equal(getattr(L, n).cpu().numpy(), Lo[n], err_msg=f"{what} {n}")
        np.testing.assert_array_equal(L.tok_group_mask.cpu().numpy().view(np.uint32), Lo["tok_group_mask"],
                                      err_msg=what)
        np.testing.assert_array_equal(L.recv_src_e.cpu().numpy()[:Lo["R_expert"]], Lo["recv_src_e"][:Lo["R_expert"]])
        np.testing.assert_array_equal(L.recv_src_g.cpu().numpy()[:Lo["R_group"]], Lo["recv_src_g"][:Lo["R_group"]])
        if fp8:
            Do = orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], idx)
            R = Do["R"]
            q = D.recv_x.cpu().numpy()
            np.testing.assert_array_equal(q[:R], Do["recv_q"], err_msg=f"{what} codes")
            assert (q[R:] == 0xA5).all(), what
            np.testing.assert_array_equal(D.recv_scale.cpu().numpy()[:R].view(np.uint32),
                                          Do["recv_scale"].view(np.uint32), err_msg=f"{what} scales")
        else:
            Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], idx)
            R = Do["R"]
            rx = D.recv_x.view(torch.int16).cpu().numpy()
            np.testing.assert_array_equal(rx[:R].view(np.uint16), Do["recv_x"], err_msg=f"{what} rows")
            assert (rx[R:] == CANARY16).all(), what
        np.testing.assert_array_equal(D.recv_topk_w.cpu().numpy()[:R], Do["recv_w"], err_msg=what)
        np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:R], Do["recv_idx"], err_msg=what)
