"""Run by test_gpu_parity.test_fused_fp8_placing_form in a process of its own with
MOE_EP_FUSED_FP8_PLACE_MAX_T set high (the library reads its tuning once per process):
the fused call's placing FP8 form, also above the token count where the default
routing leaves it, against the oracle in both layouts, with the offsets computed in
the dispatch (up to 16 tiles) and by a separate workgroup (17 tiles). Exits non-zero
on a mismatch."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import combine_moe_layout_amd as moe  # noqa: E402
import oracle as orc  # noqa: E402
import synth_inputs as si  # noqa: E402

assert int(os.environ.get("MOE_EP_FUSED_FP8_PLACE_MAX_T", "0")) >= 4097
for T, H, E, G, K in [(300, 1024, 64, 8, 8), (2000, 2048, 256, 8, 8), (4097, 1024, 128, 8, 6)]:
    d = si.make_inputs(T, H, E, K, seed=T + H)
    idx = d["topk_idx"].copy()
    idx[T // 3, 0] = E + 1                                  # an invalid entry
    Lo = orc.layout(idx, E, G)
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).cuda().view(torch.bfloat16)
    for mode in ("expert", "group"):
        Do = orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], idx)
        R = Do["R"]
        L = moe.Layout.empty(T, K, E, G)
        D = moe.alloc_dispatch(L, H, mode, "fp8")
        D.recv_x.fill_(0xA5)
        L, D = moe.moe_layout_dispatch(torch.from_numpy(idx).cuda(), E, G, x,
                                       torch.from_numpy(d["topk_w"]).cuda(), mode, "fp8", out_layout=L, out=D)
        torch.cuda.synchronize()
        assert int(L.status.item()) == Lo["status"], (T, mode)
        for n in ("expert_offset", "group_offset", "slot_e", "slot_g", "slot_tg"):
            np.testing.assert_array_equal(getattr(L, n).cpu().numpy(), Lo[n], err_msg=f"{T} {mode} {n}")
        q = D.recv_x.cpu().numpy()
        np.testing.assert_array_equal(q[:R], Do["recv_q"], err_msg=f"{T} {mode} codes")
        assert np.all(q[R:] == 0xA5), (T, mode)
        np.testing.assert_array_equal(D.recv_scale.cpu().numpy()[:R].view(np.uint32),
                                      Do["recv_scale"].view(np.uint32), err_msg=f"{T} {mode} scales")
        np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:R], Do["recv_idx"])
        print(f"T={T} H={H} E={E} K={K} {mode}: {R} rows match")
