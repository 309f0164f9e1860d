"""Run by test_gpu_parity.test_sync_fallback_is_exact in a process of its own, with
MOE_EP_BASE_WAIT_TICKS set (the library reads its tuning once per process):
  "0"  : each token's wave of the placing dispatch polls its tile's bases once and,
         if workgroup 0 has not written them yet, computes them itself from the
         count table (the path a wave takes after waiting 0.2 s by default);
  "-1" : every token computes its bases itself, without polling.
Either way every layout array and every receive row must equal the oracle's
exactly, rows past the layout's count keep their canary, and the status may carry
only the diagnostic MOE_STATUS_SYNC_FALLBACK bit (always, for "-1") besides the
input's own error bits. Covers bf16 with the offsets in the dispatch's workgroup 0
(T = 4096, 16 tiles) and with a finalize launch before it (20 tiles), both
layouts, and the placing FP8 form. Exits non-zero on a mismatch."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import combine_moe_layout_amd as moe  # noqa: E402
import oracle as orc  # noqa: E402
import synth_inputs as si  # noqa: E402

mode_env = os.environ.get("MOE_EP_BASE_WAIT_TICKS")
assert mode_env in ("0", "-1"), mode_env
CANARY = -12345
for T, H, E, G, K, dtype in [(4096, 1024, 256, 8, 8, "bf16"), (5000, 512, 64, 8, 6, "bf16"),
                             (2048, 1024, 128, 8, 8, "fp8")]:
    d = si.make_inputs(T, H, E, K, seed=77 + T)
    idx = d["topk_idx"].copy()
    idx[T // 3, 0] = E + 1                                  # an invalid entry
    x16 = np.ascontiguousarray(d["x"]).view(np.int16)
    x = torch.from_numpy(x16).cuda().view(torch.bfloat16)
    Lo = orc.layout(idx, E, G)
    for mode in ("expert", "group"):
        L = moe.Layout.empty(T, K, E, G)
        D = moe.alloc_dispatch(L, H, mode, dtype)
        if dtype == "bf16":
            Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], idx)
        else:
            Do = orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], idx)
        R = Do["R"]
        for rep in range(2):
            if dtype == "bf16":
                D.recv_x.view(torch.int16).fill_(CANARY)
            else:
                D.recv_x.fill_(0xA5)
            L, D = moe.moe_layout_dispatch(torch.from_numpy(idx).cuda(), E, G, x,
                                           torch.from_numpy(d["topk_w"]).cuda(), mode, dtype,
                                           out_layout=L, out=D)
            torch.cuda.synchronize()
            status = int(L.status.item())
            assert status & ~moe.STATUS_SYNC_FALLBACK == Lo["status"], (T, mode, status)
            if mode_env == "-1":
                assert status & moe.STATUS_SYNC_FALLBACK, (T, mode, status)
            for n in ("expert_count", "expert_offset", "group_count", "group_offset", "slot_e", "slot_g",
                      "slot_tg"):
                np.testing.assert_array_equal(getattr(L, n).cpu().numpy(), Lo[n], err_msg=f"{T} {mode} {n}")
            np.testing.assert_array_equal(L.recv_src_e.cpu().numpy()[:Lo["R_expert"]], Lo["recv_src_e"][:Lo["R_expert"]])
            np.testing.assert_array_equal(L.recv_src_g.cpu().numpy()[:Lo["R_group"]], Lo["recv_src_g"][:Lo["R_group"]])
            if dtype == "bf16":
                rx = D.recv_x.view(torch.int16).cpu().numpy().view(np.uint16)
                np.testing.assert_array_equal(rx[:R], Do["recv_x"], err_msg=f"{T} {mode} rows")
                assert (rx[R:].view(np.int16) == CANARY).all(), (T, mode)
            else:
                q = D.recv_x.cpu().numpy()
                np.testing.assert_array_equal(q[:R], Do["recv_q"], err_msg=f"{T} {mode} codes")
                assert (q[R:] == 0xA5).all(), (T, mode)
                np.testing.assert_array_equal(D.recv_scale.cpu().numpy()[:R].view(np.uint32),
                                              Do["recv_scale"].view(np.uint32))
            np.testing.assert_array_equal(D.recv_topk_w.cpu().numpy()[:R], Do["recv_w"])
            np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:R], Do["recv_idx"])
            print(f"wait={mode_env} T={T} {dtype} {mode} call {rep}: {R} rows exact, status {status}", flush=True)
