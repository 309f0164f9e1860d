"""Run by test_gpu_layout_exchange.test_exchange_wait_cut_short in a process of its
own, with MOE_EP_BASE_WAIT_TICKS set (the library reads its tuning once per process):
  "0"  : each tile's workgroup of the one-launch layout reads the other tiles' counts
         once and, if any has not arrived yet, counts every token itself (the path a
         workgroup takes after waiting 0.2 s by default);
  "-1" : every workgroup counts every token itself, without reading the table.
Either way every layout array must equal the oracle's exactly, and the status may
carry only the diagnostic MOE_STATUS_SYNC_FALLBACK bit besides the input's own error
bits (always, for "-1", since tile 0 then counts too). Covers exact and non-exact
top-k, one tile and several, a ragged last tile, more experts than one chunk per
thread, and invalid entries. Exits non-zero on a mismatch."""
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
NAMES = ("expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask", "slot_e", "slot_g",
         "slot_tg")
for T, E, G, K in [(4096, 256, 8, 8), (3000, 64, 8, 6), (1000, 16, 4, 4), (256, 256, 8, 8), (2500, 512, 16, 8),
                   (777, 8, 8, 2)]:
    d = si.make_inputs(T, 128, E, K, seed=91 + T)
    idx = d["topk_idx"].copy()
    idx[T // 3, 0] = E + 1                          # an invalid entry
    idx[T // 2, K - 1] = idx[T // 2, 0]             # a repeat
    Lo = orc.layout(idx, E, G)
    L = moe.Layout.empty(T, K, E, G)
    for rep in range(3):
        moe.moe_layout(torch.from_numpy(idx).cuda(), E, G, out=L)
        torch.cuda.synchronize()
        status = int(L.status.item())
        assert status & ~moe.STATUS_SYNC_FALLBACK == Lo["status"], (T, E, status)
        if mode_env == "-1":
            assert status & moe.STATUS_SYNC_FALLBACK, (T, E, status)
        for n in NAMES:
            np.testing.assert_array_equal(getattr(L, n).cpu().numpy().astype(np.int64),
                                          Lo[n].astype(np.int64), err_msg=f"{T} {E} {n}")
        np.testing.assert_array_equal(L.recv_src_e.cpu().numpy()[:Lo["R_expert"]], Lo["recv_src_e"][:Lo["R_expert"]])
        np.testing.assert_array_equal(L.recv_src_g.cpu().numpy()[:Lo["R_group"]], Lo["recv_src_g"][:Lo["R_group"]])
    print(f"wait={mode_env} T={T} E={E} G={G} K={K}: exact, status {status}", flush=True)
