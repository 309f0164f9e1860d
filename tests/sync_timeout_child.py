"""Run by test_gpu_parity.test_sync_timeout_skips_tokens_cleanly in a process of its
own, with MOE_EP_BASE_WAIT_TICKS=0 (the library reads its tuning once per process):
every token's wave of the placing dispatch polls its tile's bases once and gives up
if workgroup 0 has not written them yet. Checks that each token is either placed
exactly as the oracle places it or skipped whole (its layout entries -1, its rows
untouched), that the counts and offsets are exact regardless, and that the status
reports the timeout exactly when a token was skipped. Exits non-zero on a mismatch."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import combine_moe_layout_amd as moe  # noqa: E402
import oracle as orc  # noqa: E402
import synth_inputs as si  # noqa: E402

assert os.environ.get("MOE_EP_BASE_WAIT_TICKS") == "0"
T, H, E, G, K = 4096, 1024, 256, 8, 8
CANARY = -12345
d = si.make_inputs(T, H, E, K, seed=77)
idx, w = d["topk_idx"], d["topk_w"]
x16 = np.ascontiguousarray(d["x"]).view(np.int16)
x = torch.from_numpy(x16).cuda().view(torch.bfloat16)
Lo = orc.layout(idx, E, G)
so = Lo["slot_e"].reshape(T, K)
L = moe.Layout.empty(T, K, E, G)
D = moe.alloc_dispatch(L, H, "expert", "bf16")
for rep in range(2):
    D.recv_x.view(torch.int16).fill_(CANARY)
    L, D = moe.moe_layout_dispatch(torch.from_numpy(idx).cuda(), E, G, x, torch.from_numpy(w).cuda(),
                                   "expert", out_layout=L, out=D)
    torch.cuda.synchronize()
    for n in ("expert_count", "expert_offset", "group_count", "group_offset"):
        np.testing.assert_array_equal(getattr(L, n).cpu().numpy(), Lo[n], err_msg=n)
    slot_e = L.slot_e.cpu().numpy().reshape(T, K)
    slot_g = L.slot_g.cpu().numpy().reshape(T, K)
    slot_tg = L.slot_tg.cpu().numpy().reshape(T, G)
    placed = (slot_e == so).all(1) & (slot_g == Lo["slot_g"].reshape(T, K)).all(1) & \
        (slot_tg == Lo["slot_tg"].reshape(T, G)).all(1)
    skipped = (slot_e == -1).all(1) & (slot_g == -1).all(1) & (slot_tg == -1).all(1)
    assert (placed | skipped).all(), "a token neither placed as the oracle places it nor skipped whole"
    status = int(L.status.item())
    assert status == (moe.STATUS_SYNC_TIMEOUT if skipped.any() else 0), status
    rx = D.recv_x.view(torch.int16).cpu().numpy()
    src = L.recv_src_e.cpu().numpy()
    written = np.zeros(T * K, bool)
    for t in np.nonzero(placed)[0]:
        rows = so[t]
        written[rows] = True
        assert (rx[rows] == x16[t]).all(), f"token {t}: rows differ"
        assert (src[rows] == t * K + np.arange(K)).all(), f"token {t}: receive list"
    assert (rx[~written] == CANARY).all(), "a skipped token's row was written"
    print(f"call {rep}: {int(placed.sum())} tokens placed, {int(skipped.sum())} skipped, status {status}")
