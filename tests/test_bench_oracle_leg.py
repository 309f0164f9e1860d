"""CPU tests of the benchmark's oracle leg and parity checker: both oracle builds are
timed on a workload and found identical, and the parity checker passes arrays equal to
the oracle's and reports a changed element in any of them (a layout slot, a receive
row, an FP8 scale, a combine output), so a mismatch on the GPU cannot read as parity."""
import numpy as np
import pytest

import bench
import synth_inputs as si


def _as_gpu(ora, fp8):
    """The oracle's outputs in the form the benchmark reads GPU arrays back in."""
    L = ora["L"]
    g = {"L": {n: (L[n].copy().view(np.uint32) if L[n].dtype == np.int32 else L[n].copy())
               for n in L if isinstance(L[n], np.ndarray)}}
    g["L"]["status"] = np.array([L["status"]], np.uint32)
    for mode in ("expert", "group"):
        D = ora[mode]["D"]
        R = D["R"]
        m = {"out": ora[mode]["out"].copy()}
        for n in D["_names"]:
            a = D[n][:R].copy()
            m[n] = a.view(np.uint32) if a.dtype in (np.float32, np.int32) else a
        if fp8:
            m["y"] = ora[mode]["y"][:R].copy()
        g[mode] = m
    return g


@pytest.mark.parametrize("fp8", [False, True])
def test_oracle_leg_and_parity_checker(fp8):
    d = si.make_inputs(300, 512, 32, 4, seed=9)
    d["workload"] = si.Workload("probe", T=300, H=512, E=32, G=4, K=4, fp8=fp8, seed=9)
    orc, ora = bench.oracle_leg(d, 3)
    assert orc["builds_identical"] and orc["threads"] == 3
    for c in ("layout", "dispatch_expert", "combine_expert", "dispatch_group", "combine_group"):
        assert orc["calls"][c]["us_1"] > 0 and orc["calls"][c]["us_3"] > 0
    g = _as_gpu(ora, fp8)
    p = bench.parity_of(g, ora, fp8)
    assert p["ok"] and all(v == "bit-exact" for k, v in p.items() if k != "ok")
    rows = "recv_q" if fp8 else "recv_x"
    plants = [("L", "slot_e", "layout"), ("expert", rows, "dispatch_expert"), ("group", "recv_w", "dispatch_group"),
              ("expert", "out", "combine_expert")]
    if fp8:
        plants += [("group", "recv_scale", "dispatch_group"), ("expert", "y", "dequant_expert")]
    for where, name, key in plants:
        g2 = _as_gpu(ora, fp8)
        a = g2[where][name]
        a.reshape(-1)[a.size // 3] ^= 1
        p2 = bench.parity_of(g2, ora, fp8)
        assert not p2["ok"] and p2[key] != "bit-exact", (where, name)
