"""The OpenMP build of the oracle (the benchmark times it on every host core beside
the canonical single-thread build) gives the same bits as the canonical build, for
every array of every call: its parallel loops only split tokens or receive rows
whose iterations write disjoint outputs, with the same arithmetic per element."""
import numpy as np
import pytest

import synth_inputs as si


def _run(orc, d, E, G, fp8):
    L = orc.layout(d["topk_idx"], E, G)
    out = {f"L.{k}": v for k, v in L.items() if isinstance(v, np.ndarray)}
    out["L.status"] = np.array([L["status"]])
    for mode in ("expert", "group"):
        D = orc.dispatch_bf16(L, mode, d["x"], d["topk_w"], d["topk_idx"])
        out.update({f"{mode}.bf16.{k}": v for k, v in D.items() if isinstance(v, np.ndarray)})
        out[f"{mode}.combine"] = orc.combine(L, mode, D["recv_x"], d["topk_w"])
        if fp8:
            D8 = orc.dispatch_fp8(L, mode, d["x"], d["topk_w"], d["topk_idx"])
            out.update({f"{mode}.fp8.{k}": v for k, v in D8.items() if isinstance(v, np.ndarray)})
            y = orc.dequant_fp8(D8["recv_q"], D8["recv_scale"])
            out[f"{mode}.dequant"] = y
            out[f"{mode}.combine8"] = orc.combine(L, mode, y, d["topk_w"])
    Dg = orc.dispatch_bf16(L, "group", d["x"], d["topk_w"], d["topk_idx"])
    out["regroup"] = orc.regroup_rows(L, Dg["recv_x"])
    return out


@pytest.mark.parametrize("T,H,E,G,K,routing,fp8", [
    (256, 7168, 256, 8, 8, "uniform", True),     # the t256 shape
    (1024, 4096, 128, 8, 8, "zipf", False),      # the skewed shape, a quarter of its tokens
    (16, 2048, 8, 8, 2, "uniform", True),        # the tiny shape
    (777, 384, 64, 4, 6, "uniform", True),       # ragged, with invalid entries
])
@pytest.mark.parametrize("nthreads", [3, 8])
def test_openmp_build_is_bit_identical(orc, T, H, E, G, K, routing, fp8, nthreads):
    d = si.make_inputs(T, H, E, K, seed=T + H, routing=routing)
    if T > 100:
        d["topk_idx"][5, 1] = E + 1                      # out of range
        d["topk_idx"][T - 7, 2] = d["topk_idx"][T - 7, 0]   # repeat
    ref = _run(orc, d, E, G, fp8)
    with orc.variant("openmp"):
        orc.set_threads(nthreads)
        assert orc.threads() == nthreads
        got = _run(orc, d, E, G, fp8)
    assert orc.threads() == 1
    assert got.keys() == ref.keys()
    for k in ref:
        a, b = ref[k], got[k]
        assert a.dtype == b.dtype and a.shape == b.shape, k
        assert a.tobytes() == b.tobytes(), k
