"""Random-shape stress: 200 rounds, each a random routing problem run through every
call of the library (layout, dispatch or the fused small-batch call, dequant,
regroup, per-expert cast + transpose, combine) and compared with the oracle
(bit-exact; combine to the same bar as the parity tests). Shapes stay small so a
round takes milliseconds."""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

ROUNDS = 200


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _draw(rng):
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    epg = int(rng.choice([1, 2, 3, 8, 16, 32]))
    E = min(G * epg, 1024)
    K = int(rng.choice([1, 2, 3, 4, 6, 8, 8, 8, 13, 32]))
    K = min(K, E)
    T = int(rng.choice([0, 1, 2, 17, 100, 255, 256, 257, 511, 700]))
    fp8 = bool(rng.random() < 0.4)
    H = 128 * int(rng.integers(1, 17)) if fp8 else 8 * int(rng.integers(1, 257))
    routing = "zipf" if rng.random() < 0.3 else "uniform"
    return T, H, E, G, K, fp8, routing


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available()
    import combine_moe_layout_amd as moe
    import oracle
    return moe, oracle


def test_random_rounds(libs):
    moe, orc = libs
    rng = np.random.default_rng(20261202)
    for rnd in range(ROUNDS):
        T, H, E, G, K, fp8, routing = _draw(rng)
        case = f"round {rnd}: T={T} H={H} E={E} G={G} K={K} fp8={fp8} {routing}"
        d = si.make_inputs(T, H, E, K, seed=1000 + rnd, routing=routing)
        idx = d["topk_idx"].copy()
        if T and rng.random() < 0.3:                      # invalid entries
            n = int(rng.integers(1, 4))
            idx[rng.integers(0, T, n), rng.integers(0, K, n)] = rng.choice([-1, E, E + 7], n)
            if K > 1:
                t0 = int(rng.integers(0, T))
                idx[t0, K - 1] = idx[t0, 0]
        w = d["topk_w"]
        dt = "fp8" if fp8 else "bf16"
        idx_d = torch.from_numpy(idx).cuda()
        w_d = torch.from_numpy(w).cuda()
        x_d = _dev_bf16(d["x"])
        Lo = orc.layout(idx, E, G)
        fused = T <= 512 and T * K <= 16384 and rng.random() < 0.5
        mode = "group" if rng.random() < 0.5 else "expert"
        if fused:
            L, D = moe.moe_layout_dispatch(idx_d, E, G, x_d, w_d, mode, dt)
        else:
            L = moe.moe_layout(idx_d, E, G)
            D = moe.moe_dispatch(L, x_d, w_d, idx_d, mode, dt)
        torch.cuda.synchronize()
        assert int(L.status.item()) == Lo["status"], case
        for n in ("expert_count", "expert_offset", "group_count", "group_offset", "slot_e",
                  "slot_g", "slot_tg"):
            assert np.array_equal(getattr(L, n).cpu().numpy(), Lo[n]), (case, n)
        R = Lo["R_expert"] if mode == "expert" else Lo["R_group"]
        if fp8:
            Do = orc.dispatch_fp8(Lo, mode, d["x"], w, idx)
            assert np.array_equal(D.recv_x[:R].cpu().numpy(), Do["recv_q"]), case
            assert np.array_equal(D.recv_scale[:R].cpu().numpy().view(np.uint32),
                                  Do["recv_scale"].view(np.uint32)), case
            y = moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode)
            y_ref = orc.dequant_fp8(Do["recv_q"], Do["recv_scale"])
            assert np.array_equal(_bits(y)[:R], y_ref), case
        else:
            Do = orc.dispatch_bf16(Lo, mode, d["x"], w, idx)
            assert np.array_equal(_bits(D.recv_x)[:R], Do["recv_x"]), case
            y = D.recv_x
            y_ref = Do["recv_x"]
        assert np.array_equal(D.recv_topk_idx[:R].cpu().numpy(), Do["recv_idx"]), case
        assert np.array_equal(D.recv_topk_w[:R].cpu().numpy().view(np.uint32),
                              Do["recv_w"].view(np.uint32)), case
        if mode == "group" and T:
            De = moe.moe_regroup(L, D)
            Re = Lo["R_expert"]
            ref = orc.regroup(Lo, {"recv_x": Do.get("recv_x", Do.get("recv_q"))})
            got = De.recv_x[:Re].cpu().numpy() if fp8 else _bits(De.recv_x)[:Re]
            assert np.array_equal(got, ref["recv_x"]), case
        if mode == "expert" and not fp8 and H % 64 == 0:   # per-expert FP8 cast + transpose
            scale = rng.uniform(0.25, 300.0, E).astype(np.float32)
            CT = moe.moe_cast_transpose_fp8(L, D.recv_x, torch.from_numpy(scale).cuda())
            ref = orc.cast_transpose_fp8(Lo["expert_offset"], Do["recv_x"], scale)
            assert np.array_equal(CT.pad_offset.cpu().numpy(), ref["pad_offset"]), case
            assert np.array_equal(CT.c[:R].cpu().numpy(), ref["c"]), case
            nt = H * int(ref["pad_offset"][-1])
            assert np.array_equal(CT.t[:nt].cpu().numpy(), ref["t"]), case
            assert np.array_equal(CT.amax.cpu().numpy().view(np.uint32),
                                  ref["amax"].view(np.uint32)), case
        # combine with random non-identity weights
        w2 = (rng.standard_normal((T, K)) * 1.5).astype(np.float32)
        out = moe.moe_combine(L, y, torch.from_numpy(w2).cuda(), mode)
        ref = orc.combine(Lo, mode, y_ref if T else np.zeros((0, H), np.uint16), w2)
        assert np.array_equal(_bits(out), ref), case
