"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element
by element, on the same seeded inputs.

Bar: layout arrays, dispatched rows, metadata, FP8 bytes and scales are
bit-exact; combine is held to <= 1 bf16 ulp and its count of non-identical
elements is asserted to be 0 (both sides run the same fp32 fma chain).
Shapes: every named workload at full size (the sizes bench.py times), small
shapes spanning several layout tiles with ragged tails, and edge cases
(T = 0 / 1, K = 1 / 32, G = 1 / E, ragged and multi-pass H, invalid entries).
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

FULL = ["tiny", "t256", "t4096", "skew", "fp8"]
MODES = ["expert", "group"]
CANARY16 = np.uint16(0xBEEF)


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_layout_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def dev_bf16(x_u16):
    return torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


_cache = {}


def workload(name):
    if name not in _cache:
        _cache[name] = si.make_workload(name)
    return _cache[name]


LAYOUT_ARRAYS = ("expert_count", "expert_offset", "group_count", "group_offset", "slot_e",
                 "slot_g", "slot_tg")


def check_layout(L, Lo):
    torch.cuda.synchronize()
    assert int(L.status.item()) == Lo["status"]
    for n in LAYOUT_ARRAYS:
        np.testing.assert_array_equal(getattr(L, n).cpu().numpy(), Lo[n], err_msg=n)
    np.testing.assert_array_equal(L.tok_group_mask.cpu().numpy().view(np.uint32),
                                  Lo["tok_group_mask"])
    np.testing.assert_array_equal(L.recv_src_e[:Lo["R_expert"]].cpu().numpy(),
                                  Lo["recv_src_e"][:Lo["R_expert"]])
    np.testing.assert_array_equal(L.recv_src_g[:Lo["R_group"]].cpu().numpy(),
                                  Lo["recv_src_g"][:Lo["R_group"]])


def ulp_diff_bf16(a_u16, b_u16):
    """Distance in bf16 ulps between two bf16 bit arrays (monotone integer map)."""
    def key(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + (u & 0x7FFF))
    return np.abs(key(a_u16) - key(b_u16))


def assert_combine_equal(got_u16, ref_u16):
    d = ulp_diff_bf16(got_u16, ref_u16)
    assert d.max(initial=0) <= 1, f"max ulp diff {d.max()}"
    assert int((got_u16 != ref_u16).sum()) == 0, f"{int((d > 0).sum())} elements differ by 1 ulp"


# ------------------------------------------------------------------ layout

@pytest.mark.parametrize("name", FULL)
def test_layout_full_workloads(moe, orc, name):
    d = workload(name)
    wl = d["workload"]
    L = moe.moe_layout(to_dev(d["topk_idx"]), wl.E, wl.G)
    check_layout(L, orc.layout(d["topk_idx"], wl.E, wl.G))


# moe_layout on a plain stream takes the one-launch exchange layout for K <= 8 and
# up to 128 tiles of 256 tokens as its table allows (64 at E = 1024, G = 32; two
# lanes per token; E > 512 in two expert chunks), and count + place for K > 8 or
# more tiles
EDGE_SHAPES = [
    (0, 8, 256, 8), (1, 8, 256, 8), (1, 1, 1, 1), (255, 8, 256, 8), (256, 8, 256, 8),
    (257, 8, 256, 8), (1000, 1, 7, 7), (777, 32, 64, 32), (513, 6, 1024, 32), (4097, 8, 256, 1),
    (300, 2, 8, 8), (2000, 3, 12, 4), (1025, 8, 1000, 8), (600, 16, 16, 16),
    (2048, 8, 256, 8), (2049, 8, 256, 8), (4096, 4, 64, 8), (8192, 2, 8, 8), (5000, 3, 1024, 32),
    # every token takes every expert (K = E), with G = E, G = 1 and between
    (300, 32, 32, 32), (200, 8, 8, 1), (700, 16, 16, 4), (2500, 8, 8, 8),
    # ragged tile, K not 2/4/8, G = 32, exactly 16 tiles; E just above one expert chunk
    (3000, 7, 200, 8), (2300, 8, 256, 32), (4096, 8, 256, 8), (1500, 8, 520, 8),
    # at and past the exchange's limits: 64 tiles at the widest table row, 65 there
    # (count + place), 128 tiles, 129 (count + place with K <= 8)
    (16384, 8, 1024, 32), (16385, 8, 1024, 32), (32768, 8, 256, 8), (32769, 6, 64, 8),
]


@pytest.mark.parametrize("T,K,E,G", EDGE_SHAPES)
def test_layout_edge_shapes(moe, orc, T, K, E, G):
    idx = si.make_inputs(T, 8, E, K, seed=1000 + T + K + E)["topk_idx"]
    L = moe.moe_layout(to_dev(idx), E, G)
    check_layout(L, orc.layout(idx, E, G))


# seeds 0-5: 200-900 tokens, K 2-8 (odd K: the half-row split with K < 8); 6-8:
# 2100-4000 tokens, K = 8 (the exchange over 9-16 tiles)
@pytest.mark.parametrize("seed", range(9))
def test_layout_invalid_entries(moe, orc, seed):
    rng = np.random.default_rng(seed)
    T, K, E, G = int(rng.integers(200, 900)), int(rng.integers(2, 9)), 64, 8
    if seed >= 6:
        T, K = int(rng.integers(2100, 4000)), 8
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)           # repeats likely
    bad = rng.random((T, K)) < 0.05
    idx[bad] = rng.choice([-1, -7, E, E + 5, 1 << 30], size=int(bad.sum()))
    L = moe.moe_layout(to_dev(idx), E, G)
    Lo = orc.layout(idx, E, G)
    assert Lo["status"] == 3
    check_layout(L, Lo)


@pytest.mark.parametrize("T", [1500, 2500])   # one launch; count + place
def test_layout_reuses_buffers_without_stale_state(moe, orc, T):
    """A layout written into buffers that hold an earlier, different layout equals a
    fresh one (the stale-map hazard of cached routing)."""
    a = si.make_inputs(T, 8, 256, 8, seed=41)["topk_idx"]
    b = si.make_inputs(T, 8, 256, 8, seed=42)["topk_idx"]
    b[:7, 3] = 999                                                    # invalid entries in b
    L = moe.moe_layout(to_dev(a), 256, 8)
    L = moe.moe_layout(to_dev(b), 256, 8, out=L)
    check_layout(L, orc.layout(b, 256, 8))
    L = moe.moe_layout(to_dev(a), 256, 8, out=L)
    check_layout(L, orc.layout(a, 256, 8))                           # status cleared again


@pytest.mark.parametrize("T", [1500, 4096, 4097])   # offsets in the dispatch (two sizes); finalize kernel
def test_fused_call_reuses_buffers_without_stale_state(moe, orc, T):
    """moe_layout_dispatch into a layout, workspace and receive buffers that hold an
    earlier, different call's results equals a fresh call: the per-tile bases and the
    status of the earlier call must not leak into the next."""
    E, G, K, H = 256, 8, 8, 256
    a = si.make_inputs(T, H, E, K, seed=43)
    b = si.make_inputs(T, H, E, K, seed=44)
    b["topk_idx"][:5, 2] = -3                                         # invalid entries in b
    L = moe.Layout.empty(T, K, E, G)
    D = moe.alloc_dispatch(L, H, "expert", "bf16")
    for d in (a, b, a):
        x = dev_bf16(d["x"])
        L, D = moe.moe_layout_dispatch(to_dev(d["topk_idx"]), E, G, x, to_dev(d["topk_w"]), "expert",
                                       out_layout=L, out=D)
        Lo = orc.layout(d["topk_idx"], E, G)
        check_layout(L, Lo)
        R = Lo["R_expert"]
        src = Lo["recv_src_e"][:R] // K
        assert torch.equal(D.recv_x[:R].view(torch.int16).cpu(), x.view(torch.int16).cpu()[torch.from_numpy(src).long()])


def test_fused_fp8_placing_form():
    """The fused call's placing FP8 form at every batch size, including those the default
    routing sends through moe_layout + the plain dispatch, matches the oracle; run in a
    process of its own so the knob takes effect."""
    env = dict(os.environ, MOE_EP_FUSED_FP8_PLACE_MAX_T="1000000")
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_place_child.py")
    r = subprocess.run([sys.executable, "-u", child], env=env, capture_output=True, text=True, timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("wait", ["0", "-1"])
def test_sync_fallback_is_exact(wait):
    """The placing dispatch's bounded wait for its tile's bases, cut short from the
    host in a process of its own: with a wait limit of 0 ticks the tokens whose bases
    are not written at their first poll, and with -1 every token, compute the bases
    themselves from the count table; every layout array and receive row is still
    exactly the oracle's, and only the diagnostic status bit is added."""
    env = dict(os.environ, MOE_EP_BASE_WAIT_TICKS=wait)
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sync_fallback_child.py")
    r = subprocess.run([sys.executable, "-u", child], env=env, capture_output=True, text=True, timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


def test_check_status_raises_on_bad_input(moe):
    """Layout.check_status() reads the device status word and raises on its error bits
    (here an index out of range, then a repeated expert); a clean layout returns 0."""
    L = moe.moe_layout(to_dev(np.array([[0, 1], [2, 9]], np.int32)), 8, 4)
    with pytest.raises(moe.MoeDataError) as ei:
        L.check_status()
    assert ei.value.status & moe.STATUS_BAD_INDEX
    L = moe.moe_layout(to_dev(np.array([[0, 1], [3, 3]], np.int32)), 8, 4)
    with pytest.raises(moe.MoeDataError):
        L.check_status()
    L = moe.moe_layout(to_dev(np.array([[0, 1], [2, 3]], np.int32)), 8, 4)
    assert L.check_status() == 0


@pytest.mark.parametrize("T,K,E,G", [(700, 8, 256, 8), (300, 4, 64, 4), (513, 2, 16, 8)])
def test_layout_slot_arrays_4_byte_aligned(moe, orc, T, K, E, G):
    """Slot arrays that are 4-byte but not 16-byte aligned (allowed by the ABI) take
    the scalar store path and give the same layout."""
    idx = si.make_inputs(T, 8, E, K, seed=T + K)["topk_idx"]
    L = moe.Layout.empty(T, K, E, G)
    for name, n in (("slot_e", T * K), ("slot_g", T * K), ("slot_tg", T * G)):
        buf = torch.empty(n + 1, dtype=torch.int32, device="cuda")
        setattr(L, name, buf[1:])
        assert getattr(L, name).data_ptr() % 16 != 0
    L = moe.moe_layout(to_dev(idx), E, G, out=L)
    check_layout(L, orc.layout(idx, E, G))


# ------------------------------------------------------------------ dispatch

def dispatch_with_canary(moe, L, x, w, idx, mode, dtype="bf16"):
    H = x.shape[1]
    D = moe.alloc_dispatch(L, H, mode, dtype, device="cuda")
    if dtype == "bf16":
        D.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    else:
        D.recv_x.fill_(0xA5)
        D.recv_scale.fill_(-1.5)
    D.recv_topk_w.fill_(-3.0)
    D.recv_topk_idx.fill_(-77)
    return moe.moe_dispatch(L, x, w, idx, mode, dtype, out=D)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", FULL)
def test_dispatch_bf16_full_workloads(moe, orc, name, mode):
    d = workload(name)
    wl = d["workload"]
    idx_d = to_dev(d["topk_idx"])
    L = moe.moe_layout(idx_d, wl.E, wl.G)
    D = dispatch_with_canary(moe, L, dev_bf16(d["x"]), to_dev(d["topk_w"]), idx_d, mode)
    Lo = orc.layout(d["topk_idx"], wl.E, wl.G)
    Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])
    R = Do["R"]
    got = host_u16(D.recv_x)
    np.testing.assert_array_equal(got[:R], Do["recv_x"])
    assert np.all(got[R:] == CANARY16)
    w_got = D.recv_topk_w.cpu().numpy()
    np.testing.assert_array_equal(w_got[:R].view(np.uint32), Do["recv_w"].view(np.uint32))
    assert np.all(w_got[R:] == -3.0)
    i_got = D.recv_topk_idx.cpu().numpy()
    np.testing.assert_array_equal(i_got[:R], Do["recv_idx"])
    assert np.all(i_got[R:] == -77)


DISPATCH_EDGE = [  # (T, H, E, G, K): ragged / multi-pass hidden sizes, one group, one expert per group
    (1, 8, 8, 8, 2), (3, 520, 16, 4, 3), (129, 1024, 32, 8, 4), (40, 16392, 64, 8, 8),
    (300, 4096, 128, 1, 8), (77, 2048, 8, 8, 2), (513, 7168, 256, 8, 8), (50, 8200, 16, 16, 16),
    (60, 1024, 16, 4, 16), (5, 8, 1, 1, 1),   # K = E: every expert of every token; one expert
]


@pytest.mark.parametrize("T,H,E,G,K", DISPATCH_EDGE)
@pytest.mark.parametrize("mode", MODES)
def test_dispatch_bf16_edge_shapes(moe, orc, T, H, E, G, K, mode):
    d = si.make_inputs(T, H, E, K, seed=T + H + K)
    idx_d = to_dev(d["topk_idx"])
    L = moe.moe_layout(idx_d, E, G)
    D = dispatch_with_canary(moe, L, dev_bf16(d["x"]), to_dev(d["topk_w"]), idx_d, mode)
    Lo = orc.layout(d["topk_idx"], E, G)
    Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])
    got = host_u16(D.recv_x)
    np.testing.assert_array_equal(got[:Do["R"]], Do["recv_x"])
    assert np.all(got[Do["R"]:] == CANARY16)
    np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:Do["R"]], Do["recv_idx"])


@pytest.mark.parametrize("mode", MODES)
def test_dispatch_with_invalid_entries(moe, orc, mode):
    rng = np.random.default_rng(9)
    T, H, E, G, K = 333, 1024, 32, 4, 6
    d = si.make_inputs(T, H, E, K, seed=9)
    idx = d["topk_idx"].copy()
    idx[rng.random((T, K)) < 0.04] = 40          # out of range
    idx[5, 1] = idx[5, 0]                        # repeat
    idx_d = to_dev(idx)
    L = moe.moe_layout(idx_d, E, G)
    D = dispatch_with_canary(moe, L, dev_bf16(d["x"]), to_dev(d["topk_w"]), idx_d, mode)
    Lo = orc.layout(idx, E, G)
    Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], idx)
    got = host_u16(D.recv_x)
    np.testing.assert_array_equal(got[:Do["R"]], Do["recv_x"])
    assert np.all(got[Do["R"]:] == CANARY16)
    np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:Do["R"]], Do["recv_idx"])
    assert int(L.status.item()) == 3


def fp8_check(D, Do):
    R = Do["R"]
    q = D.recv_x.cpu().numpy()
    np.testing.assert_array_equal(q[:R], Do["recv_q"])
    assert np.all(q[R:] == 0xA5)
    s = D.recv_scale.cpu().numpy()
    np.testing.assert_array_equal(s[:R].view(np.uint32), Do["recv_scale"].view(np.uint32))
    assert np.all(s[R:] == -1.5)
    np.testing.assert_array_equal(D.recv_topk_w.cpu().numpy()[:R].view(np.uint32),
                                  Do["recv_w"].view(np.uint32))
    np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:R], Do["recv_idx"])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["fp8", "t256", "skew", "tiny"])
def test_dispatch_fp8_full_workloads(moe, orc, name, mode):
    d = workload(name)
    wl = d["workload"]
    idx_d = to_dev(d["topk_idx"])
    L = moe.moe_layout(idx_d, wl.E, wl.G)
    D = dispatch_with_canary(moe, L, dev_bf16(d["x"]), to_dev(d["topk_w"]), idx_d, mode, "fp8")
    Lo = orc.layout(d["topk_idx"], wl.E, wl.G)
    fp8_check(D, orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], d["topk_idx"]))


def adversarial_rows(T, H, seed):
    """bf16 rows whose 128-blocks stress the conversion: amax exactly 448 (scale 1,
    codes = RNE of the inputs), e4m3 midpoints, subnormal codes, signed zeros,
    all-zero blocks, huge and tiny magnitudes, bf16 subnormals next to normals."""
    import oracle
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, H)) * rng.choice([1e-3, 1, 30, 1e4], size=(T, 1))).astype(np.float32)
    codes = np.array([oracle.e4m3_to_f32(c) for c in range(127)], np.float64)
    mids = ((codes[:-1] + codes[1:]) / 2).astype(np.float32)
    nb = H // 128
    for t in range(T):
        for b in range(nb):
            kind = (t * nb + b) % 6
            blk = x[t, b * 128:(b + 1) * 128]
            if kind == 0:          # amax 448, midpoints and codes themselves
                blk[:] = rng.choice(np.concatenate([mids, -mids, codes.astype(np.float32)]), 128)
                blk[rng.integers(128)] = 448.0 * rng.choice([-1, 1])
            elif kind == 1:        # zeros of both signs, one block all zero
                blk[:] = 0.0 if t % 2 else -0.0
            elif kind == 2:        # one large element, the rest land on subnormal e4m3 codes
                blk[:] = rng.standard_normal(128) * 0.3
                blk[rng.integers(128)] = 3.0e4
            elif kind == 3:        # bf16 subnormals next to a unit element
                blk[:] = rng.standard_normal(128).astype(np.float32) * np.float32(1e-39)
                blk[0] = 1.0
            elif kind == 4:        # huge magnitudes
                blk[:] = rng.standard_normal(128) * 1e30
    import torch as _t
    return _t.from_numpy(x).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,H,E,G,K", [(96, 1024, 16, 4, 4), (50, 8320, 32, 8, 8), (7, 128, 8, 8, 2)])
def test_dispatch_fp8_adversarial_blocks(moe, orc, mode, T, H, E, G, K):
    d = si.make_inputs(T, 8, E, K, seed=T + H)
    x = adversarial_rows(T, H, seed=H)
    idx_d = to_dev(d["topk_idx"])
    L = moe.moe_layout(idx_d, E, G)
    D = dispatch_with_canary(moe, L, dev_bf16(x), to_dev(d["topk_w"]), idx_d, mode, "fp8")
    Lo = orc.layout(d["topk_idx"], E, G)
    fp8_check(D, orc.dispatch_fp8(Lo, mode, x, d["topk_w"], d["topk_idx"]))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("H", [2056, 3072, 5120, 6144, 6152, 8192])   # 3..8 vectors per lane, two ragged
@pytest.mark.parametrize("T", [300, 1500])
def test_dispatch_bf16_every_vector_count(moe, orc, mode, H, T):
    """The bf16 dispatch at every vector count per lane it compiles, plain and through
    the fused call (the placing instances), with ragged last passes. At T = 300 the
    plain dispatch takes its split form (a workgroup per token and row slice, while
    T x slices <= 4096), at T = 1500 the whole-row form."""
    E, G, K = 64, 8, 8
    d = si.make_inputs(T, H, E, K, seed=H + 3)
    idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])
    Lo = orc.layout(d["topk_idx"], E, G)
    Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])
    R = Do["R"]
    L = moe.moe_layout(idx_d, E, G)
    D = dispatch_with_canary(moe, L, x_d, w_d, idx_d, mode)
    L2 = moe.Layout.empty(T, K, E, G)
    D2 = moe.alloc_dispatch(L2, H, mode, "bf16")
    D2.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    L2, D2 = moe.moe_layout_dispatch(idx_d, E, G, x_d, w_d, mode, out_layout=L2, out=D2)
    check_layout(L2, Lo)
    for got in (D, D2):
        rx = host_u16(got.recv_x)
        np.testing.assert_array_equal(rx[:R], Do["recv_x"])
        assert np.all(rx[R:] == CANARY16)
        np.testing.assert_array_equal(got.recv_topk_idx.cpu().numpy()[:R], Do["recv_idx"])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("H", [2944, 4096, 5120, 6016, 8192])   # 3..8 passes of 64 lanes, two ragged
def test_dispatch_fp8_every_pass_count(moe, orc, mode, H):
    """The one-wave FP8 dispatch at every pass count it compiles (per-expert and
    per-group instances differ), plain and through the fused call, on adversarial
    blocks."""
    T, E, G, K = 200, 64, 8, 8
    d = si.make_inputs(T, 8, E, K, seed=H)
    x = adversarial_rows(T, H, seed=H + 1)
    idx_d, w_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"])
    Lo = orc.layout(d["topk_idx"], E, G)
    Do = orc.dispatch_fp8(Lo, mode, x, d["topk_w"], d["topk_idx"])
    L = moe.moe_layout(idx_d, E, G)
    fp8_check(dispatch_with_canary(moe, L, dev_bf16(x), w_d, idx_d, mode, "fp8"), Do)
    L2 = moe.Layout.empty(T, K, E, G)
    D2 = moe.alloc_dispatch(L2, H, mode, "fp8")
    D2.recv_x.fill_(0xA5)
    D2.recv_scale.fill_(-1.5)
    L2, D2 = moe.moe_layout_dispatch(idx_d, E, G, dev_bf16(x), w_d, mode, "fp8", out_layout=L2, out=D2)
    check_layout(L2, Lo)
    fp8_check(D2, Do)


@pytest.mark.parametrize("mode", MODES)
def test_fp8_dequant_matches_oracle(moe, orc, mode):
    d = workload("fp8") if mode == "expert" else workload("t256")
    wl = d["workload"]
    idx_d = to_dev(d["topk_idx"])
    L = moe.moe_layout(idx_d, wl.E, wl.G)
    D = moe.moe_dispatch(L, dev_bf16(d["x"]), to_dev(d["topk_w"]), idx_d, mode, "fp8")
    y = torch.full((D.recv_x.shape[0], wl.H), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode, out=y)
    Lo = orc.layout(d["topk_idx"], wl.E, wl.G)
    Do = orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])
    yo = orc.dequant_fp8(Do["recv_q"], Do["recv_scale"])
    got = host_u16(y)
    np.testing.assert_array_equal(got[:Do["R"]], yo)
    assert np.all(got[Do["R"]:] == host_u16(torch.tensor([7.0], dtype=torch.bfloat16))[0])


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", FULL)
def test_combine_full_workloads(moe, orc, name, mode):
    """Expert outputs y: the dispatched rows (identity) for bf16 workloads, the
    dequantised FP8 rows for the FP8 workload, each compared with the oracle's
    fma chain; plus a non-identity y (random rows) to exercise every slot."""
    d = workload(name)
    wl = d["workload"]
    idx_d, w_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"])
    L = moe.moe_layout(idx_d, wl.E, wl.G)
    Lo = orc.layout(d["topk_idx"], wl.E, wl.G)
    if wl.fp8:
        D = moe.moe_dispatch(L, dev_bf16(d["x"]), w_d, idx_d, mode, "fp8")
        y = moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode)
        Do = orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])
        y_ref = orc.dequant_fp8(Do["recv_q"], Do["recv_scale"])
    else:
        D = moe.moe_dispatch(L, dev_bf16(d["x"]), w_d, idx_d, mode)
        y = D.recv_x
        y_ref = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])["recv_x"]
    out = moe.moe_combine(L, y, w_d, mode)
    ref = orc.combine(Lo, mode, y_ref, d["topk_w"])
    got = host_u16(out)
    assert_combine_equal(got, ref)
    if not wl.fp8:
        np.testing.assert_array_equal(got, d["x"])           # identity round trip
    # random expert outputs (every receive row different from its source)
    rng = np.random.default_rng(wl.seed)
    R = y_ref.shape[0]
    yr = torch.from_numpy(rng.standard_normal((R, wl.H), dtype=np.float32)).to(torch.bfloat16)
    yr_u16 = yr.view(torch.int16).numpy().view(np.uint16)
    out = moe.moe_combine(L, dev_bf16(yr_u16), w_d, mode)
    assert_combine_equal(host_u16(out), orc.combine(Lo, mode, yr_u16, d["topk_w"]))


COMBINE_EDGE = [(1, 8, 8, 8, 2), (3, 520, 16, 4, 3), (200, 1024, 32, 8, 5), (40, 16392, 64, 8, 8),
                (300, 4096, 128, 1, 8), (100, 2048, 64, 32, 32), (77, 7168, 256, 8, 4),
                (90, 3072, 96, 4, 6), (64, 2048, 32, 32, 32), (33, 1024, 8, 2, 8), (5, 8, 1, 1, 1),
                # two vectors per lane (rows of 1025-2048 whole waves' vectors), and the 128-thread
                # form at 2, 4 and 7 vectors per lane with ragged passes
                (60, 12288, 64, 8, 8), (50, 16384, 32, 8, 5), (70, 1544, 32, 8, 8), (70, 3080, 32, 4, 6),
                (70, 6152, 64, 8, 8)]


@pytest.mark.parametrize("T,H,E,G,K", COMBINE_EDGE)
@pytest.mark.parametrize("mode", MODES)
def test_combine_edge_shapes(moe, orc, T, H, E, G, K, mode):
    d = si.make_inputs(T, H, E, K, seed=5 * T + H)
    idx_d, w_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"])
    L = moe.moe_layout(idx_d, E, G)
    Lo = orc.layout(d["topk_idx"], E, G)
    R = Lo["R_expert"] if mode == "expert" else Lo["R_group"]
    rng = np.random.default_rng(T)
    w = (rng.standard_normal((T, K)) * 2).astype(np.float32)        # any weights, any sign
    y = torch.from_numpy(rng.standard_normal((R, H), dtype=np.float32)).to(torch.bfloat16)
    y_u16 = y.view(torch.int16).numpy().view(np.uint16)
    out = moe.moe_combine(L, dev_bf16(y_u16), to_dev(w), mode)
    assert_combine_equal(host_u16(out), orc.combine(Lo, mode, y_u16, w))


def test_combine_skips_invalid_and_short_y(moe, orc):
    T, H, E, G, K = 150, 1024, 32, 4, 8
    d = si.make_inputs(T, H, E, K, seed=3)
    idx = d["topk_idx"].copy()
    idx[::7, 2] = -1
    idx[3, 5] = idx[3, 4]
    idx_d, w_d = to_dev(idx), to_dev(d["topk_w"])
    L = moe.moe_layout(idx_d, E, G)
    Lo = orc.layout(idx, E, G)
    for mode in MODES:
        D = moe.moe_dispatch(L, dev_bf16(d["x"]), w_d, idx_d, mode)
        R = Lo["R_expert"] if mode == "expert" else Lo["R_group"]
        y_ref = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], idx)["recv_x"]
        out = moe.moe_combine(L, D.recv_x, w_d, mode)
        assert_combine_equal(host_u16(out), orc.combine(Lo, mode, y_ref, d["topk_w"]))
        assert int(L.status.item()) == 3
        # y with too few rows: slots beyond it are skipped and reported
        short = R - 10
        out = moe.moe_combine(L, D.recv_x[:short].contiguous(), w_d, mode)
        torch.cuda.synchronize()
        assert int(L.status.item()) & moe.STATUS_Y_ROWS
        slot = (Lo["slot_e"] if mode == "expert" else Lo["slot_g"]).copy()
        slot[slot >= short] = -1
        Lc = dict(Lo, slot_e=slot, slot_g=slot)
        assert_combine_equal(host_u16(out), orc.combine(Lc, mode, y_ref, d["topk_w"]))
        moe.moe_layout(idx_d, E, G, out=L)      # restore status for the next mode


# ------------------------------------------------------------------ whole path

@pytest.mark.parametrize("name", ["t256", "skew"])
def test_path_is_deterministic(moe, name):
    """100 repeats of the whole path give the same bits: the layout arrays, bf16 and
    FP8 dispatch in both layouts, combine, and the fused call (an order-dependent race
    would show as a difference). Compared on the device against the first repeat."""
    d = workload(name)
    wl = d["workload"]
    idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])

    def run():
        L = moe.moe_layout(idx_d, wl.E, wl.G)
        re, rg = int(L.expert_offset[-1].item()), int(L.group_offset[-1].item())
        # (the receive lists are defined up to the row counts; the rest is untouched)
        outs = [L.slot_e, L.slot_g, L.slot_tg, L.recv_src_e[:re], L.recv_src_g[:rg], L.expert_offset,
                L.group_offset]
        for mode in MODES:
            D = moe.moe_dispatch(L, x_d, w_d, idx_d, mode)
            R = int((L.expert_offset if mode == "expert" else L.group_offset)[-1].item())
            outs += [D.recv_x[:R].view(torch.int16), moe.moe_combine(L, D.recv_x, w_d, mode).view(torch.int16)]
            Dq = moe.moe_dispatch(L, x_d, w_d, idx_d, mode, "fp8")
            outs += [Dq.recv_x[:R], Dq.recv_scale[:R]]
        Lf, Df = moe.moe_layout_dispatch(idx_d, wl.E, wl.G, x_d, w_d, "expert")
        outs += [Lf.slot_e, Df.recv_x[:int(Lf.expert_offset[-1].item())].view(torch.int16)]
        return [o.clone() for o in outs]

    first = run()
    for rep in range(99):
        for i, (a, b) in enumerate(zip(first, run())):
            assert torch.equal(a, b), (rep, i)


def test_stream_ordering_on_side_stream(moe, orc):
    """Calls on a non-default stream are ordered by that stream alone."""
    d = workload("t256")
    wl = d["workload"]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])
        L = moe.moe_layout(idx_d, wl.E, wl.G)
        D = moe.moe_dispatch(L, x_d, w_d, idx_d, "group")
        out = moe.moe_combine(L, D.recv_x, w_d, "group")
    s.synchronize()
    np.testing.assert_array_equal(host_u16(out), d["x"])


# ------------------------------------------------------------------ fused layout + dispatch

# (T, H, E, G, K). Forms: one launch for T * K * E <= 4096 (and for T <= 512 without a
# workspace); else (K <= 8) the count kernel + a placing dispatch whose workgroup 0 computes
# the offsets (up to 16 tiles and 4 expert columns per thread; beyond, an offsets
# workgroup in between); K > 8, the two calls
FUSED_SHAPES = [
    (1, 8, 8, 8, 2), (16, 2048, 8, 8, 2), (256, 7168, 256, 8, 8), (512, 1024, 64, 8, 8),
    (300, 520, 16, 4, 3), (100, 1024, 1024, 32, 32), (511, 4096, 128, 1, 8), (77, 2048, 7, 7, 1),
    (257, 1152, 96, 4, 6),
    (513, 1024, 64, 8, 8), (1000, 512, 32, 4, 3), (2000, 256, 16, 16, 1), (777, 384, 40, 1, 5),
    (600, 256, 64, 8, 13), (4097, 2048, 256, 8, 8), (3000, 128, 1024, 32, 8), (1030, 512, 64, 8, 8),
    (600, 8320, 32, 8, 8),    # rows over 8192: multi-pass placing bf16 dispatch
    (1100, 8320, 32, 8, 8),   # rows over 8192: multi-pass placing bf16 dispatch; FP8 takes the two calls
    (2000, 1024, 200, 8, 8),  # offsets computed in the dispatch: a partial second round of columns
    (1500, 256, 256, 32, 8),  # ... with 32 groups
]


def _fused_cases():
    # FP8 needs H % 128 == 0; the call without a workspace (one launch) takes
    # T <= 512 and T * K <= 16384 only
    for T, H, E, G, K in FUSED_SHAPES:
        for dtype in ("bf16", "fp8"):
            if dtype == "fp8" and H % 128:
                continue
            for use_ws in (True, False):
                if not use_ws and (T > 512 or T * K > 16384):
                    continue
                yield pytest.param(T, H, E, G, K, dtype, use_ws,
                                   id=f"{T}-{H}-{E}-{G}-{K}-{dtype}-{'auto' if use_ws else 'one_launch'}")


@pytest.mark.parametrize("T,H,E,G,K,dtype,use_ws", list(_fused_cases()))
@pytest.mark.parametrize("mode", MODES)
def test_fused_layout_dispatch_matches_oracle(moe, orc, T, H, E, G, K, mode, dtype, use_ws):
    if not use_ws:
        assert T <= moe.FUSED_MAX_TOKENS and T * K <= moe.FUSED_MAX_PAIRS
    d = si.make_inputs(T, H, E, K, seed=7 * T + H + K)
    idx = d["topk_idx"].copy()
    if T > 40:
        idx[T // 3, 0] = E + 3                 # out of range
        if K > 1:
            idx[T // 2, 1] = idx[T // 2, 0]    # repeat
    idx_d = to_dev(idx)
    x = dev_bf16(d["x"])
    L = moe.Layout.empty(T, K, E, G)
    D = moe.alloc_dispatch(L, H, mode, dtype)
    if dtype == "bf16":
        D.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    else:
        D.recv_x.fill_(0xA5)
        D.recv_scale.fill_(-1.5)
    D.recv_topk_w.fill_(-3.0)
    D.recv_topk_idx.fill_(-77)
    L, D = moe.moe_layout_dispatch(idx_d, E, G, x, to_dev(d["topk_w"]), mode, dtype, out_layout=L, out=D,
                                   use_workspace=use_ws)
    Lo = orc.layout(idx, E, G)
    check_layout(L, Lo)
    if dtype == "bf16":
        Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], idx)
        got = host_u16(D.recv_x)
        np.testing.assert_array_equal(got[:Do["R"]], Do["recv_x"])
        assert np.all(got[Do["R"]:] == CANARY16)
        np.testing.assert_array_equal(D.recv_topk_w.cpu().numpy()[:Do["R"]].view(np.uint32),
                                      Do["recv_w"].view(np.uint32))
        np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:Do["R"]], Do["recv_idx"])
    else:
        fp8_check(D, orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], idx))


@pytest.mark.parametrize("name", ["t4096", "skew", "fp8"])
@pytest.mark.parametrize("mode", MODES)
def test_fused_layout_dispatch_full_workloads(moe, orc, name, mode):
    d = workload(name)
    wl = d["workload"]
    dtype = "fp8" if wl.fp8 else "bf16"
    idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])
    L = moe.Layout.empty(wl.T, wl.K, wl.E, wl.G)
    D = moe.alloc_dispatch(L, wl.H, mode, dtype)
    if dtype == "bf16":
        D.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    else:
        D.recv_x.fill_(0xA5)
        D.recv_scale.fill_(-1.5)
    L, D = moe.moe_layout_dispatch(idx_d, wl.E, wl.G, x_d, w_d, mode, dtype, out_layout=L, out=D)
    Lo = orc.layout(d["topk_idx"], wl.E, wl.G)
    check_layout(L, Lo)
    for n in ("recv_src_e", "tok_group_mask"):
        R = Lo["R_expert"] if n == "recv_src_e" else wl.T
        assert np.array_equal(getattr(L, n).cpu().numpy()[:R].view(np.int32), Lo[n][:R].view(np.int32)), n
    P = Lo["R_group"]
    assert np.array_equal(L.recv_src_g.cpu().numpy()[:P], Lo["recv_src_g"][:P])
    if dtype == "bf16":
        Do = orc.dispatch_bf16(Lo, mode, d["x"], d["topk_w"], d["topk_idx"])
        got = host_u16(D.recv_x)
        np.testing.assert_array_equal(got[:Do["R"]], Do["recv_x"])
        assert np.all(got[Do["R"]:] == CANARY16)
        np.testing.assert_array_equal(D.recv_topk_idx.cpu().numpy()[:Do["R"]], Do["recv_idx"])
    else:
        fp8_check(D, orc.dispatch_fp8(Lo, mode, d["x"], d["topk_w"], d["topk_idx"]))


@pytest.mark.parametrize("name", ["t256", "t4096"])
def test_fused_layout_dispatch_equals_two_calls(moe, name):
    d = workload(name)
    wl = d["workload"]
    idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])
    for mode in MODES:
        L1 = moe.moe_layout(idx_d, wl.E, wl.G)
        D1 = moe.moe_dispatch(L1, x_d, w_d, idx_d, mode)
        L2, D2 = moe.moe_layout_dispatch(idx_d, wl.E, wl.G, x_d, w_d, mode)
        torch.cuda.synchronize()
        for n in LAYOUT_ARRAYS + ("tok_group_mask",):
            assert torch.equal(getattr(L1, n), getattr(L2, n)), n
        Re, Pg = int(L1.expert_offset[wl.E].item()), int(L1.group_offset[wl.G].item())
        assert torch.equal(L1.recv_src_e[:Re], L2.recv_src_e[:Re])
        assert torch.equal(L1.recv_src_g[:Pg], L2.recv_src_g[:Pg])
        R = int(L1.rows(mode).item())
        assert torch.equal(D1.recv_x[:R].view(torch.int16), D2.recv_x[:R].view(torch.int16))
        out1 = moe.moe_combine(L1, D1.recv_x, w_d, mode)
        out2 = moe.moe_combine(L2, D2.recv_x, w_d, mode)
        assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


# ------------------------------------------------------------------ receive-side regroup

REGROUP_SHAPES = [("t256", None), ("skew", None), ("fp8", None), ("tiny", None),
                  (None, (300, 520, 16, 4, 3)), (None, (129, 1024, 64, 1, 8)), (None, (50, 16392, 64, 8, 8)),
                  # 3, 5, 6 and 8 vectors per lane (bf16); 2 and 3 ragged, 3 and 4 whole (FP8)
                  (None, (200, 3072, 32, 8, 8)), (None, (200, 5120, 32, 8, 8)), (None, (200, 6144, 64, 8, 8)),
                  (None, (100, 8192, 32, 8, 8))]
# FP8 needs H % 128 == 0: not for H = 520 or 16392
REGROUP_CASES = [(n, s, dt) for n, s in REGROUP_SHAPES for dt in ("bf16", "fp8")
                 if not (dt == "fp8" and s is not None and s[1] % 128)]


@pytest.mark.parametrize("name,shape,dtype", REGROUP_CASES)
def test_regroup_matches_expert_dispatch(moe, orc, name, shape, dtype):
    if name:
        d = workload(name)
        wl = d["workload"]
        T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
        idx = d["topk_idx"]
    else:
        T, H, E, G, K = shape
        d = si.make_inputs(T, H, E, K, seed=T + H)
        idx = d["topk_idx"].copy()
        idx[T // 2, 0] = -3                    # an invalid entry is skipped
    assert dtype == "bf16" or H % 128 == 0
    idx_d, w_d, x_d = to_dev(idx), to_dev(d["topk_w"]), dev_bf16(d["x"])
    L = moe.moe_layout(idx_d, E, G)
    Dg = moe.moe_dispatch(L, x_d, w_d, idx_d, "group", dtype)
    De = moe.alloc_dispatch(L, H, "expert", dtype)
    if dtype == "bf16":
        De.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    else:
        De.recv_x.fill_(0xA5)
        De.recv_scale.fill_(-1.5)
    De.recv_topk_w.fill_(-3.0)
    De.recv_topk_idx.fill_(-77)
    De = moe.moe_regroup(L, Dg, out=De)
    Lo = orc.layout(idx, E, G)
    if dtype == "bf16":
        Do = orc.dispatch_bf16(Lo, "expert", d["x"], d["topk_w"], idx)
        got = host_u16(De.recv_x)
        np.testing.assert_array_equal(got[:Do["R"]], Do["recv_x"])
        assert np.all(got[Do["R"]:] == CANARY16)
        np.testing.assert_array_equal(De.recv_topk_idx.cpu().numpy()[:Do["R"]], Do["recv_idx"])
        np.testing.assert_array_equal(De.recv_topk_w.cpu().numpy()[:Do["R"]].view(np.uint32),
                                      Do["recv_w"].view(np.uint32))
    else:
        fp8_check(De, orc.dispatch_fp8(Lo, "expert", d["x"], d["topk_w"], idx))


def test_regroup_of_arbitrary_rows(moe, orc):
    """Rows that are not a dispatch result: the kernel is the oracle's gather."""
    T, H, E, G, K = 333, 2048, 48, 6, 5
    d = si.make_inputs(T, H, E, K, seed=4)
    idx_d = to_dev(d["topk_idx"])
    L = moe.moe_layout(idx_d, E, G)
    Lo = orc.layout(d["topk_idx"], E, G)
    Dg = moe.alloc_dispatch(L, H, "group")
    rng = np.random.default_rng(1)
    rows = rng.integers(0, 1 << 16, size=tuple(Dg.recv_x.shape), dtype=np.uint16)
    wts = rng.standard_normal(tuple(Dg.recv_topk_w.shape)).astype(np.float32)
    ids = rng.integers(-5, 99, size=tuple(Dg.recv_topk_idx.shape)).astype(np.int32)
    Dg.recv_x.copy_(dev_bf16(rows))
    Dg.recv_topk_w.copy_(to_dev(wts))
    Dg.recv_topk_idx.copy_(to_dev(ids))
    De = moe.moe_regroup(L, Dg)
    R = Lo["R_expert"]
    np.testing.assert_array_equal(host_u16(De.recv_x)[:R], orc.regroup_rows(Lo, rows))
    np.testing.assert_array_equal(De.recv_topk_w.cpu().numpy()[:R], orc.regroup_rows(Lo, wts))
    np.testing.assert_array_equal(De.recv_topk_idx.cpu().numpy()[:R], orc.regroup_rows(Lo, ids))


# ------------------------------------------------------------------ per-expert FP8 cast + transpose

CT_CASES = [("t256", None), ("t4096", None), ("skew", None), ("tiny", None),
            (None, (300, 640, 16, 4, 3)), (None, (1000, 64, 1024, 32, 1)), (None, (37, 1024, 8, 1, 8))]


@pytest.mark.parametrize("name,shape", CT_CASES)
def test_cast_transpose_matches_oracle(moe, orc, name, shape):
    if name:
        d = workload(name)
        wl = d["workload"]
        T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    else:
        T, H, E, G, K = shape
        d = si.make_inputs(T, H, E, K, seed=3 * T + H)
    idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])
    L = moe.moe_layout(idx_d, E, G)
    D = moe.moe_dispatch(L, x_d, w_d, idx_d, "expert")
    rng = np.random.default_rng(T + E)
    scale = rng.uniform(0.25, 300.0, E).astype(np.float32)     # large scales saturate
    amax0 = (rng.random(E) * 3).astype(np.float32)              # accumulates into these
    CT = moe.moe_cast_transpose_fp8(L, D.recv_x, to_dev(scale), amax=to_dev(amax0))
    torch.cuda.synchronize()
    Lo = orc.layout(d["topk_idx"], E, G)
    De = orc.dispatch_bf16(Lo, "expert", d["x"], d["topk_w"], d["topk_idx"])
    ref = orc.cast_transpose_fp8(Lo["expert_offset"], De["recv_x"], scale, amax_in=amax0)
    np.testing.assert_array_equal(CT.pad_offset.cpu().numpy(), ref["pad_offset"])
    R = Lo["R_expert"]
    np.testing.assert_array_equal(CT.c[:R].cpu().numpy(), ref["c"])
    nt = H * int(ref["pad_offset"][-1])
    np.testing.assert_array_equal(CT.t[:nt].cpu().numpy(), ref["t"])
    np.testing.assert_array_equal(CT.amax.cpu().numpy().view(np.uint32), ref["amax"].view(np.uint32))


# ------------------------------------------------------------------ guards
# A layout not written by moe_layout() for these sizes (stale or corrupted) must
# not lead any kernel out of the buffers the host checked. Each case below leaves
# spare room around every buffer it corrupts an index into, so that even an
# unguarded access would stay in allocated memory; the checks are on the values.

def _padded_i32(n, pad=64):
    """An int32 [n] view of a buffer with `pad` more entries, all -1 (no slot)."""
    return torch.full((n + pad,), -1, dtype=torch.int32, device="cuda")[:n]


def test_guard_dispatch_skips_slots_outside_the_bound(moe, orc):
    T, H, E, G, K = 300, 256, 32, 4, 4
    d = si.make_inputs(T, H, E, K, seed=71)
    idx, w, x = d["topk_idx"], d["topk_w"], d["x"]
    idx_d, w_d, x_d = to_dev(idx), to_dev(w), dev_bf16(x)
    L = moe.moe_layout(idx_d, E, G)
    torch.cuda.synchronize()
    Lo = orc.layout(idx, E, G)
    bound = T * K
    L.slot_e[5 * K + 1] = bound + 3          # past the bound, inside the spare rows
    L.slot_e[9 * K + 0] = -5
    D = moe.alloc_dispatch(L, H, "expert", capacity=bound + 16)
    D.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    moe.moe_dispatch(L, x_d, w_d, idx_d, "expert", out=D)
    torch.cuda.synchronize()
    got = host_u16(D.recv_x)
    assert np.all(got[bound:] == CANARY16)
    Do = orc.dispatch_bf16(Lo, "expert", x, w, idx)
    R = Lo["R_expert"]
    skipped = [int(Lo["slot_e"][5 * K + 1]), int(Lo["slot_e"][9 * K + 0])]
    keep = np.ones(R, bool)
    keep[skipped] = False
    assert np.array_equal(got[:R][keep], Do["recv_x"][keep])
    assert np.all(got[skipped] == CANARY16)


def test_guard_regroup_skips_tokens_outside_the_batch(moe, orc):
    T, H, E, G, K = 300, 256, 32, 4, 4
    d = si.make_inputs(T, H, E, K, seed=72)
    idx, w, x = d["topk_idx"], d["topk_w"], d["x"]
    idx_d, w_d, x_d = to_dev(idx), to_dev(w), dev_bf16(x)
    L = moe.Layout.empty(T, K, E, G)
    L.slot_g, L.slot_e = _padded_i32(T * K), _padded_i32(T * K)   # room past token T - 1
    moe.moe_layout(idx_d, E, G, out=L)
    Dg = moe.moe_dispatch(L, x_d, w_d, idx_d, "group")
    torch.cuda.synchronize()
    Lo = orc.layout(idx, E, G)
    L.recv_src_g[3] = T                      # group row 3 names a token past the batch
    De = moe.alloc_dispatch(L, H, "expert")
    De.recv_x.view(torch.int16).fill_(int(CANARY16.astype(np.int16)))
    moe.moe_regroup(L, Dg, out=De)
    torch.cuda.synchronize()
    t3 = int(Lo["recv_src_g"][3])
    skipped = [int(Lo["slot_e"][t3 * K + k]) for k in range(K) if Lo["slot_g"][t3 * K + k] == 3]
    assert skipped
    Do = orc.dispatch_bf16(Lo, "expert", x, w, idx)
    R = Lo["R_expert"]
    got = host_u16(De.recv_x)
    keep = np.ones(R, bool)
    keep[skipped] = False
    assert np.array_equal(got[:R][keep], Do["recv_x"][keep])
    assert np.all(got[skipped] == CANARY16)


def test_guard_cast_transpose_writes_nothing_for_offsets_past_the_bound(moe, orc):
    T, H, E, G, K = 300, 256, 32, 4, 4
    d = si.make_inputs(T, H, E, K, seed=73)
    idx_d, w_d, x_d = to_dev(d["topk_idx"]), to_dev(d["topk_w"]), dev_bf16(d["x"])
    L = moe.moe_layout(idx_d, E, G)
    bound = T * K
    D = moe.alloc_dispatch(L, H, "expert", capacity=bound + 64)    # x rows to spare
    moe.moe_dispatch(L, x_d, w_d, idx_d, "expert", out=D)
    torch.cuda.synchronize()
    L.expert_offset[E] = bound + 8           # past T*K: not a layout of these sizes
    nb = H * (bound + 15 * E)                 # moe_cast_transpose_t_bytes(T, K, E, H)
    CT = moe.CastTransposed(torch.full((bound + 64, H), 0xA5, dtype=torch.uint8, device="cuda"),
                            torch.full((nb + 64 * H,), 0x5A, dtype=torch.uint8, device="cuda"),
                            torch.full((E,), 2.5, dtype=torch.float32, device="cuda"),
                            torch.full((E + 1,), -9, dtype=torch.int32, device="cuda"))
    scale = torch.full((E,), 16.0, dtype=torch.float32, device="cuda")
    moe.moe_cast_transpose_fp8(L, D.recv_x, scale, out=CT)
    torch.cuda.synchronize()
    assert bool((CT.c == 0xA5).all())
    assert bool((CT.t == 0x5A).all())
    assert bool((CT.amax == 2.5).all())
    assert bool((CT.pad_offset == -9).all())


# ------------------------------------------------------------------ non-finite values

def assert_bf16_equal_nan_by_class(got, want):
    """Bit-exact where the oracle's bf16 is not a NaN; a NaN where it is. The sign and
    payload of a NaN computed from NaN inputs are not unique (IEEE 754 leaves open
    which input's payload propagates), so only NaN-ness is compared there."""
    is_nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape
    wn = is_nan(want)
    np.testing.assert_array_equal(is_nan(got), wn)
    np.testing.assert_array_equal(got[~wn], want[~wn])
    return int(wn.sum())


def test_nonfinite_values_match_oracle(moe, orc):
    """Infinities and NaNs (both signs, quiet and signalling payloads) in the tokens'
    rows, including a 128-block that is all NaN and one that holds an infinity,
    through every call that computes on the values: FP8 dispatch (both layouts) and
    its dequantisation, combine, the cast-transpose and the one-launch fused FP8
    dispatch. FP8 codes and scales bit for bit as the oracle's (a NaN is the code
    0x7F; finite values and infinities saturate at +-448); bf16 rows copied by the
    dispatch bit for bit; bf16 results computed from the values (combine, dequant)
    bit for bit except that a NaN is compared as a NaN."""
    T, H, E, G, K = 300, 1024, 32, 4, 4
    d = si.make_inputs(T, H, E, K, seed=91)
    rng = np.random.default_rng(91)
    x = d["x"].copy()
    special = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF], np.uint16)
    pos = rng.choice(x.size, 400, replace=False)
    x.flat[pos] = rng.choice(special, 400)
    x[5, 128:256] = 0x7FC0                           # a block of NaNs
    x[7, 0] = 0x7F80                                 # an infinity in a block of finite values
    x[9, 512:640] = 0xFF80                           # a block of infinities
    idx, w = d["topk_idx"], d["topk_w"]
    idx_d, w_d, x_d = to_dev(idx), to_dev(w), dev_bf16(x)
    L = moe.moe_layout(idx_d, E, G)
    Lo = orc.layout(idx, E, G)
    check_layout(L, Lo)
    for mode in MODES:
        D = dispatch_with_canary(moe, L, x_d, w_d, idx_d, mode, "fp8")
        Do = orc.dispatch_fp8(Lo, mode, x, w, idx)
        fp8_check(D, Do)
        y = moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode)
        assert assert_bf16_equal_nan_by_class(host_u16(y)[:Do["R"]],
                                              orc.dequant_fp8(Do["recv_q"], Do["recv_scale"])) > 0
    De = moe.moe_dispatch(L, x_d, w_d, idx_d, "expert")
    Deo = orc.dispatch_bf16(Lo, "expert", x, w, idx)
    np.testing.assert_array_equal(host_u16(De.recv_x)[:Lo["R_expert"]], Deo["recv_x"])
    out = moe.moe_combine(L, De.recv_x, w_d, "expert")
    got = host_u16(out)
    assert assert_bf16_equal_nan_by_class(got, orc.combine(Lo, "expert", Deo["recv_x"], w)) > 0
    inf_rows = (x == 0x7F80).any(axis=1) | (x == 0xFF80).any(axis=1)
    assert np.any((got == 0x7F80) | (got == 0xFF80)) or not inf_rows.any()
    scale = rng.uniform(0.5, 50.0, E).astype(np.float32)
    CT = moe.moe_cast_transpose_fp8(L, De.recv_x, to_dev(scale))
    ref = orc.cast_transpose_fp8(Lo["expert_offset"], Deo["recv_x"], scale)
    np.testing.assert_array_equal(CT.c[:Lo["R_expert"]].cpu().numpy(), ref["c"])
    nt = H * int(ref["pad_offset"][-1])
    np.testing.assert_array_equal(CT.t[:nt].cpu().numpy(), ref["t"])
    np.testing.assert_array_equal(CT.amax.cpu().numpy().view(np.uint32), ref["amax"].view(np.uint32))
    L2 = moe.Layout.empty(T, K, E, G)
    D2 = moe.alloc_dispatch(L2, H, "expert", "fp8")
    D2.recv_x.fill_(0xA5)
    D2.recv_scale.fill_(-1.5)
    L2, D2 = moe.moe_layout_dispatch(idx_d, E, G, x_d, w_d, "expert", "fp8", out_layout=L2, out=D2,
                                     use_workspace=False)
    fp8_check(D2, orc.dispatch_fp8(Lo, "expert", x, w, idx))


# ------------------------------------------------------------------ FP8 over a wide dynamic range

def test_fp8_wide_dynamic_range_matches_oracle(moe, orc):
    """Rows whose 128-blocks have amax anywhere from 2^-110 to 2^120 and elements down to 40
    binades below their block's amax (e4m3 subnormal codes, values that round to zero,
    bf16 subnormal inputs), with exact zeros of both signs: FP8 dispatch in both layouts,
    dequantisation and cast-transpose (scales that saturate part of each expert) all bit
    for bit as the oracle's."""
    T, H, E, G, K = 200, 2048, 32, 4, 4
    d = si.make_inputs(T, H, E, K, seed=77)
    rng = np.random.default_rng(77)
    nb = H // 128
    block_e = rng.uniform(-110, 120, (T, nb, 1))                      # log2 of each block's amax
    below = rng.uniform(0, 40, (T, nb, 128))                           # binades below it
    below[:, :, 0] = 0                                                  # one element at the amax
    mag = np.exp2(block_e - below)
    sign = np.where(rng.random((T, nb, 128)) < 0.5, -1.0, 1.0)
    xf = (sign * mag).reshape(T, H).astype(np.float32)
    xf[rng.random((T, H)) < 0.05] = 0.0
    xf[rng.random((T, H)) < 0.02] = -0.0
    x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    amax = np.abs(bf.reshape(T, nb, 128)).max(axis=2)
    assert amax.min() > 2.0 ** -112 and np.isfinite(amax).all()        # inside the supported range
    assert np.any((np.abs(bf) < 2.0 ** -126) & (bf != 0))                # bf16 subnormal inputs occur
    idx, w = d["topk_idx"], d["topk_w"]
    idx_d, w_d, x_d = to_dev(idx), to_dev(w), dev_bf16(x)
    L = moe.moe_layout(idx_d, E, G)
    Lo = orc.layout(idx, E, G)
    for mode in MODES:
        D = dispatch_with_canary(moe, L, x_d, w_d, idx_d, mode, "fp8")
        Do = orc.dispatch_fp8(Lo, mode, x, w, idx)
        fp8_check(D, Do)
        y = moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode)
        np.testing.assert_array_equal(host_u16(y)[:Do["R"]], orc.dequant_fp8(Do["recv_q"], Do["recv_scale"]))
    De = moe.moe_dispatch(L, x_d, w_d, idx_d, "expert")
    Deo = orc.dispatch_bf16(Lo, "expert", x, w, idx)
    off = Lo["expert_offset"]
    rows = torch.from_numpy(Deo["recv_x"].view(np.int16)).view(torch.bfloat16).float().numpy()
    scale = np.ones(E, np.float32)
    for e in range(E):
        if off[e + 1] > off[e]:
            a = float(np.abs(rows[off[e]:off[e + 1]]).max())
            scale[e] = np.float32(448.0 / a * 2.0 ** rng.uniform(-4, 4))   # part of the rows saturate
    CT = moe.moe_cast_transpose_fp8(L, De.recv_x, to_dev(scale))
    ref = orc.cast_transpose_fp8(off, Deo["recv_x"], scale)
    np.testing.assert_array_equal(CT.c[:Lo["R_expert"]].cpu().numpy(), ref["c"])
    nt = H * int(ref["pad_offset"][-1])
    np.testing.assert_array_equal(CT.t[:nt].cpu().numpy(), ref["t"])
    np.testing.assert_array_equal(CT.amax.cpu().numpy().view(np.uint32), ref["amax"].view(np.uint32))


def test_combine_wide_dynamic_range_matches_oracle(moe, orc):
    """Expert outputs over the whole bf16 range (subnormals included) and weights from 2^-20
    to 2^20 of either sign: sums that overflow to infinity, that land in the bf16 subnormal
    range and that cancel to signed zeros, with the fma chain's k order. Bit for bit as the
    oracle's, a NaN (both infinities in one sum) compared as a NaN."""
    T, H, E, G, K = 300, 1024, 64, 8, 8
    d = si.make_inputs(T, H, E, K, seed=78)
    rng = np.random.default_rng(78)
    idx = d["topk_idx"]
    idx_d = to_dev(idx)
    L = moe.moe_layout(idx_d, E, G)
    Lo = orc.layout(idx, E, G)
    # a fifth of the tokens read only tiny rows with weights <= 1: their sums are subnormal
    tiny = rng.random(T) < 0.2
    wmag = np.where(tiny[:, None], np.exp2(rng.uniform(-4, 0, (T, K))), np.exp2(rng.uniform(-20, 20, (T, K))))
    w = (np.where(rng.random((T, K)) < 0.5, -1.0, 1.0) * wmag).astype(np.float32)
    for mode in MODES:
        R = Lo["R_expert"] if mode == "expert" else Lo["R_group"]
        mag = np.exp2(rng.uniform(-140, 127.9, (R, H)))
        sl = Lo["slot_e"].reshape(T, K) if mode == "expert" else Lo["slot_tg"].reshape(T, G)
        own = sl[tiny].ravel()                                        # rows of one token each
        own = own[own >= 0]
        mag[own] = np.exp2(rng.uniform(-140, -128, (own.size, H)))
        yf = (np.where(rng.random((R, H)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
        yf[rng.random((R, H)) < 0.05] = 0.0
        y_u16 = torch.from_numpy(yf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        out = host_u16(moe.moe_combine(L, dev_bf16(y_u16), to_dev(w), mode))
        ref = orc.combine(Lo, mode, y_u16, w)
        assert_bf16_equal_nan_by_class(out, ref)
        r = ref[(ref & 0x7FFF) <= 0x7F80]
        assert np.any((r & 0x7FFF) == 0x7F80)                                  # infinities
        assert np.any(((r & 0x7F80) == 0) & ((r & 0x7F) != 0))                 # subnormal results


# ------------------------------------------------------------------ buffers past 4 GiB

def test_receive_buffers_past_4gib(moe, orc):
    """40,000 tokens x 7168 bf16, top-8 of 256 experts: the per-expert receive buffer holds
    320,000 rows (4.6 GB, more than 2^31 elements), so every row offset must be 64-bit. The
    layout equals the oracle's; every receive row equals its source row (per-expert through
    the fused call, per-group through moe_dispatch); sampled FP8 receive rows equal the
    oracle's quantisation of their source rows; identity experts come back bit for bit
    through combine (weights summing to 1); sampled cast-transpose rows equal the oracle's
    encoding and every expert's transposed block is the transpose of its rows; the regroup
    of the per-group rows equals the per-expert dispatch. x is drawn on the GPU from a
    seeded generator."""
    T, H, E, G, K = 40000, 7168, 256, 8, 8
    d = si.make_inputs(T, 8, E, K, seed=99)            # routing and weights (x drawn below)
    idx, w = d["topk_idx"], d["topk_w"]
    gen = torch.Generator(device="cuda").manual_seed(99)
    x = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
    idx_d, w_d = to_dev(idx), to_dev(w)
    Lo = orc.layout(idx, E, G)

    L, D = moe.moe_layout_dispatch(idx_d, E, G, x, w_d, "expert")
    check_layout(L, Lo)
    R = Lo["R_expert"]
    assert R == T * K and R * H > 2 ** 31
    src_e = torch.from_numpy(Lo["recv_src_e"][:R].astype(np.int64)).cuda()
    for a in range(0, R, 32768):
        b = min(R, a + 32768)
        tok = src_e[a:b] // K
        assert torch.equal(D.recv_x[a:b].view(torch.int16), x[tok].view(torch.int16)), (a, b)
        assert torch.equal(D.recv_topk_idx[a:b], idx_d[tok]), (a, b)
    out = moe.moe_combine(L, D.recv_x, w_d, "expert")
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))
    del out

    # cast-transpose of the per-expert rows: sampled rows of C against the oracle's encoding
    # of x * scale, and every expert's T_e against the transpose of its C rows
    off = Lo["expert_offset"]
    scale = np.random.default_rng(98).uniform(4.0, 400.0, E).astype(np.float32)
    CT = moe.moe_cast_transpose_fp8(L, D.recv_x, to_dev(scale))
    po = CT.pad_offset.cpu().numpy()
    erows = np.random.default_rng(97).choice(R, 40, replace=False)
    for r in erows:
        e = int(np.searchsorted(off, r, side="right") - 1)
        xr = D.recv_x[int(r)].float().cpu().numpy()
        ref = orc.f32_to_e4m3_array((xr * scale[e]).astype(np.float32))
        np.testing.assert_array_equal(CT.c[int(r)].cpu().numpy(), ref)
    for e in range(E):
        n, npad = int(off[e + 1] - off[e]), int(po[e + 1] - po[e])
        assert npad == (n + 15) // 16 * 16
        te = CT.t[H * int(po[e]):H * int(po[e + 1])].view(H, npad)
        assert torch.equal(te[:, :n], CT.c[int(off[e]):int(off[e + 1])].t()), e
        assert not bool(te[:, n:].any()), e
    del CT

    # per-group dispatch, and its regroup into per-expert rows (equal to the dispatch above)
    Dg = moe.moe_dispatch(L, x, w_d, idx_d, "group")
    P = Lo["R_group"]
    src_g = torch.from_numpy(Lo["recv_src_g"][:P].astype(np.int64)).cuda()
    for a in range(0, P, 32768):
        b = min(P, a + 32768)
        assert torch.equal(Dg.recv_x[a:b].view(torch.int16), x[src_g[a:b]].view(torch.int16)), (a, b)
    Dr = moe.moe_regroup(L, Dg)
    assert torch.equal(Dr.recv_x[:R].view(torch.int16), D.recv_x[:R].view(torch.int16))
    assert torch.equal(Dr.recv_topk_idx[:R], D.recv_topk_idx[:R])
    del Dg, Dr, D

    Df = moe.moe_dispatch(L, x, w_d, idx_d, "expert", "fp8")
    rng = np.random.default_rng(99)
    rows = np.concatenate([rng.choice(R, 60, replace=False), [0, R - 1]])
    for r in rows:
        t = int(Lo["recv_src_e"][r]) // K
        xr = x[t].view(torch.int16).cpu().numpy().view(np.uint16)
        q, s = orc.quantize_row_fp8(xr)
        np.testing.assert_array_equal(Df.recv_x[int(r)].cpu().numpy(), q)
        np.testing.assert_array_equal(Df.recv_scale[int(r)].cpu().numpy().view(np.uint32), s.view(np.uint32))


# ------------------------------------------------------------------ guard bands

GUARD_BYTES = 4096


class Guarded:
    """Views into allocations that carry a filled band of GUARD_BYTES on each side."""

    def __init__(self):
        self.bases = []

    def __call__(self, shape, dtype, fill=0):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        base = torch.empty(n + 2 * GUARD_BYTES, dtype=torch.uint8, device="cuda")
        base.fill_(0xC3)
        view = base[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)
        view.view(torch.uint8).fill_(fill)
        self.bases.append((base, n))
        return view

    def intact(self):
        for base, n in self.bases:
            if not (bool((base[:GUARD_BYTES] == 0xC3).all()) and bool((base[GUARD_BYTES + n:] == 0xC3).all())):
                return False
        return True


@pytest.mark.parametrize("T,H,E,G,K", [(300, 1024, 32, 4, 4), (2100, 512, 64, 8, 8), (77, 2048, 8, 8, 2)])
def test_guard_bands_untouched_by_every_call(moe, orc, T, H, E, G, K):
    """Every array a call writes sits between two filled 4 KiB bands: layout (one launch
    and count + place), dispatch bf16 / FP8 in both layouts, the fused call, combine,
    regroup, cast-transpose and dequant leave the bands as they were; results still
    match the oracle."""
    g = Guarded()
    d = si.make_inputs(T, H, E, K, seed=T + H)
    idx, w, x = d["topk_idx"], d["topk_w"], d["x"]
    idx_d, w_d, x_d = to_dev(idx), to_dev(w), dev_bf16(x)
    Lo = orc.layout(idx, E, G)
    L = moe.Layout.empty(T, K, E, G)
    for name, n in (("expert_count", E), ("expert_offset", E + 1), ("group_count", G), ("group_offset", G + 1),
                    ("tok_group_mask", T), ("slot_e", T * K), ("slot_g", T * K), ("slot_tg", T * G),
                    ("recv_src_e", T * K), ("recv_src_g", T * min(K, G)), ("status", 1)):
        setattr(L, name, g((n,), torch.int32))
    L.workspace = g((L.workspace.numel(),), torch.uint8)
    moe.moe_layout(idx_d, E, G, out=L)
    check_layout(L, Lo)

    def recv(mode, dtype):
        cap = moe.recv_rows_bound(T, K, G, mode)
        fp8 = dtype == "fp8"
        return moe.Dispatched(g((cap, H), torch.uint8 if fp8 else torch.bfloat16),
                              g((cap, H // 128), torch.float32) if fp8 else None,
                              g((cap, K), torch.float32), g((cap, K), torch.int32))

    Ds = {}
    for mode in MODES:
        for dtype in ("bf16", "fp8"):
            if dtype == "fp8" and H % 128:
                continue
            Ds[mode, dtype] = moe.moe_dispatch(L, x_d, w_d, idx_d, mode, dtype, out=recv(mode, dtype))
        out = g((T, H), torch.bfloat16)
        moe.moe_combine(L, Ds[mode, "bf16"].recv_x, w_d, mode, out=out)
        Do = orc.dispatch_bf16(Lo, mode, x, w, idx)
        assert_combine_equal(host_u16(out), orc.combine(Lo, mode, Do["recv_x"], w))
    Dr = moe.moe_regroup(L, Ds["group", "bf16"], out=recv("expert", "bf16"))
    R = Lo["R_expert"]
    assert torch.equal(Dr.recv_x[:R].view(torch.int16), Ds["expert", "bf16"].recv_x[:R].view(torch.int16))
    if H % 128 == 0:
        y = g((moe.recv_rows_bound(T, K, G, "expert"), H), torch.bfloat16)
        moe.moe_fp8_dequant(L, Ds["expert", "fp8"].recv_x, Ds["expert", "fp8"].recv_scale, "expert", out=y)
        nb = moe._lib.moe_cast_transpose_t_bytes(T, K, E, H)
        CT = moe.CastTransposed(g((R, H), torch.uint8), g((max(nb, 16),), torch.uint8),
                                g((E,), torch.float32), g((E + 1,), torch.int32))
        moe.moe_cast_transpose_fp8(L, Ds["expert", "bf16"].recv_x, to_dev(np.full(E, 3.0, np.float32)), out=CT)
        rows_e = orc.dispatch_bf16(Lo, "expert", x, w, idx)["recv_x"]
        ref = orc.cast_transpose_fp8(Lo["expert_offset"], rows_e, np.full(E, 3.0, np.float32))
        np.testing.assert_array_equal(CT.c.cpu().numpy(), ref["c"][:R])
    L2 = moe.Layout.empty(T, K, E, G)
    for name in ("slot_e", "slot_g", "slot_tg", "recv_src_e", "recv_src_g", "tok_group_mask"):
        setattr(L2, name, g((getattr(L2, name).numel(),), torch.int32))
    L2.workspace = g((L2.workspace.numel(),), torch.uint8)
    moe.moe_layout_dispatch(idx_d, E, G, x_d, w_d, "expert", out_layout=L2, out=recv("expert", "bf16"))
    check_layout(L2, Lo)
    torch.cuda.synchronize()
    assert g.intact()


def test_binding_stream_is_torchs_current_stream(moe):
    """The binding's stream handle is torch's current stream, default and inside a
    side-stream context."""
    assert moe._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert moe._stream(None) == s.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert moe._stream(s) == s.cuda_stream
