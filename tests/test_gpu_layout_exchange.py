"""GPU tests of moe_layout's one-launch form that exchanges per-tile counts between
its workgroups through tagged tables in library memory (one table per stream):
the wait for the other tiles cut short from the host (every workgroup then counts
the tokens itself), calls of different shapes back to back on one stream (stale
entries of other shapes and earlier calls in the table), layouts on several
streams at once, and more streams than the library has tables (the later streams
take the two-launch layout). Every result is checked against the oracle, array by
array, bit for bit."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

NAMES = ("expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask", "slot_e", "slot_g",
         "slot_tg")


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_layout_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def check(L, Lo, what):
    assert int(L.status.item()) == Lo["status"], what
    for n in NAMES:
        got = getattr(L, n).cpu().numpy()
        if n == "tok_group_mask":   # uint32 bits held as int32 (group 31 is the sign bit)
            got = got.view(np.uint32)
        np.testing.assert_array_equal(got.astype(np.int64), Lo[n].astype(np.int64), err_msg=f"{what} {n}")
    np.testing.assert_array_equal(L.recv_src_e.cpu().numpy()[:Lo["R_expert"]], Lo["recv_src_e"][:Lo["R_expert"]])
    np.testing.assert_array_equal(L.recv_src_g.cpu().numpy()[:Lo["R_group"]], Lo["recv_src_g"][:Lo["R_group"]])


@pytest.mark.parametrize("wait", ["0", "-1"])
def test_exchange_wait_cut_short(wait):
    """With a wait limit of 0 ticks a workgroup that does not find every tile's
    counts at its first read counts the tokens itself; with -1 every workgroup does.
    The layout stays exactly the oracle's (checked in a process of its own, since
    the library reads the limit once per process)."""
    env = dict(os.environ, MOE_EP_BASE_WAIT_TICKS=wait)
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "layout_exchange_child.py")
    r = subprocess.run([sys.executable, "-u", child], env=env, capture_output=True, text=True, timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


def test_alternating_shapes_on_one_stream(moe, orc):
    """Layouts of different shapes and inputs queued back to back on one stream,
    with no synchronisation between them: each call's table holds entries of the
    other shape and of every earlier call, at other places; none may be taken."""
    shapes = [(4096, 256, 8, 8), (3000, 64, 8, 6), (1536, 128, 16, 4), (4096, 256, 8, 8), (513, 32, 4, 2)]
    runs = []
    for i in range(3):
        for j, (T, E, G, K) in enumerate(shapes):
            d = si.make_inputs(T, 128, E, K, seed=1000 + 10 * i + j)
            L = moe.Layout.empty(T, K, E, G)
            moe.moe_layout(torch.from_numpy(d["topk_idx"]).cuda(), E, G, out=L)
            runs.append((L, d["topk_idx"], E, G))
    torch.cuda.synchronize()
    for n, (L, idx, E, G) in enumerate(runs):
        check(L, orc.layout(idx, E, G), f"call {n}")


def test_layouts_on_several_streams_at_once(moe, orc):
    """Three streams each queue five layouts of their own inputs; the streams run
    concurrently and each has a table of its own."""
    streams = [torch.cuda.Stream() for _ in range(3)]
    runs = []
    for s_i, st in enumerate(streams):
        with torch.cuda.stream(st):
            for r in range(5):
                T, E, G, K = (4096, 256, 8, 8) if r % 2 == 0 else (2048, 128, 8, 8)
                d = si.make_inputs(T, 128, E, K, seed=2000 + 10 * s_i + r)
                idx = torch.from_numpy(d["topk_idx"]).cuda()
                L = moe.Layout.empty(T, K, E, G)
                moe.moe_layout(idx, E, G, out=L)
                runs.append((L, d["topk_idx"], E, G))
    torch.cuda.synchronize()
    for n, (L, idx, E, G) in enumerate(runs):
        check(L, orc.layout(idx, E, G), f"run {n}")


def test_more_streams_than_tables(moe, orc):
    """A layout on each of twelve streams, more than the library keeps tables for:
    the later streams take the two-launch layout, with the same results."""
    runs = []
    for s_i in range(12):
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            T, E, G, K = 3000, 256, 8, 8
            d = si.make_inputs(T, 128, E, K, seed=3000 + s_i)
            L = moe.Layout.empty(T, K, E, G)
            moe.moe_layout(torch.from_numpy(d["topk_idx"]).cuda(), E, G, out=L)
            runs.append((L, d["topk_idx"], E, G))
    torch.cuda.synchronize()
    for n, (L, idx, E, G) in enumerate(runs):
        check(L, orc.layout(idx, E, G), f"stream {n}")


def test_random_layouts_up_to_128_tiles(moe, orc):
    """60 random routing problems of 1-128 tiles (the exchange's range; past 16 tiles
    its reads take several rounds), top-k 1-8 (the two lanes of a token split its
    entries; odd K leaves the second lane short), E up to 1024 in G groups, with
    repeated experts at random positions of a token (within one lane's half and
    across the two halves) and out-of-range entries; every layout array against the
    oracle, bit for bit. Layouts that do not fit the exchange table take count +
    place, which is checked the same way."""
    rng = np.random.default_rng(20261203)
    for rnd in range(60):
        G = int(rng.choice([1, 4, 8, 32]))
        E = G * int(rng.choice([1, 2, 8, 32])) if G < 32 else 32 * int(rng.choice([1, 8, 32]))
        K = int(rng.integers(1, 9))
        K = min(K, E)
        T = int(rng.integers(1, 128 * 256 + 1))
        d = si.make_inputs(T, 8, E, K, seed=3000 + rnd, routing="zipf" if rnd % 3 == 0 else "uniform")
        idx = d["topk_idx"].copy()
        if K > 1 and rnd % 2 == 0:                       # repeats: random token, random positions
            n = int(rng.integers(1, 20))
            ts, k1 = rng.integers(0, T, n), rng.integers(1, K, n)
            k0 = (rng.random(n) * k1).astype(np.int64)   # an earlier position
            idx[ts, k1] = idx[ts, k0]
        if rnd % 5 == 0:                                  # out of range
            n = int(rng.integers(1, 10))
            idx[rng.integers(0, T, n), rng.integers(0, K, n)] = rng.choice([-1, E, E + 3, -100], n)
        what = f"round {rnd}: T={T} E={E} G={G} K={K}"
        print(what, flush=True)
        L = moe.moe_layout(torch.from_numpy(idx).cuda(), E, G)
        torch.cuda.synchronize()
        check(L, orc.layout(idx, E, G), what)
