"""Pins for the CPU oracle: each test ties an oracle function to something other
than itself — a hand-worked example, a library routine that computes the same
thing by another route, a closed form, an invariant, or a brute force on tiny
inputs. A dropped term, a wrong index or sign, or a transposed operand in the
oracle fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import synth_inputs as si


# ------------------------------------------------------------------ helpers

def bf16_bits_of(vals):
    t = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_float(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def rne_f32(q: Fraction) -> float:
    """Exact value -> nearest binary32, ties to even (subnormals included)."""
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** 128:
        return -math.inf if neg else math.inf
    f = float(v)
    return -f if neg else f


def fma_f32(a: float, b: float, c: float) -> float:
    """IEEE fused multiply-add in binary32, round to nearest even, from exact rationals.
    An exact zero sum is -0 only when both addends are -0 (or a -0 product meets -0)."""
    p = Fraction(a) * Fraction(b)
    s = p + Fraction(c)
    if s == 0:
        p_neg = (math.copysign(1.0, a) * math.copysign(1.0, b) < 0) if p == 0 else p < 0
        c_neg = math.copysign(1.0, c) < 0 if c == 0 else c < 0
        return -0.0 if (p_neg and c_neg) else 0.0
    return rne_f32(s)


# ------------------------------------------------------------------ hand-worked golden examples

def test_golden_layout_by_hand(orc, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "layout_hand_T4_E4_G2_K2.json")))
    idx = np.array(g["topk_idx"], np.int32)
    L = orc.layout(idx, g["E"], g["G"])
    assert L["status"] == 0
    for name in ("expert_count", "expert_offset", "group_count", "group_offset"):
        np.testing.assert_array_equal(L[name], g[name], err_msg=name)
    np.testing.assert_array_equal(L["slot_e"], np.ravel(g["slot_e"]))
    np.testing.assert_array_equal(L["slot_g"], np.ravel(g["slot_g"]))
    np.testing.assert_array_equal(L["slot_tg"], np.ravel(g["slot_tg"]))
    np.testing.assert_array_equal(L["tok_group_mask"], g["tok_group_mask"])
    np.testing.assert_array_equal(L["recv_src_e"][:L["R_expert"]], g["recv_src_e"])
    np.testing.assert_array_equal(L["recv_src_g"][:L["R_group"]], g["recv_src_g"])


def test_golden_combine_by_hand(orc, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "layout_hand_T4_E4_G2_K2.json")))
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    x = bf16_bits_of(g["x"])
    L = orc.layout(idx, g["E"], g["G"])
    epg = g["E"] // g["G"]
    for mode in ("expert", "group"):
        D = orc.dispatch_bf16(L, mode, x, w, idx)
        out = orc.combine(L, mode, D["recv_x"], w)
        np.testing.assert_array_equal(bf16_to_float(out), np.array(g["combine_identity"], np.float32))
    # per-expert scaled expert: receive row r of expert e is x * (1 + e)
    D = orc.dispatch_bf16(L, "expert", x, w, idx)
    e_of_row = np.searchsorted(L["expert_offset"], np.arange(L["R_expert"]), side="right") - 1
    y = bf16_bits_of(bf16_to_float(D["recv_x"]) * (1 + e_of_row)[:, None])
    out = orc.combine(L, "expert", y, w)
    np.testing.assert_array_equal(bf16_to_float(out), np.array(g["combine_expert_scaled"], np.float32))
    # per-group scaled expert
    D = orc.dispatch_bf16(L, "group", x, w, idx)
    g_of_row = np.searchsorted(L["group_offset"], np.arange(L["R_group"]), side="right") - 1
    y = bf16_bits_of(bf16_to_float(D["recv_x"]) * (1 + g_of_row)[:, None])
    out = orc.combine(L, "group", y, w)
    np.testing.assert_array_equal(bf16_to_float(out), np.array(g["combine_group_scaled"], np.float32))
    assert epg == 2


def test_golden_fp8_block_by_hand(orc, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "fp8_block_hand.json")))
    row = np.zeros(256, np.float32)
    codes_a = np.zeros(128, np.uint8)
    for i, (v, c) in enumerate(g["block_a"]):
        row[i] = v
        codes_a[i] = c
    codes_b = np.zeros(128, np.uint8)
    for i, (v, c) in enumerate(g["block_b"]):
        row[128 + i] = v
        codes_b[i] = c
    bits = bf16_bits_of(row)
    np.testing.assert_array_equal(bf16_to_float(bits), row)   # inputs are exact in bf16
    q, s = orc.quantize_row_fp8(bits)
    np.testing.assert_array_equal(q[:128], codes_a)
    np.testing.assert_array_equal(q[128:], codes_b)
    assert s[0] == np.float32(g["block_a_scale"])
    assert s[1] == np.float32(1.0) / np.float32(448.0)


# ------------------------------------------------------------------ layout: reductions to library routines

def _shapes():
    yield 1, 1, 1, 1
    yield 5, 2, 8, 8
    yield 37, 3, 12, 4
    yield 300, 8, 256, 8
    yield 513, 4, 64, 1
    yield 129, 6, 96, 32
    yield 64, 1, 7, 7


@pytest.mark.parametrize("T,K,E,G", list(_shapes()))
def test_layout_equals_stable_argsort(orc, T, K, E, G):
    idx = si.make_inputs(T, 8, E, K, seed=T * 131 + K)["topk_idx"]
    L = orc.layout(idx, E, G)
    assert L["status"] == 0
    flat = idx.ravel()
    # expert histogram by bincount, receive order by a stable sort of the flat pair list
    np.testing.assert_array_equal(L["expert_count"], np.bincount(flat, minlength=E))
    order = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(L["recv_src_e"], order)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(L["slot_e"], inv)
    # groups: the deduplicated (t, g) pairs, enumerated t-major, stably sorted by g
    epg = E // G
    pairs = sorted({(t, int(e) // epg) for t in range(T) for e in idx[t]})
    tg = np.array(pairs, np.int64).reshape(-1, 2)
    gorder = np.argsort(tg[:, 1], kind="stable")
    np.testing.assert_array_equal(L["recv_src_g"][:len(pairs)], tg[gorder, 0])
    np.testing.assert_array_equal(L["group_count"], np.bincount(tg[:, 1], minlength=G))
    slot_tg = np.full((T, G), -1, np.int64)
    slot_tg[tg[gorder, 0], tg[gorder, 1]] = np.arange(len(pairs))
    np.testing.assert_array_equal(L["slot_tg"], slot_tg.ravel())


def _brute_layout(idx, E, G):
    """Python brute force, written from the definition with sets and sorted()."""
    T, K = len(idx), (len(idx[0]) if len(idx) else 0)
    epg = E // G
    status = 0
    valid = {}
    for t in range(T):
        seen = set()
        for k in range(K):
            e = idx[t][k]
            if not (0 <= e < E):
                status |= 1
                valid[(t, k)] = False
            elif e in seen:
                status |= 2
                valid[(t, k)] = False
            else:
                seen.add(e)
                valid[(t, k)] = True
    keys = sorted((idx[t][k], t, k) for t in range(T) for k in range(K) if valid[(t, k)])
    slot_e = {(t, k): -1 for t in range(T) for k in range(K)}
    for r, (_, t, k) in enumerate(keys):
        slot_e[(t, k)] = r
    gkeys = sorted({(idx[t][k] // epg, t) for t in range(T) for k in range(K) if valid[(t, k)]})
    slot_tg = {(t, g): -1 for t in range(T) for g in range(G)}
    for r, (g, t) in enumerate(gkeys):
        slot_tg[(t, g)] = r
    slot_g = {(t, k): (slot_tg[(t, idx[t][k] // epg)] if valid[(t, k)] else -1)
              for t in range(T) for k in range(K)}
    return status, keys, gkeys, slot_e, slot_tg, slot_g


def test_layout_brute_force_with_invalid_entries(orc):
    rng = np.random.default_rng(7)
    for trial in range(300):
        T = int(rng.integers(0, 9))
        K = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 4]))
        E = G * int(rng.integers(1, 4))
        idx = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
        if trial % 3 == 0:
            idx = rng.integers(0, E, size=(T, K)).astype(np.int32)   # repeats, all in range
        L = orc.layout(idx, E, G)
        status, keys, gkeys, slot_e, slot_tg, slot_g = _brute_layout(idx.tolist(), E, G)
        assert L["status"] == status
        assert L["R_expert"] == len(keys) and L["R_group"] == len(gkeys)
        for (t, k), s in slot_e.items():
            assert L["slot_e"][t * K + k] == s
            assert L["slot_g"][t * K + k] == slot_g[(t, k)]
        for (t, g), s in slot_tg.items():
            assert L["slot_tg"][t * G + g] == s
        for r, (_, t, k) in enumerate(keys):
            assert L["recv_src_e"][r] == t * K + k
        for r, (_, t) in enumerate(gkeys):
            assert L["recv_src_g"][r] == t


@settings(max_examples=300, deadline=None)
@given(st.data())
def test_layout_brute_force_hypothesis(orc, data):
    """Hypothesis-generated tiny shapes and index arrays (out-of-range, negative and
    repeated entries included) against the Python brute force."""
    G = data.draw(st.sampled_from([1, 2, 4]))
    E = G * data.draw(st.integers(1, 3))
    K = data.draw(st.integers(1, 4))
    T = data.draw(st.integers(0, 7))
    flat = data.draw(st.lists(st.integers(-2, E + 1), min_size=T * K, max_size=T * K))
    idx = np.array(flat, np.int32).reshape(T, K)
    L = orc.layout(idx, E, G)
    status, keys, gkeys, slot_e, slot_tg, slot_g = _brute_layout(idx.tolist(), E, G)
    assert L["status"] == status
    assert L["R_expert"] == len(keys) and L["R_group"] == len(gkeys)
    for (t, k), s in slot_e.items():
        assert L["slot_e"][t * K + k] == s and L["slot_g"][t * K + k] == slot_g[(t, k)]
    for (t, g), s in slot_tg.items():
        assert L["slot_tg"][t * G + g] == s
    assert [int(v) for v in L["recv_src_e"][:len(keys)]] == [t * K + k for _, t, k in keys]
    assert [int(v) for v in L["recv_src_g"][:len(gkeys)]] == [t for _, t in gkeys]


@pytest.mark.parametrize("name", ["tiny", "t256", "t4096", "skew"])
def test_layout_invariants(orc, name):
    wl = si.WORKLOADS[name]
    idx = si.make_inputs(wl.T, 8, wl.E, wl.K, seed=wl.seed, routing=wl.routing,
                         zipf_s=wl.zipf_s)["topk_idx"]
    T, K, E, G = wl.T, wl.K, wl.E, wl.G
    L = orc.layout(idx, E, G)
    assert L["status"] == 0
    assert L["expert_count"].sum() == T * K
    P = L["group_count"].sum()
    assert P <= T * min(K, G) and P <= T * G and P >= T
    assert sorted(L["slot_e"].tolist()) == list(range(T * K))
    v = L["slot_tg"][L["slot_tg"] >= 0]
    assert sorted(v.tolist()) == list(range(P))
    for e in range(E):
        seg = L["recv_src_e"][L["expert_offset"][e]:L["expert_offset"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(idx.ravel()[seg] == e)
    for g in range(G):
        seg = L["recv_src_g"][L["group_offset"][g]:L["group_offset"][g + 1]]
        assert np.all(np.diff(seg) > 0)
    epg = E // G
    stg = L["slot_tg"].reshape(T, G)
    np.testing.assert_array_equal(L["slot_g"].reshape(T, K), stg[np.arange(T)[:, None], idx // epg])
    bits = np.array([[(m >> g) & 1 for g in range(G)] for m in L["tok_group_mask"]])
    np.testing.assert_array_equal(bits.astype(bool), stg >= 0)


def test_layout_special_cases(orc):
    # one expert per group: the deduplicated layout is the per-expert layout
    idx = si.make_inputs(64, 8, 16, 4, seed=11)["topk_idx"]
    L = orc.layout(idx, 16, 16)
    np.testing.assert_array_equal(L["slot_g"], L["slot_e"])
    np.testing.assert_array_equal(L["group_count"], L["expert_count"])
    np.testing.assert_array_equal(L["recv_src_g"], L["recv_src_e"] // 4)
    # one group: every token is one row, in token order
    L = orc.layout(idx, 16, 1)
    np.testing.assert_array_equal(L["recv_src_g"][:64], np.arange(64))
    np.testing.assert_array_equal(L["slot_g"], np.repeat(np.arange(64), 4))
    # top-1: a counting sort of the tokens by expert
    idx1 = si.make_inputs(100, 8, 10, 1, seed=12)["topk_idx"]
    L = orc.layout(idx1, 10, 5)
    np.testing.assert_array_equal(L["recv_src_e"], np.argsort(idx1[:, 0], kind="stable"))
    # no tokens
    L = orc.layout(np.zeros((0, 8), np.int32), 256, 8)
    assert L["expert_count"].sum() == 0 and L["group_offset"][-1] == 0 and L["status"] == 0


def test_generator_distinct_groups_closed_form():
    """E[distinct groups per token] = G (1 - C(E-epg, K) / C(E, K)) for a uniform K-subset."""
    E, G, K = 256, 8, 8
    epg = E // G
    expect = G * (1 - math.comb(E - epg, K) / math.comb(E, K))
    assert abs(expect - 5.2947) < 1e-4
    idx = si.make_inputs(4096, 8, E, K, seed=3)["topk_idx"]
    P = len({(t, int(e) // epg) for t in range(idx.shape[0]) for e in idx[t]})
    assert abs(P / 4096 - expect) < 0.05
    # every token's K experts are distinct and in range
    assert all(len(set(r)) == K for r in idx.tolist())


def test_generator_zipf_is_skewed():
    wl = si.WORKLOADS["skew"]
    idx = si.make_inputs(wl.T, 8, wl.E, wl.K, seed=wl.seed, routing="zipf")["topk_idx"]
    cnt = np.bincount(idx.ravel(), minlength=wl.E)
    assert cnt.max() > 3000 and cnt.min() < 200 and cnt.sum() == wl.T * wl.K
    assert all(len(set(r)) == wl.K for r in idx.tolist())


# ------------------------------------------------------------------ dispatch

@pytest.mark.parametrize("name", ["tiny", "t256"])
def test_dispatch_bf16_against_sender_view(orc, name):
    d = si.make_workload(name)
    wl = d["workload"]
    x, w, idx = d["x"], d["topk_w"], d["topk_idx"]
    L = orc.layout(idx, wl.E, wl.G)
    cap = wl.T * wl.K + 3
    canary = 0xBEEF
    D = orc.dispatch_bf16(L, "expert", x, w, idx, capacity=cap, fill=canary)
    # sender view: token t's k-th row sits at slot_e[t, k]
    se = L["slot_e"].reshape(wl.T, wl.K)
    for t in range(wl.T):
        for k in range(wl.K):
            np.testing.assert_array_equal(D["recv_x"][se[t, k]], x[t])
            np.testing.assert_array_equal(D["recv_w"][se[t, k]], w[t])
            np.testing.assert_array_equal(D["recv_idx"][se[t, k]], idx[t])
    assert np.all(D["recv_x"][wl.T * wl.K:] == canary)
    # library route: rows of x gathered by a stable sort of the flat expert list
    np.testing.assert_array_equal(D["recv_x"][:wl.T * wl.K],
                                  x[np.argsort(idx.ravel(), kind="stable") // wl.K])
    Dg = orc.dispatch_bf16(L, "group", x, w, idx)
    stg = L["slot_tg"].reshape(wl.T, wl.G)
    for t in range(wl.T):
        for g in range(wl.G):
            if stg[t, g] >= 0:
                np.testing.assert_array_equal(Dg["recv_x"][stg[t, g]], x[t])
                np.testing.assert_array_equal(Dg["recv_idx"][stg[t, g]], idx[t])


def test_dispatch_one_group_is_identity_copy(orc):
    d = si.make_inputs(50, 64, 16, 4, seed=5)
    L = orc.layout(d["topk_idx"], 16, 1)
    D = orc.dispatch_bf16(L, "group", d["x"], d["topk_w"], d["topk_idx"])
    np.testing.assert_array_equal(D["recv_x"], d["x"])
    np.testing.assert_array_equal(D["recv_w"], d["topk_w"])


# ------------------------------------------------------------------ codecs

def test_bf16_decode_exhaustive(orc):
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bf16_to_float(allbits)
    got = np.array([orc.bf16_to_f32(int(b)) for b in allbits], np.float32)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[~np.isfinite(ref) & np.isnan(ref)]))


def test_bf16_encode_against_torch(orc):
    rng = np.random.default_rng(0)
    a = rng.standard_normal(1 << 20).astype(np.float32) * np.float32(3.0)
    b = (rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    b = b[np.isfinite(b)]
    # exact ties: bf16 value plus half its ulp (low 16 bits = 0x8000), both parities
    hi = rng.integers(0, 0x7F7F, 1 << 16, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    for arr in (a, b, ties, -ties):
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(orc.f32_to_bf16_array(arr), ref)
    # the tie 1 + 2^-8 goes to 1.0, and 1 + 3*2^-8 goes to 1 + 2^-6... up to even
    assert orc.f32_to_bf16(1.0 + 2 ** -8) == 0x3F80
    assert orc.f32_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82


def test_bf16_encode_non_finite(orc):
    """Infinities stay infinities, values past the largest bf16 round to them, and every
    NaN (either sign, any payload: quiet, signalling, all ones) becomes a NaN: the
    canonical quiet NaN 0x7FC0 (torch's CPU cast also gives a NaN, with another payload)."""
    special = np.array([0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF,
                        0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF, 0xFFFFFFFF,
                        0x7FBFFFFF, 0xFFFF8000], np.uint32).view(np.float32)
    got = orc.f32_to_bf16_array(special)
    ref = torch.from_numpy(special).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got[:6], ref[:6])
    is_nan = lambda b: (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
    assert all(is_nan(int(b)) for b in ref[6:]) and all(is_nan(int(b)) for b in got[6:])
    assert list(got[:2]) == [0x7F80, 0xFF80]
    assert list(got[4:6]) == [0x7F80, 0x7F7F]            # the tie above the max rounds to inf
    assert np.all(got[6:] == 0x7FC0)


def test_e4m3_decode_all_codes(orc):
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        got = orc.e4m3_to_f32(c)
        if e == 15 and m == 7:
            assert math.isnan(got)
            continue
        v = (2.0 ** (e - 7)) * (1 + m / 8) if e else (2.0 ** -6) * (m / 8)
        v = -v if s else v
        assert got == v and math.copysign(1, got) == (-1 if s else 1), c
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([orc.e4m3_to_f32(c) for c in range(256)], np.float32)
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    assert np.isnan(got[~fin]).all()


def test_e4m3_encode_against_torch_and_midpoints(orc):
    rng = np.random.default_rng(1)
    sweeps = [
        np.linspace(-464, 464, 400001, dtype=np.float32),
        (rng.standard_normal(1 << 20) * 60).astype(np.float32),
        (rng.standard_normal(1 << 18) * 2e-3).astype(np.float32),   # subnormal region
        np.float32(2.0) ** rng.uniform(-12, 8.8, 1 << 18).astype(np.float32),
    ]
    # every midpoint between neighbouring finite codes, both signs
    vals = np.array([orc.e4m3_to_f32(c) for c in range(127)], np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)  # exact in fp32
    sweeps += [mids, -mids]
    for arr in sweeps:
        arr = arr[np.abs(arr) <= 464]
        ref = torch.from_numpy(arr).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(orc.f32_to_e4m3_array(arr), ref)
    # midpoints go to the even code
    enc = orc.f32_to_e4m3_array(mids)
    assert np.all(enc % 2 == 0)
    # saturation above the last midpoint (torch gives NaN there; the reading is satfinite)
    assert orc.f32_to_e4m3(1e6) == 0x7E and orc.f32_to_e4m3(-500.0) == 0xFE
    assert orc.f32_to_e4m3(-0.0) == 0x80 and orc.f32_to_e4m3(0.0) == 0
    # infinities saturate like any value past 448; a NaN of either sign is the NaN
    # code 0x7F (torch's cast gives the same code for a positive NaN)
    assert orc.f32_to_e4m3(math.inf) == 0x7E and orc.f32_to_e4m3(-math.inf) == 0xFE
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], np.uint32).view(np.float32)
    assert list(orc.f32_to_e4m3_array(nans)) == [0x7F] * 4
    assert torch.tensor([math.nan]).to(torch.float8_e4m3fn).view(torch.uint8).item() == 0x7F


def test_fp8_quantisation_bounds(orc):
    d = si.make_inputs(64, 1024, 8, 2, seed=21)
    x = d["x"]
    xf = bf16_to_float(x)
    for t in range(x.shape[0]):
        q, s = orc.quantize_row_fp8(x[t])
        for b in range(x.shape[1] // 128):
            blk = xf[t, b * 128:(b + 1) * 128].astype(np.float64)
            amax = np.abs(blk).max()
            assert s[b] == np.float32(amax) / np.float32(448)
            dq = np.array([orc.e4m3_to_f32(int(c)) for c in q[b * 128:(b + 1) * 128]])
            # the largest element lands on +-448 exactly
            j = int(np.abs(blk).argmax())
            assert abs(dq[j]) == 448.0 and np.sign(dq[j]) == np.sign(blk[j])
            rec = dq * float(s[b])
            err = np.abs(rec - blk)
            normal = np.abs(dq) >= 2 ** -6
            assert np.all(err[normal] <= 2 ** -4 * np.abs(blk[normal]) * (1 + 1e-6) + 1e-30)
            assert np.all(err[~normal] <= 2 ** -10 * float(s[b]) * (1 + 1e-6))


def test_fp8_blocks_with_non_finite_values(orc):
    """A NaN (quiet, signalling, either sign) is skipped by the block amax, so the
    block's scale and every other code are those of the block with the NaNs set to
    zero (numpy's nanmax gives the same amax) and the NaNs encode as 0x7F; an
    infinity makes amax infinite, so scale = inf, inv = 448 / inf = 0 and every
    finite value encodes as a zero of its sign while inf * 0 is the NaN code; a
    block of NaNs only has amax 0, scale 0 and NaN codes."""
    rng = np.random.default_rng(5)
    base = bf16_bits_of((rng.standard_normal(512) * 3).astype(np.float32))
    xf = bf16_to_float(base)
    for payload in (0x7FC0, 0x7F81, 0xFFC0, 0xFFFF):
        row = base.copy()
        blk = 1
        seg = np.abs(xf[128:256])
        pos = 128 + rng.choice([j for j in range(128) if j != int(seg.argmax())], 9, replace=False)
        row[pos] = payload
        zeroed = row.copy()
        zeroed[pos] = 0
        q, sc = orc.quantize_row_fp8(row)
        qz, sz = orc.quantize_row_fp8(zeroed)
        np.testing.assert_array_equal(sc.view(np.uint32), sz.view(np.uint32))
        amax = np.nanmax(np.abs(bf16_to_float(row)[128 * blk:128 * (blk + 1)]))
        assert sc[blk] == np.float32(amax) / np.float32(448)
        keep = np.ones(512, bool)
        keep[pos] = False
        np.testing.assert_array_equal(q[keep], qz[keep])
        assert np.all(q[pos] == 0x7F)
    for inf in (0x7F80, 0xFF80):
        row = base.copy()
        row[300] = inf
        q, sc = orc.quantize_row_fp8(row)
        q0, s0 = orc.quantize_row_fp8(base)
        assert math.isinf(sc[2]) and sc[2] > 0
        blk = slice(256, 384)
        expect = np.where(np.signbit(xf[blk]), 0x80, 0x00).astype(np.uint8)
        expect[300 - 256] = 0x7F
        np.testing.assert_array_equal(q[blk], expect)
        other = np.r_[0:256, 384:512]
        np.testing.assert_array_equal(q[other], q0[other])
        np.testing.assert_array_equal(np.delete(sc, 2), np.delete(s0, 2))
    row = base.copy()
    row[0:128] = 0x7F81
    q, sc = orc.quantize_row_fp8(row)
    assert sc[0] == 0.0 and np.all(q[:128] == 0x7F)


def test_cast_transpose_non_finite_values(orc):
    """Cast-transpose: NaNs are skipped by the expert amax (numpy's nanmax of |x|),
    an infinity makes it infinite; a NaN encodes as 0x7F, an infinity times a finite
    scale saturates to +-448 (0x7E / 0xFE), and the transpose carries the same codes."""
    off = np.array([0, 4, 7], np.int32)
    rng = np.random.default_rng(8)
    xv = (rng.standard_normal((7, 32)) * 4).astype(np.float32)
    x = bf16_bits_of(xv)
    x[1, 3], x[2, 30], x[0, 0] = 0x7F81, 0xFFC0, 0x7FC0          # NaNs in expert 0
    x[5, 7], x[6, 9] = 0xFF80, 0x7FFF                             # -inf and a NaN in expert 1
    scale = np.array([2.0, 0.5], np.float32)
    out = orc.cast_transpose_fp8(off, x, scale)
    xf = bf16_to_float(x)
    assert out["amax"][0] == np.nanmax(np.abs(xf[0:4]))
    assert math.isinf(out["amax"][1])
    c = out["c"]
    assert c[1, 3] == c[2, 30] == c[0, 0] == c[6, 9] == 0x7F
    assert c[5, 7] == 0xFE
    fin = ~np.isnan(xf) & ~np.isinf(xf)
    with np.errstate(invalid="ignore"):
        prod = xf * np.repeat(scale, [4, 3])[:, None]
    ref = np.array([orc.f32_to_e4m3(float(v)) for v in prod.ravel()], np.uint8).reshape(7, 32)
    np.testing.assert_array_equal(c[:7][fin], ref[fin])
    t1 = out["t"][32 * 16:32 * 32].reshape(32, 16)
    np.testing.assert_array_equal(t1[:, :3], c[4:7].T)


def test_dequant_identity_on_exact_codes(orc):
    # a row whose block amax is 448 has scale 1, so decode(q) * 1 recovers every
    # input that is itself an e4m3 value
    codes = np.arange(0, 126, dtype=np.uint8)
    vals = np.array([orc.e4m3_to_f32(int(c)) for c in codes], np.float32)
    row = np.zeros(128, np.float32)
    row[:126] = vals
    row[126] = 448.0
    row[127] = -448.0
    bits = bf16_bits_of(row)
    q, s = orc.quantize_row_fp8(bits)
    assert s[0] == 1.0
    y = orc.dequant_fp8(q[None, :], s[None, :])
    np.testing.assert_array_equal(y[0], bits)


def e4m3_closed_form(codes):
    """float64 value of each e4m3fn code, written from the format's definition (not
    through the oracle): (-1)^s * 2^(e-7) * (1 + m/8), subnormals (e = 0)
    2^-6 * m/8, and S.1111.111 a NaN."""
    c = np.asarray(codes, np.int64)
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    v = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    v = np.where(s == 1, -v, v)
    return np.where((e == 15) & (m == 7), np.nan, v)


def test_dequant_multi_block_closed_form(orc):
    """Several rows of several 128-blocks, every block with its own scale (none of
    them 1, most not powers of two): each element is the closed-form value of its
    code times the scale of ITS row and block, one fp32 multiply, rounded to bf16
    by torch's CPU cast. A dequant that divided by the scale, or took the scale of
    another block or row, fails here."""
    rng = np.random.default_rng(44)
    R, nb = 5, 6
    H = nb * 128
    codes = rng.integers(0, 256, (R, H)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                      # NaN codes: below
    scale = (rng.uniform(0.5, 2.0, (R, nb)) * 2.0 ** rng.integers(-14, 8, (R, nb))).astype(np.float32)
    scale[0, :4] = [np.float32(1) / np.float32(448), 3.0, 0.1, 2.0 ** -7]
    assert len(np.unique(scale)) == R * nb and not np.any(scale == 1.0)
    y = orc.dequant_fp8(codes, scale)
    prod = e4m3_closed_form(codes).astype(np.float32) * np.repeat(scale, 128, axis=1)
    assert prod.dtype == np.float32                             # one fp32 rounding
    np.testing.assert_array_equal(y, bf16_bits_of(prod))
    # rows past R are not written; a NaN code comes back a NaN
    y3 = orc.dequant_fp8(codes, scale, R=3)
    np.testing.assert_array_equal(y3[:3], y[:3])
    assert np.all(y3[3:] == 0)
    q = codes[:1].copy()
    q[0, 5], q[0, 300] = 0x7F, 0xFF
    yn = bf16_to_float(orc.dequant_fp8(q, scale[:1]))
    assert np.isnan(yn[0, 5]) and np.isnan(yn[0, 300]) and np.isfinite(np.delete(yn[0], [5, 300])).all()


def test_fp8_round_trip_error_bound_on_fp8_workload(orc):
    """Rows of the FP8 workload's input through quantize_row_fp8 and then the
    oracle's dequant: for every element, with d = decode(q),
      |y - x| <= 2^-4 |x| + 2^-8 |y|           where |d| >= 2^-6 (normal e4m3)
      |y - x| <= 2^-10 scale + 2^-8 |y|        where |d| <  2^-6 (subnormal e4m3)
    (half an e4m3 ulp of x * inv, scaled back; then half a bf16 ulp of the dequant's
    rounding; the 1 + 2^-23 from inv * scale is covered by a 1e-6 slack). The element
    of largest |x| in each block comes back bit for bit: it encodes to +-448, and
    448 * scale rounds back to amax in bf16."""
    d = si.make_workload("fp8")
    rows = d["x"][::16][:256]                                   # 256 of the 4096 rows
    H = rows.shape[1]
    q = np.zeros_like(rows, dtype=np.uint8)
    sc = np.zeros((rows.shape[0], H // 128), np.float32)
    for r in range(rows.shape[0]):
        q[r], sc[r] = orc.quantize_row_fp8(rows[r])
    y = bf16_to_float(orc.dequant_fp8(q, sc)).astype(np.float64)
    x = bf16_to_float(rows).astype(np.float64)
    dq = e4m3_closed_form(q)
    s = np.repeat(sc.astype(np.float64), 128, axis=1)
    err = np.abs(y - x)
    normal = np.abs(dq) >= 2.0 ** -6
    bound = np.where(normal, 2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) * (1 + 1e-6) + 2.0 ** -8 * np.abs(y)
    assert np.all(err <= bound)
    xb = np.abs(x).reshape(x.shape[0], -1, 128)
    j = xb.argmax(axis=2)
    yb, xs = y.reshape(xb.shape), x.reshape(xb.shape)
    np.testing.assert_array_equal(np.take_along_axis(yb, j[..., None], 2), np.take_along_axis(xs, j[..., None], 2))


def _expected_sources(idx, E, G):
    """Source token of every receive row, from library routines alone: per-expert
    rows in the order of a stable argsort of the flat pair list; per-group rows from
    the deduplicated (token, group) pairs, enumerated token-major, stably sorted by
    group."""
    T, K = idx.shape
    src_e = np.argsort(idx.ravel(), kind="stable") // K
    epg = E // G
    tg = np.array(sorted({(t, int(e) // epg) for t in range(T) for e in idx[t]}), np.int64).reshape(-1, 2)
    src_g = tg[np.argsort(tg[:, 1], kind="stable"), 0]
    return {"expert": src_e, "group": src_g}


@pytest.mark.parametrize("T,H,E,G,K", [(60, 512, 32, 4, 4), (33, 384, 12, 12, 3), (40, 256, 16, 1, 5)])
def test_dispatch_fp8_rows_are_their_sources_quantised(orc, T, H, E, G, K):
    """Every receive row of the FP8 dispatch, in both layouts, holds exactly the codes
    and the H/128 scales that quantize_row_fp8 gives for its source token's row, and
    the token's K weights and indices; the source of each row is found without the
    oracle's layout."""
    d = si.make_inputs(T, H, E, K, seed=T + H + K)
    x = d["x"].copy()
    x[3, 128:256] = 0                                            # an all-zero block: scale 0
    L = orc.layout(d["topk_idx"], E, G)
    src = _expected_sources(d["topk_idx"], E, G)
    per_tok = [orc.quantize_row_fp8(x[t]) for t in range(T)]
    for mode in ("expert", "group"):
        D = orc.dispatch_fp8(L, mode, x, d["topk_w"], d["topk_idx"])
        assert D["R"] == len(src[mode])
        for r, t in enumerate(src[mode]):
            np.testing.assert_array_equal(D["recv_q"][r], per_tok[t][0], err_msg=f"{mode} row {r}")
            np.testing.assert_array_equal(D["recv_scale"][r].view(np.uint32), per_tok[t][1].view(np.uint32))
            np.testing.assert_array_equal(D["recv_w"][r], d["topk_w"][t])
            np.testing.assert_array_equal(D["recv_idx"][r], d["topk_idx"][t])


def test_dispatch_fp8_hand_worked_row_lands_in_its_rows(orc, golden_dir):
    """The hand-worked two-block row (tests/golden/fp8_block_hand.json) as token 1 of
    three tokens, top-2 over E = 4 experts in G = 2 groups:
        token 0 -> experts 0, 2;  token 1 -> experts 3, 1;  token 2 -> experts 2, 0.
    Per expert the rows are expert 0: tokens 0, 2; expert 1: token 1; expert 2:
    tokens 0, 2; expert 3: token 1, so token 1 owns per-expert rows 2 and 5. Every
    token reaches both groups (experts 0, 1 are group 0; 2, 3 group 1), so the
    per-group rows are tokens 0, 1, 2 in group 0 and again in group 1: token 1 owns
    rows 1 and 4. Those rows carry the hand-worked codes, scale 1 for block A and
    fp32(1/448) for block B, in that order."""
    g = json.load(open(os.path.join(golden_dir, "fp8_block_hand.json")))
    H = 256
    row = np.zeros(H, np.float32)
    codes = np.zeros(H, np.uint8)
    for i, (v, c) in enumerate(g["block_a"]):
        row[i], codes[i] = v, c
    for i, (v, c) in enumerate(g["block_b"]):
        row[128 + i], codes[128 + i] = v, c
    rng = np.random.default_rng(9)
    x = bf16_bits_of(np.stack([rng.standard_normal(H).astype(np.float32), row,
                               rng.standard_normal(H).astype(np.float32)]))
    idx = np.array([[0, 2], [3, 1], [2, 0]], np.int32)
    w = np.array([[0.25, 0.75], [0.5, 0.5], [0.125, 0.875]], np.float32)
    L = orc.layout(idx, 4, 2)
    scales = np.array([g["block_a_scale"], np.float32(1) / np.float32(448)], np.float32)
    for mode, rows in (("expert", (2, 5)), ("group", (1, 4))):
        D = orc.dispatch_fp8(L, mode, x, w, idx)
        assert D["R"] == 6
        for r in rows:
            np.testing.assert_array_equal(D["recv_q"][r], codes, err_msg=f"{mode} row {r}")
            np.testing.assert_array_equal(D["recv_scale"][r], scales)
            np.testing.assert_array_equal(D["recv_w"][r], w[1])
            np.testing.assert_array_equal(D["recv_idx"][r], idx[1])
        others = [r for r in range(6) if r not in rows]
        assert not any(np.array_equal(D["recv_q"][r], codes) for r in others)


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("name", ["tiny", "t256"])
@pytest.mark.parametrize("mode", ["expert", "group"])
def test_combine_identity_round_trip(orc, name, mode):
    """Weights summing to 1 (to fp32 rounding) with identity experts give x back bit-exactly."""
    d = si.make_workload(name)
    wl = d["workload"]
    L = orc.layout(d["topk_idx"], wl.E, wl.G)
    D = orc.dispatch_bf16(L, mode, d["x"], d["topk_w"], d["topk_idx"])
    out = orc.combine(L, mode, D["recv_x"], d["topk_w"])
    np.testing.assert_array_equal(out, d["x"])


def test_combine_scaled_expert_closed_form(orc):
    """Expert e multiplies its rows by c_e = 1 + e/E; the result must be within
    1 bf16 ulp of sum_k w_k c_{e_k} x_t computed in float64."""
    T, H, E, G, K = 96, 256, 32, 4, 6
    d = si.make_inputs(T, H, E, K, seed=31)
    L = orc.layout(d["topk_idx"], E, G)
    D = orc.dispatch_bf16(L, "expert", d["x"], d["topk_w"], d["topk_idx"])
    e_of_row = np.searchsorted(L["expert_offset"], np.arange(L["R_expert"]), side="right") - 1
    c = (1.0 + np.arange(E) / E).astype(np.float32)
    y = bf16_bits_of(bf16_to_float(D["recv_x"]) * c[e_of_row][:, None])
    out = bf16_to_float(orc.combine(L, "expert", y, d["topk_w"])).astype(np.float64)
    yf = bf16_to_float(y).astype(np.float64)
    se = L["slot_e"].reshape(T, K)
    ref = np.zeros((T, H))
    for k in range(K):
        ref += d["topk_w"][:, k:k + 1].astype(np.float64) * yf[se[:, k]]
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(out - ref) <= ulp)


def test_combine_exact_fma_chain_brute_force(orc):
    """Tiny inputs: the fp32 chain acc = fma(w_k, y_k, acc), k ascending from -0, then
    one round to bf16 — emulated with exact rationals — equals the oracle bit for bit."""
    rng = np.random.default_rng(5)
    mism = 0
    for trial in range(40):
        T, H = 3, 16
        E, G, K = 12, int(rng.choice([1, 3, 4, 12])), int(rng.integers(1, 6))
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        w = rng.standard_normal((T, K)).astype(np.float32)
        L = orc.layout(idx, E, G)
        for mode, R, slot in (("expert", L["R_expert"], L["slot_e"]),
                              ("group", L["R_group"], L["slot_g"])):
            y = bf16_bits_of(rng.standard_normal((R, H)).astype(np.float32) * 4)
            y[rng.random(y.shape) < 0.05] = 0x8000       # some signed zeros
            y[rng.random(y.shape) < 0.05] = 0x0000
            yf = bf16_to_float(y)
            out = orc.combine(L, mode, y, w)
            ref = np.zeros((T, H), np.float32)
            for t in range(T):
                for i in range(H):
                    acc = -0.0
                    for k in range(K):
                        acc = fma_f32(float(w[t, k]), float(yf[slot[t * K + k], i]), acc)
                    ref[t, i] = acc
            refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            mism += int((out != refb).sum())
    assert mism == 0


def test_combine_skips_invalid_entries(orc):
    idx = np.array([[0, 0, 9], [1, 2, 3]], np.int32)   # repeat and out-of-range in token 0
    w = np.array([[0.5, 0.25, 0.25], [0.5, 0.25, 0.25]], np.float32)
    L = orc.layout(idx, 4, 2)
    assert L["status"] == 3
    assert L["slot_e"][1] == -1 and L["slot_e"][2] == -1
    x = bf16_bits_of([[2.0, 4.0], [8.0, -8.0]])
    D = orc.dispatch_bf16(L, "expert", x, w, idx)
    out = bf16_to_float(orc.combine(L, "expert", D["recv_x"], w))
    np.testing.assert_array_equal(out, np.array([[1.0, 2.0], [8.0, -8.0]], np.float32))


# ------------------------------------------------------------------ regroup (per-group rows -> per-expert rows)

@pytest.mark.parametrize("name", ["tiny", "t256"])
def test_regroup_of_group_dispatch_is_expert_dispatch(orc, name):
    """Composition identity: dispatching per group and regrouping gives, array by
    array, exactly the per-expert dispatch (bf16 and FP8)."""
    d = si.make_workload(name)
    wl = d["workload"]
    L = orc.layout(d["topk_idx"], wl.E, wl.G)
    Dg = orc.dispatch_bf16(L, "group", d["x"], d["topk_w"], d["topk_idx"])
    De = orc.dispatch_bf16(L, "expert", d["x"], d["topk_w"], d["topk_idx"])
    Rg = orc.regroup(L, Dg)
    for n in ("recv_x", "recv_w", "recv_idx"):
        np.testing.assert_array_equal(Rg[n], De[n][:L["R_expert"]], err_msg=n)
    Dg8 = orc.dispatch_fp8(L, "group", d["x"], d["topk_w"], d["topk_idx"])
    De8 = orc.dispatch_fp8(L, "expert", d["x"], d["topk_w"], d["topk_idx"])
    Rg8 = orc.regroup(L, Dg8)
    for n in ("recv_q", "recv_scale", "recv_w", "recv_idx"):
        np.testing.assert_array_equal(Rg8[n], De8[n][:L["R_expert"]], err_msg=n)


def test_regroup_rows_is_a_gather(orc):
    """Arbitrary per-group rows: the result is numpy's gather of the rows named by
    slot_g of each per-expert row's pair; with one group per expert it is the identity."""
    rng = np.random.default_rng(3)
    d = si.make_inputs(200, 8, 32, 5, seed=8)
    L = orc.layout(d["topk_idx"], 32, 4)
    rows = rng.integers(0, 1 << 16, size=(L["R_group"], 24), dtype=np.uint16)
    got = orc.regroup_rows(L, rows)
    np.testing.assert_array_equal(got, rows[L["slot_g"][L["recv_src_e"][:L["R_expert"]]]])
    L1 = orc.layout(d["topk_idx"], 32, 32)
    rows1 = rng.integers(0, 1 << 16, size=(L1["R_group"], 8), dtype=np.uint16)
    np.testing.assert_array_equal(orc.regroup_rows(L1, rows1), rows1)


# ------------------------------------------------------------------ per-expert FP8 cast + transpose

def test_cast_transpose_against_library_routes(orc):
    """C is torch's e4m3fn cast of x*scale (where it does not saturate), each T_e is
    numpy's transpose of the expert's C rows followed by zero padding to 16 columns,
    and amax is numpy's max |x| per expert."""
    rng = np.random.default_rng(11)
    T, H, E, G, K = 150, 256, 12, 4, 3
    d = si.make_inputs(T, H, E, K, seed=12)
    L = orc.layout(d["topk_idx"], E, G)
    De = orc.dispatch_bf16(L, "expert", d["x"], d["topk_w"], d["topk_idx"])
    scale = rng.uniform(0.5, 40.0, E).astype(np.float32)
    out = orc.cast_transpose_fp8(L["expert_offset"], De["recv_x"], scale)
    xf = bf16_to_float(De["recv_x"])
    off = L["expert_offset"]
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        n = off[e + 1] - off[e]
        prod = (xf[rows] * scale[e]).astype(np.float32)
        ok = np.abs(prod) <= 448
        ref = torch.from_numpy(np.clip(prod, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(out["c"][rows][ok], ref[ok])
        assert np.all(out["c"][rows][~ok] & 0x7F == 0x7E)          # saturated to +-448
        npad = (n + 15) // 16 * 16
        assert out["pad_offset"][e + 1] - out["pad_offset"][e] == npad
        te = out["t"][H * out["pad_offset"][e]:H * out["pad_offset"][e + 1]].reshape(H, npad)
        np.testing.assert_array_equal(te[:, :n], out["c"][rows].T)
        assert np.all(te[:, n:] == 0)
        assert out["amax"][e] == (np.abs(xf[rows]).max() if n else 0.0)


def test_cast_transpose_amax_accumulates_and_scale_one_is_exact(orc):
    off = np.array([0, 3, 3, 5], np.int32)                    # an expert with no rows
    vals = np.array([1.0, -0.5, 448.0, 2.0 ** -9, 0.0, 96.0, -240.0, 1.125], np.float32)
    x = bf16_bits_of(np.resize(vals, (5, 16)))
    out = orc.cast_transpose_fp8(off, x, np.ones(3, np.float32), amax_in=np.array([1000, 7, 0], np.float32))
    codes = np.array([orc.f32_to_e4m3(float(v)) for v in np.resize(vals, (5, 16)).ravel()], np.uint8)
    np.testing.assert_array_equal(out["c"].ravel(), codes)
    np.testing.assert_array_equal(out["amax"], np.array([1000, 7, 448], np.float32))
    assert list(out["pad_offset"]) == [0, 16, 16, 32]
