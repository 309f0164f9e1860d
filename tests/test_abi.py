"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call (so these
run without a GPU). No compute is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def moe():
    import __graft_entry__
    b = __graft_entry__._hip_build_module()
    if b.is_stale():
        b.build()
    import combine_moe_layout_amd as m
    return m


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_three_calls():
    names = header_functions()
    for n in ("moe_layout", "moe_dispatch", "moe_combine", "moe_layout_workspace_bytes",
              "moe_recv_rows_bound", "moe_status_string"):
        assert n in names
    assert len(names) >= 9


def test_library_exports_every_declared_symbol(moe):
    lib = ctypes.CDLL(moe.library_path())
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert moe._lib.moe_abi_version() == 3


def test_query_functions(moe):
    assert moe.recv_rows_bound(4096, 8, 8, "expert") == 32768
    assert moe.recv_rows_bound(4096, 8, 8, "group") == 32768
    assert moe.recv_rows_bound(16, 2, 8, "group") == 32
    assert moe.recv_rows_bound(100, 8, 4, "group") == 400
    assert moe.recv_rows_bound(0, 8, 4, "expert") == 0
    assert moe.layout_workspace_bytes(4096, 8, 256, 8) >= 4 * (256 + 8 + 1) * 16
    assert moe.layout_workspace_bytes(0, 8, 256, 8) == 0
    with pytest.raises(moe.MoeError):
        moe.layout_workspace_bytes(16, 8, 255, 8)       # E % G != 0
    with pytest.raises(moe.MoeError):
        moe.layout_workspace_bytes(16, 33, 256, 8)      # K > 32
    with pytest.raises(moe.MoeError):
        moe.layout_workspace_bytes(16, 8, 2048, 8)      # E > 1024
    with pytest.raises(moe.MoeError):
        moe.layout_workspace_bytes(16, 8, 256, 64)      # G > 32
    with pytest.raises(moe.MoeError):
        moe.layout_workspace_bytes(1 << 27, 8, 256, 8)  # T * K >= 2^30
    with pytest.raises(moe.MoeError):
        moe.recv_rows_bound(16, 2, 8, 5)


def _fake_layout(moe, T=16, K=2, E=8, G=8, null=None):
    """A moe_layout_t whose pointers are fake but aligned non-NULL addresses: the
    calls below must return before dereferencing or launching anything."""
    addr = 1 << 20
    vals = {}
    for n in ("expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask",
              "slot_e", "slot_g", "slot_tg", "recv_src_e", "recv_src_g", "status"):
        vals[n] = None if n == null else addr
        addr += 1 << 16
    return moe._LayoutT(T, K, E, G, *vals.values())


def test_host_validation_errors(moe):
    lib = moe._lib
    P = ctypes.c_void_p
    A = P(1 << 24)          # aligned fake device address (never dereferenced)
    M = P((1 << 24) + 2)    # misaligned
    NULL = None
    L = _fake_layout(moe)
    ref = ctypes.byref
    # layout
    assert lib.moe_layout(A, ref(_fake_layout(moe, null="slot_e")), A, 1 << 20, NULL) == -1
    assert lib.moe_layout(A, ref(_fake_layout(moe, E=9)), A, 1 << 20, NULL) == -2
    assert lib.moe_layout(A, ref(_fake_layout(moe, K=0)), A, 1 << 20, NULL) == -2
    assert lib.moe_layout(A, ref(_fake_layout(moe, T=-1)), A, 1 << 20, NULL) == -2
    assert lib.moe_layout(A, ref(L), A, 0, NULL) == -5
    assert lib.moe_layout(A, ref(L), NULL, 1 << 20, NULL) == -5
    assert lib.moe_layout(NULL, ref(L), A, 1 << 20, NULL) == -1
    assert lib.moe_layout(M, ref(L), A, 1 << 20, NULL) == -3
    # dispatch: mode, dtype, H, capacity, alignment, null
    d = lambda mode=0, dt=0, H=2048, x=A, rx=A, sc=NULL, cap=32, Lp=L: lib.moe_dispatch(
        ref(Lp), mode, dt, H, x, A, A, rx, sc, A, A, cap, NULL)
    assert d() != -7
    assert d(mode=2) == -7
    assert d(dt=3) == -7
    assert d(H=2047) == -2
    assert d(H=0) == -2
    assert d(dt=1, H=1000, sc=A) == -2        # FP8 needs H % 128 == 0
    assert d(dt=1, H=1024, sc=NULL) == -1      # FP8 needs scales
    assert d(cap=31) == -4                      # EXPERT bound is T*K = 32
    assert d(mode=1, cap=31) == -4              # GROUP bound is T*min(K,G) = 32
    assert d(x=M) == -3 and d(rx=M) == -3
    assert d(x=NULL) == -1
    assert d(Lp=_fake_layout(moe, T=0), x=NULL) == 0
    # fused layout + dispatch: a workspace beyond the one-launch sizes
    f = lambda T=16, K=2, H=2048, cap=32, ws=NULL, nb=0: lib.moe_layout_dispatch(
        A, ref(_fake_layout(moe, T=T, K=K, E=64, G=8)), ws, nb, 0, 0, H, A, A, A, NULL, A, A, cap, NULL)
    assert f(T=513, cap=513 * 2) == -5          # no workspace
    need = moe.layout_workspace_bytes(513, 2, 64, 8)
    assert f(T=513, cap=513 * 2, ws=A, nb=need - 4) == -5
    assert f(T=513, cap=513 * 2, ws=M, nb=need) == -3
    assert f(T=512, K=33) == -2                 # K > 32
    assert f(T=16, H=12) == -2
    assert f(T=16, cap=31) == -4
    # regroup
    rg = lambda dt=0, H=2048, gcap=32, ecap=32, sc=NULL: lib.moe_regroup(
        ref(L), dt, H, A, sc, A, A, gcap, A, sc, A, A, ecap, NULL)
    assert rg(dt=2) == -7
    assert rg(H=12) == -2
    assert rg(dt=1, H=1000, sc=A) == -2
    assert rg(dt=1, H=1024, sc=NULL) == -1
    assert rg(gcap=31) == -4 and rg(ecap=31) == -4
    # combine
    c = lambda mode=0, H=2048, y=A, rows=32, out=A, Lp=L: lib.moe_combine(
        ref(Lp), mode, H, y, rows, A, out, NULL)
    assert c(mode=3) == -7
    assert c(H=12) == -2
    assert c(rows=-1) == -2
    assert c(y=M) == -3 and c(out=M) == -3
    assert c(y=NULL) == -1
    assert c(Lp=_fake_layout(moe, null="status")) == -1
    assert c(Lp=_fake_layout(moe, T=0), y=NULL) == 0
    # dequant and copy
    assert lib.moe_fp8_dequant(ref(L), 0, 1000, A, A, A, 32, NULL) == -2
    assert lib.moe_fp8_dequant(ref(L), 0, 1024, M, A, A, 32, NULL) == -3
    assert lib.moe_ref_copy(A, A, 15, NULL) == -2
    assert lib.moe_ref_copy(A, M, 16, NULL) == -3
    assert lib.moe_ref_copy(A, A, 0, NULL) == 0
    mix = lambda rb=14336, u=8, nr=8, nw=1, d=A: lib.moe_ref_mix(d, A, rb, u, nr, nw, NULL)
    assert mix(nr=3) == -7 and mix(nr=2, nw=2) == -7 and mix(nw=16) == -7
    assert mix(rb=15) == -2 and mix(u=-1) == -2
    assert mix(d=M) == -3 and mix(d=NULL) == -1
    assert mix(u=0, d=NULL) == 0
    # the no-allocation call: a workspace beyond its fixed array is refused before any HIP call
    nd = lambda Lp, mode=0, cap=1 << 20: lib.moe_layout_dispatch_noalloc(A, ref(Lp), mode, 0, 2048, A, A, A, NULL,
                                                                          A, A, cap, NULL)
    big = _fake_layout(moe, T=60000, K=8, E=1024, G=32)
    assert nd(big, cap=60000 * 8) == -8
    assert nd(big, mode=3) == -7 and nd(big, cap=10) == -4
    for code in range(-8, 1):
        assert lib.moe_status_string(code)


def test_package_has_no_cpu_fallback():
    """The binding must not route through the oracle or any CPU path."""
    pkg = os.path.join(ROOT, "combine_moe_layout_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn


def test_binding_constants_match_the_header(moe):
    """The Python binding's status bits, modes, dtypes and one-launch limits are the
    values include/moe_ep.h defines (the binding restates them; this keeps them equal)."""
    text = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    defs = dict(re.findall(r"#define\s+(MOE_[A-Z0-9_]+)\s+(\d+)", text))
    enums = dict(re.findall(r"(MOE_(?:MODE|DTYPE)_[A-Z0-9_]+)\s*=\s*(\d+)", text))
    assert int(defs["MOE_STATUS_BAD_INDEX"]) == moe.STATUS_BAD_INDEX
    assert int(defs["MOE_STATUS_DUPLICATE"]) == moe.STATUS_DUPLICATE
    assert int(defs["MOE_STATUS_Y_ROWS"]) == moe.STATUS_Y_ROWS
    assert int(defs["MOE_STATUS_SYNC_FALLBACK"]) == moe.STATUS_SYNC_FALLBACK
    assert int(defs["MOE_FUSED_MAX_TOKENS"]) == moe.FUSED_MAX_TOKENS
    assert int(defs["MOE_FUSED_MAX_PAIRS"]) == moe.FUSED_MAX_PAIRS
    assert int(defs["MOE_NOALLOC_SCRATCH_BYTES"]) == moe.NOALLOC_SCRATCH_BYTES
    assert moe.STATUS_ERRORS == moe.STATUS_BAD_INDEX | moe.STATUS_DUPLICATE | moe.STATUS_Y_ROWS
    assert int(enums["MOE_MODE_EXPERT"]) == moe.MODE_EXPERT and int(enums["MOE_MODE_GROUP"]) == moe.MODE_GROUP
    assert int(enums["MOE_DTYPE_BF16"]) == moe.DTYPE_BF16
    assert int(enums["MOE_DTYPE_FP8_E4M3_B128"]) == moe.DTYPE_FP8
    bits = [int(v) for k, v in defs.items() if k.startswith("MOE_STATUS_")]
    assert sorted(bits) == [1 << i for i in range(len(bits))]      # distinct single bits
