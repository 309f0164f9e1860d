"""CPU oracle for the MoE token path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It loads `liboracle.so`, built from `oracle.c` with gcc
(`-O2 -ffp-contract=off`, single thread), and wraps each function for numpy
arrays. It shares nothing with the HIP library and never imports it.

A second build of the same source, `liboracle_omp.so` (gcc -fopenmp), runs the
oracle's independent per-token and per-row loops on several threads; it exists
to time the oracle on every host core and gives the same bits as the canonical
build (tested). `with oracle.variant("openmp"): ...` routes the calls in the
block to it; `set_threads(n)` and `threads()` control and report its threads.

Every function follows the plain definition written out in `oracle.c`; see the
header of that file for the passages of the pages each one follows and for
the readings taken where the pages are silent.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-Wextra", "-Wno-unknown-pragmas"]
# variant -> (library file, extra gcc flags)
VARIANTS = {"serial": ("liboracle.so", ()), "openmp": ("liboracle_omp.so", ("-fopenmp",))}

STATUS_BAD_INDEX = 1
STATUS_DUPLICATE = 2


def _lib_path(v: str) -> str:
    return _LIB if v == "serial" else os.path.join(_HERE, VARIANTS[v][0])


def build(force: bool = True, extra_flags=(), variant: str | None = None) -> str:
    """Compile oracle.c (gcc, host only): the canonical single-thread liboracle.so and,
    with variant=None, also the OpenMP build; returns the path of the canonical one
    (or of the one variant asked for)."""
    for v in ([variant] if variant else list(VARIANTS)):
        path = _lib_path(v)
        if not force and os.path.exists(path) and os.path.getmtime(path) >= os.path.getmtime(_SRC):
            continue
        tmp = path + f".tmp{os.getpid()}"
        cmd = ["gcc", *GCC_FLAGS, *VARIANTS[v][1], *extra_flags, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    return _lib_path(variant or "serial")


_libs: dict = {}
_active = "serial"


@contextlib.contextmanager
def variant(name: str):
    """Route the oracle calls made inside the block to the build `name` ("serial",
    the canonical one, or "openmp")."""
    global _active
    if name not in VARIANTS:
        raise ValueError(name)
    old, _active = _active, name
    try:
        yield
    finally:
        _active = old


def threads() -> int:
    """Threads the active build's parallel loops use (1 for the canonical build)."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _load():
    v = _active
    if v not in _libs:
        build(force=False, variant=v)
        lib = ctypes.CDLL(_lib_path(v))
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.oracle_layout.argtypes = [i32, i32, i32, i32, P] + [P] * 10
        lib.oracle_layout.restype = i32
        lib.oracle_dispatch_bf16.argtypes = [i32, i32, i32, i64, P, P, P, P, P, P, P]
        lib.oracle_dispatch_bf16.restype = None
        lib.oracle_dispatch_fp8.argtypes = [i32, i32, i32, i32, i64, P, P, P, P, P, P, P, P]
        lib.oracle_dispatch_fp8.restype = None
        lib.oracle_quantize_row_fp8.argtypes = [i32, P, P, P]
        lib.oracle_quantize_row_fp8.restype = None
        lib.oracle_dequant_fp8.argtypes = [i64, i32, P, P, P]
        lib.oracle_dequant_fp8.restype = None
        lib.oracle_combine.argtypes = [i32, i32, i32, P, P, P, P]
        lib.oracle_combine.restype = None
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_f32.restype = ctypes.c_float
        lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
        lib.oracle_f32_to_bf16_n.argtypes = [i64, P, P]
        lib.oracle_f32_to_bf16_n.restype = None
        lib.oracle_f32_to_e4m3_n.argtypes = [i64, P, P]
        lib.oracle_f32_to_e4m3_n.restype = None
        lib.oracle_regroup_rows.argtypes = [i64, i64, P, P, P, P]
        lib.oracle_regroup_rows.restype = None
        lib.oracle_cast_transpose_fp8.argtypes = [i32, i32, P, P, P, P, P, P, P]
        lib.oracle_cast_transpose_fp8.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = i32
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_set_threads.restype = None
        _libs[v] = lib
    return _libs[v]


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def layout(topk_idx: np.ndarray, E: int, G: int) -> dict:
    """Routing layout of int32 [T, K] expert indices into E experts, G groups."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    if E % G or G > 32 or G < 1:
        raise ValueError("E must be a multiple of G and 1 <= G <= 32")
    out = {
        "expert_count": np.zeros(E, np.int32),
        "expert_offset": np.zeros(E + 1, np.int32),
        "group_count": np.zeros(G, np.int32),
        "group_offset": np.zeros(G + 1, np.int32),
        "tok_group_mask": np.zeros(T, np.uint32),
        "slot_e": np.zeros(T * K, np.int32),
        "slot_g": np.zeros(T * K, np.int32),
        "slot_tg": np.zeros(T * G, np.int32),
        "recv_src_e": np.full(T * K, -1, np.int32),
        "recv_src_g": np.full(T * min(K, G), -1, np.int32),
    }
    st = _load().oracle_layout(T, K, E, G, _p(idx), *(_p(out[n]) for n in (
        "expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask",
        "slot_e", "slot_g", "slot_tg", "recv_src_e", "recv_src_g")))
    out["status"] = int(st)
    out["T"], out["K"], out["E"], out["G"] = T, K, E, G
    out["R_expert"] = int(out["expert_offset"][E])
    out["R_group"] = int(out["group_offset"][G])
    return out


def _rows_and_src(L: dict, mode: str):
    if mode == "expert":
        return 0, L["R_expert"], L["recv_src_e"]
    if mode == "group":
        return 1, L["R_group"], L["recv_src_g"]
    raise ValueError(mode)


def _out_arrays(out, specs):
    """The output arrays of a call: those of `out` (a previous result of the same call,
    reused so that a timed call does not allocate), else new ones."""
    if out is None:
        return [np.full(shape, fill, dt) for shape, dt, fill in specs]
    arrs = []
    for (name, (shape, dt, _)) in zip(out["_names"], specs):
        a = out[name]
        if a.shape != shape or a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError(f"out[{name!r}] must be a contiguous {np.dtype(dt)} array of shape {shape}")
        arrs.append(a)
    return arrs


def dispatch_bf16(L: dict, mode: str, x: np.ndarray, topk_w: np.ndarray,
                  topk_idx: np.ndarray, capacity: int | None = None, fill: int = 0,
                  out: dict | None = None) -> dict:
    """bf16 dispatch; `out` (an earlier result of the same shapes) is written in place."""
    x = _c(x, np.uint16)
    w = _c(topk_w, np.float32)
    idx = _c(topk_idx, np.int32)
    T, H = x.shape
    K = L["K"]
    m, R, src = _rows_and_src(L, mode)
    cap = R if capacity is None else capacity
    recv_x, recv_w, recv_i = _out_arrays(out, [((cap, H), np.uint16, fill), ((cap, K), np.float32, 0),
                                               ((cap, K), np.int32, 0)])
    _load().oracle_dispatch_bf16(m, K, H, R, _p(src), _p(x), _p(w), _p(idx), _p(recv_x),
                                 _p(recv_w), _p(recv_i))
    return {"recv_x": recv_x, "recv_w": recv_w, "recv_idx": recv_i, "R": R,
            "_names": ("recv_x", "recv_w", "recv_idx")}


def dispatch_fp8(L: dict, mode: str, x: np.ndarray, topk_w: np.ndarray,
                 topk_idx: np.ndarray, capacity: int | None = None, out: dict | None = None) -> dict:
    """FP8 dispatch; `out` (an earlier result of the same shapes) is written in place."""
    x = _c(x, np.uint16)
    w = _c(topk_w, np.float32)
    idx = _c(topk_idx, np.int32)
    T, H = x.shape
    if H % 128:
        raise ValueError("FP8 dispatch needs H % 128 == 0")
    K = L["K"]
    m, R, src = _rows_and_src(L, mode)
    cap = R if capacity is None else capacity
    recv_q, recv_s, recv_w, recv_i = _out_arrays(out, [
        ((cap, H), np.uint8, 0), ((cap, H // 128), np.float32, 0), ((cap, K), np.float32, 0),
        ((cap, K), np.int32, 0)])
    _load().oracle_dispatch_fp8(m, T, K, H, R, _p(src), _p(x), _p(w), _p(idx), _p(recv_q),
                                _p(recv_s), _p(recv_w), _p(recv_i))
    return {"recv_q": recv_q, "recv_scale": recv_s, "recv_w": recv_w, "recv_idx": recv_i, "R": R,
            "_names": ("recv_q", "recv_scale", "recv_w", "recv_idx")}


def quantize_row_fp8(xrow: np.ndarray):
    xrow = _c(xrow, np.uint16)
    H = xrow.shape[0]
    q = np.zeros(H, np.uint8)
    s = np.zeros(H // 128, np.float32)
    _load().oracle_quantize_row_fp8(H, _p(xrow), _p(q), _p(s))
    return q, s


def dequant_fp8(q: np.ndarray, scale: np.ndarray, R: int | None = None) -> np.ndarray:
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    rows, H = q.shape
    R = rows if R is None else R
    y = np.zeros((rows, H), np.uint16)
    _load().oracle_dequant_fp8(R, H, _p(q), _p(scale), _p(y))
    return y


def combine(L: dict, mode: str, y: np.ndarray, topk_w: np.ndarray,
            out: np.ndarray | None = None) -> np.ndarray:
    """Combine; `out` (a bf16-bits [T, H] array) is written in place if given."""
    y = _c(y, np.uint16)
    w = _c(topk_w, np.float32)
    T, K = L["T"], L["K"]
    H = y.shape[1]
    slot = L["slot_e"] if mode == "expert" else L["slot_g"]
    if out is None:
        out = np.zeros((T, H), np.uint16)
    elif out.shape != (T, H) or out.dtype != np.uint16 or not out.flags.c_contiguous:
        raise ValueError(f"out must be a contiguous uint16 array of shape {(T, H)}")
    _load().oracle_combine(T, K, H, _p(slot), _p(y), _p(w), _p(out))
    return out


def regroup_rows(L: dict, rows_g: np.ndarray) -> np.ndarray:
    """Per-group receive rows -> per-expert receive rows (any per-row array)."""
    rows_g = np.ascontiguousarray(rows_g)
    R = L["R_expert"]
    out = np.zeros((R,) + rows_g.shape[1:], rows_g.dtype)
    row_bytes = rows_g.dtype.itemsize * int(np.prod(rows_g.shape[1:], dtype=np.int64))
    _load().oracle_regroup_rows(R, row_bytes, _p(L["recv_src_e"]), _p(L["slot_g"]), _p(rows_g),
                                _p(out))
    return out


def regroup(L: dict, D_group: dict) -> dict:
    """Regroup every array of a per-group dispatch result into the per-expert layout."""
    out = {"R": L["R_expert"]}
    for name in ("recv_x", "recv_q", "recv_scale", "recv_w", "recv_idx"):
        if name in D_group:
            out[name] = regroup_rows(L, D_group[name])
    return out


def cast_transpose_fp8(expert_offset: np.ndarray, x: np.ndarray, scale: np.ndarray,
                       amax_in: np.ndarray | None = None) -> dict:
    """Per-expert FP8 cast + padded transpose of per-expert rows x (bf16 bits [R, H])."""
    off = _c(expert_offset, np.int32)
    E = off.shape[0] - 1
    x = _c(x, np.uint16)
    H = x.shape[1]
    R = int(off[E])
    counts = np.diff(off)
    tot = int(((counts + 15) // 16 * 16).sum())
    c = np.zeros((max(R, x.shape[0]), H), np.uint8)
    t = np.zeros(tot * H, np.uint8)
    amax = np.zeros(E, np.float32) if amax_in is None else _c(amax_in, np.float32).copy()
    po = np.zeros(E + 1, np.int32)
    _load().oracle_cast_transpose_fp8(E, H, _p(off), _p(x), _p(_c(scale, np.float32)), _p(c), _p(t),
                                      _p(amax), _p(po))
    return {"c": c[:R], "t": t, "amax": amax, "pad_offset": po}


# scalar codecs, exposed for exhaustive tests
def bf16_to_f32(h: int) -> float:
    return _load().oracle_bf16_to_f32(h)


def f32_to_bf16(f: float) -> int:
    return _load().oracle_f32_to_bf16(f)


def e4m3_to_f32(c: int) -> float:
    return _load().oracle_e4m3_to_f32(c)


def f32_to_e4m3(f: float) -> int:
    return _load().oracle_f32_to_e4m3(f)


def f32_to_bf16_array(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32).ravel()
    out = np.zeros(a.shape, np.uint16)
    _load().oracle_f32_to_bf16_n(a.size, _p(a), _p(out))
    return out


def f32_to_e4m3_array(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32).ravel()
    out = np.zeros(a.shape, np.uint8)
    _load().oracle_f32_to_e4m3_n(a.size, _p(a), _p(out))
    return out
