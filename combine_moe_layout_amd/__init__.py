"""MoE token path on one MI355X (gfx950): routing layout -> dispatch -> combine.

A thin Python binding over the C ABI of libmoe_ep.so (include/moe_ep.h). It
only marshals arguments: every step of the path runs in the library's HIP
kernels, on the current torch stream. torch provides device memory and
streams; the helpers below allocate outputs with torch when the caller does
not pass them.

The binding names follow the C ABI:
    moe_layout(topk_idx, E, G)                          -> Layout
    moe_dispatch(L, x, topk_w, topk_idx, mode, dtype)   -> Dispatched
    moe_layout_dispatch(topk_idx, E, G, x, topk_w, mode, dtype) -> (Layout, Dispatched)
    moe_regroup(L, Dispatched_group)                    -> Dispatched (per-expert)
    moe_cast_transpose_fp8(L, x_expert, scale)          -> CastTransposed
    moe_combine(L, y, topk_w, mode)                     -> bf16 [T, H]
    moe_fp8_dequant(L, q, scale, mode)                  -> bf16 [capacity, H]
If the library is missing this module raises on import; there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

__all__ = [
    "MoeError", "MoeDataError", "Layout", "Dispatched", "moe_layout", "moe_dispatch", "moe_combine",
    "moe_layout_dispatch", "moe_layout_dispatch_noalloc", "moe_regroup", "moe_cast_transpose_fp8", "CastTransposed",
    "moe_fp8_dequant", "moe_ref_copy", "moe_ref_mix", "recv_rows_bound", "layout_workspace_bytes",
    "library_path", "MODE_EXPERT", "MODE_GROUP", "DTYPE_BF16", "DTYPE_FP8",
    "STATUS_BAD_INDEX", "STATUS_DUPLICATE", "STATUS_Y_ROWS", "STATUS_SYNC_FALLBACK",
    "STATUS_ERRORS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_EP_LIB selects another build of the same library (e.g. a tuning variant).
_LIB_PATH = os.environ.get("MOE_EP_LIB") or os.path.join(_PKG, "libmoe_ep.so")

MODE_EXPERT, MODE_GROUP = 0, 1
DTYPE_BF16, DTYPE_FP8 = 0, 1
STATUS_BAD_INDEX, STATUS_DUPLICATE, STATUS_Y_ROWS, STATUS_SYNC_FALLBACK = 1, 2, 4, 8
STATUS_ERRORS = STATUS_BAD_INDEX | STATUS_DUPLICATE | STATUS_Y_ROWS
_MODES = {"expert": MODE_EXPERT, "group": MODE_GROUP, MODE_EXPERT: MODE_EXPERT, MODE_GROUP: MODE_GROUP}
_DTYPES = {"bf16": DTYPE_BF16, "fp8": DTYPE_FP8, DTYPE_BF16: DTYPE_BF16, DTYPE_FP8: DTYPE_FP8}

_P = ctypes.c_void_p


class _LayoutT(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("K", ctypes.c_int32), ("E", ctypes.c_int32),
                ("G", ctypes.c_int32)] + [(n, _P) for n in (
                    "expert_count", "expert_offset", "group_count", "group_offset",
                    "tok_group_mask", "slot_e", "slot_g", "slot_tg", "recv_src_e",
                    "recv_src_g", "status")]


def _load_library() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python combine_moe_layout_amd/build.py` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(_LayoutT)
    sig = {
        "moe_abi_version": (i32, []),
        "moe_layout_workspace_bytes": (i32, [i32, i32, i32, i32, ctypes.POINTER(sz)]),
        "moe_recv_rows_bound": (i64, [i32, i32, i32, i32]),
        "moe_layout": (i32, [_P, LP, _P, sz, _P]),
        "moe_dispatch": (i32, [LP, i32, i32, i32, _P, _P, _P, _P, _P, _P, _P, i64, _P]),
        "moe_combine": (i32, [LP, i32, i32, _P, i64, _P, _P, _P]),
        "moe_layout_dispatch": (i32, [_P, LP, _P, ctypes.c_size_t, i32, i32, i32, _P, _P, _P, _P, _P, _P, i64, _P]),
        "moe_layout_dispatch_noalloc": (i32, [_P, LP, i32, i32, i32, _P, _P, _P, _P, _P, _P, i64, _P]),
        "moe_regroup": (i32, [LP, i32, i32, _P, _P, _P, _P, i64, _P, _P, _P, _P, i64, _P]),
        "moe_cast_transpose_t_bytes": (i64, [i32, i32, i32, i32]),
        "moe_cast_transpose_fp8": (i32, [LP, i32, _P, i64, _P, _P, _P, i64, _P, _P, _P]),
        "moe_fp8_dequant": (i32, [LP, i32, i32, _P, _P, _P, i64, _P]),
        "moe_ref_copy": (i32, [_P, _P, i64, _P]),
        "moe_ref_mix": (i32, [_P, _P, i64, i64, i32, i32, _P]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load_library()


def library_path() -> str:
    return _LIB_PATH


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.moe_status_string(code).decode()} (code {code})")


class MoeDataError(RuntimeError):
    """The device status word reports bad input (see Layout.check_status)."""

    def __init__(self, status: int):
        self.status = status
        why = [n for b, n in ((STATUS_BAD_INDEX, "expert index out of range"),
                              (STATUS_DUPLICATE, "expert repeated within a token"),
                              (STATUS_Y_ROWS, "combine slot past the rows of y")) if status & b]
        super().__init__(f"layout status {status:#x}: " + ", ".join(why))


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise MoeError(rc, where)


def _ptr(t: torch.Tensor | None):
    """Device address of a tensor for the C ABI. A host tensor is refused here: its
    address given to a kernel would be a GPU memory fault, not an error code."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("arrays passed to the library must be GPU tensors (device memory)")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    """hipStream_t of `stream`, or of torch's current stream on the current device.
    torch's raw-handle getter avoids building a Stream object per call (about 2.8 us
    of host time per call on MI355X hosts); the public API is the fallback."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor | None, dtype: torch.dtype, shape: tuple, name: str) -> None:
    """Refuse an array the library would read or write out of bounds: the C ABI gets
    only pointers and row counts, so a wrong dtype, shape or stride here would be a
    GPU memory fault there, not an error code."""
    if t is not None and t.dtype is dtype and t.shape == shape and t.is_contiguous():
        return
    got = "None" if t is None else f"{t.dtype} {tuple(t.shape)}" + ("" if t.is_contiguous() else " (strided)")
    raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}; got {got}")


def _rows(t: torch.Tensor, name: str) -> int:
    if t is None or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return t.shape[0]


def _mode(mode) -> int:
    if mode not in _MODES:
        raise MoeError(-7, f"mode {mode!r}")
    return _MODES[mode]


def _dtype(dtype) -> int:
    if dtype not in _DTYPES:
        raise MoeError(-7, f"dtype {dtype!r}")
    return _DTYPES[dtype]


def recv_rows_bound(T: int, K: int, G: int, mode="expert") -> int:
    r = _lib.moe_recv_rows_bound(T, K, G, _mode(mode))
    if r < 0:
        raise MoeError(int(r), "moe_recv_rows_bound")
    return int(r)


def layout_workspace_bytes(T: int, K: int, E: int, G: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_layout_workspace_bytes(T, K, E, G, ctypes.byref(n)), "moe_layout_workspace_bytes")
    return int(n.value)


@dataclasses.dataclass
class Layout:
    """Device arrays of one routing layout (see moe_layout_t in include/moe_ep.h)."""
    T: int
    K: int
    E: int
    G: int
    expert_count: torch.Tensor
    expert_offset: torch.Tensor
    group_count: torch.Tensor
    group_offset: torch.Tensor
    tok_group_mask: torch.Tensor
    slot_e: torch.Tensor
    slot_g: torch.Tensor
    slot_tg: torch.Tensor
    recv_src_e: torch.Tensor
    recv_src_g: torch.Tensor
    status: torch.Tensor
    workspace: torch.Tensor

    @classmethod
    def empty(cls, T: int, K: int, E: int, G: int, device="cuda") -> "Layout":
        i32 = dict(dtype=torch.int32, device=device)
        ws = layout_workspace_bytes(T, K, E, G)
        return cls(T, K, E, G,
                   torch.empty(E, **i32), torch.empty(E + 1, **i32),
                   torch.empty(G, **i32), torch.empty(G + 1, **i32),
                   torch.empty(T, **i32),    # uint32 bits, held as int32
                   torch.empty(T * K, **i32), torch.empty(T * K, **i32),
                   torch.empty(T * G, **i32), torch.empty(T * K, **i32),
                   torch.empty(T * min(K, G), **i32), torch.zeros(1, **i32),
                   torch.empty(max(ws, 1), dtype=torch.uint8, device=device))

    _FIELDS = ("expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask",
               "slot_e", "slot_g", "slot_tg", "recv_src_e", "recv_src_g", "status")

    def struct(self) -> _LayoutT:
        """The moe_layout_t of these tensors (built once; the tensors of a Layout
        must not be replaced after its first use)."""
        st = self.__dict__.get("_struct")
        if st is None:
            self._validate()
            st = _LayoutT(self.T, self.K, self.E, self.G, *(_ptr(getattr(self, n)) for n in self._FIELDS))
            self.__dict__["_struct"] = st
            self.__dict__["_struct_ref"] = ctypes.byref(st)
        return st

    def _validate(self) -> None:
        T, K, E, G = self.T, self.K, self.E, self.G
        sizes = {"expert_count": E, "expert_offset": E + 1, "group_count": G, "group_offset": G + 1,
                 "tok_group_mask": T, "slot_e": T * K, "slot_g": T * K, "slot_tg": T * G,
                 "recv_src_e": T * K, "recv_src_g": T * min(K, G), "status": 1}
        for n, size in sizes.items():
            _need(getattr(self, n), torch.int32, (size,), f"Layout.{n}")
        ws = self.workspace
        if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
            raise ValueError("Layout.workspace must be a contiguous 1-D uint8 tensor")

    def ref(self):
        self.struct()
        return self.__dict__["_struct_ref"]

    def rows(self, mode="expert") -> torch.Tensor:
        """Device scalar tensor: number of receive rows in `mode`."""
        return self.expert_offset[self.E] if _mode(mode) == MODE_EXPERT else self.group_offset[self.G]

    def slots(self, mode="expert") -> torch.Tensor:
        return self.slot_e if _mode(mode) == MODE_EXPERT else self.slot_g

    def check_status(self) -> int:
        """Read the device status word (this waits for the work queued before it on the
        current stream) and raise MoeDataError if an error bit is set: an expert index
        out of range, an expert repeated within a token, or a combine slot past the rows
        of y. Returns the word, which may also hold the diagnostic STATUS_SYNC_FALLBACK
        (results exact). The calls themselves stay asynchronous and never read it."""
        st = int(self.status.item())
        if st & STATUS_ERRORS:
            raise MoeDataError(st)
        return st


def moe_layout(topk_idx: torch.Tensor, E: int, G: int, *, out: Layout | None = None,
               stream=None) -> Layout:
    """Routing layout of device int32 [T, K] expert indices (moe_layout)."""
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 2 or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous int32 [T, K] tensor")
    T, K = topk_idx.shape
    L = out if out is not None else Layout.empty(T, K, E, G, device=topk_idx.device)
    if (L.T, L.K, L.E, L.G) != (T, K, E, G):
        raise ValueError("layout buffers were made for other sizes")
    _check(_lib.moe_layout(_ptr(topk_idx), L.ref(), _ptr(L.workspace),
                           L.workspace.numel(), _stream(stream)), "moe_layout")
    return L


@dataclasses.dataclass(frozen=True)
class Dispatched:
    """Receive arrays. Checked once, here, for agreeing shapes and dense storage; a
    call then checks only H, K and the element type (the arrays must not be resized
    in place afterwards)."""
    recv_x: torch.Tensor          # bf16 [cap, H] or uint8 [cap, H]
    recv_scale: torch.Tensor | None   # fp32 [cap, H/128] for FP8
    recv_topk_w: torch.Tensor     # fp32 [cap, K]
    recv_topk_idx: torch.Tensor   # int32 [cap, K]

    def __post_init__(self):
        x = self.recv_x
        if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.uint8):
            raise ValueError("recv_x must be a bf16 or uint8 [cap, H] tensor")
        cap, H = x.shape
        _need(x, x.dtype, (cap, H), "recv_x")
        if self.recv_scale is not None:
            _need(self.recv_scale, torch.float32, (cap, H // 128), "recv_scale")
        if self.recv_topk_w.dim() != 2:
            raise ValueError("recv_topk_w must be a [cap, K] tensor")
        K = self.recv_topk_w.shape[1]
        _need(self.recv_topk_w, torch.float32, (cap, K), "recv_topk_w")
        _need(self.recv_topk_idx, torch.int32, (cap, K), "recv_topk_idx")


def _check_dispatched(D: Dispatched, H: int, K: int, fp8: bool, name: str) -> None:
    """Receive arrays (consistent since construction) fit this call's H, K and dtype."""
    if D.recv_x.dtype is not (torch.uint8 if fp8 else torch.bfloat16) or D.recv_x.shape[1] != H:
        raise ValueError(f"{name}.recv_x must be {'uint8' if fp8 else 'bf16'} [cap, {H}]")
    if fp8 and D.recv_scale is None:
        raise ValueError(f"{name}.recv_scale is needed for FP8 rows")
    if D.recv_topk_w.shape[1] != K:
        raise ValueError(f"{name}.recv_topk_w must have K = {K} columns")


def alloc_dispatch(L: Layout, H: int, mode="expert", dtype="bf16", device="cuda",
                   capacity: int | None = None) -> Dispatched:
    cap = recv_rows_bound(L.T, L.K, L.G, mode) if capacity is None else capacity
    fp8 = _dtype(dtype) == DTYPE_FP8
    return Dispatched(
        torch.empty((cap, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=device),
        torch.empty((cap, H // 128), dtype=torch.float32, device=device) if fp8 else None,
        torch.empty((cap, L.K), dtype=torch.float32, device=device),
        torch.empty((cap, L.K), dtype=torch.int32, device=device))


def moe_dispatch(L: Layout, x: torch.Tensor, topk_w: torch.Tensor, topk_idx: torch.Tensor,
                 mode="expert", dtype="bf16", *, out: Dispatched | None = None,
                 stream=None) -> Dispatched:
    """Scatter bf16 rows x [T, H] (+ weights, indices) into receive buffers (moe_dispatch)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T, H] tensor")
    for t, dt in ((topk_w, torch.float32), (topk_idx, torch.int32)):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != (L.T, L.K):
            raise ValueError("topk_w / topk_idx must be contiguous [T, K] fp32 / int32")
    if x.shape[0] != L.T:
        raise ValueError("x must have one row per token of the layout")
    H = x.shape[1]
    D = out if out is not None else alloc_dispatch(L, H, mode, dtype, x.device)
    _check_dispatched(D, H, L.K, _dtype(dtype) == DTYPE_FP8, "out")
    _check(_lib.moe_dispatch(L.ref(), _mode(mode), _dtype(dtype), H, _ptr(x),
                             _ptr(topk_w), _ptr(topk_idx), _ptr(D.recv_x), _ptr(D.recv_scale),
                             _ptr(D.recv_topk_w), _ptr(D.recv_topk_idx), D.recv_x.shape[0],
                             _stream(stream)), "moe_dispatch")
    return D


FUSED_MAX_TOKENS, FUSED_MAX_PAIRS = 512, 16384


def moe_layout_dispatch(topk_idx: torch.Tensor, E: int, G: int, x: torch.Tensor,
                        topk_w: torch.Tensor, mode="expert", dtype="bf16", *,
                        out_layout: Layout | None = None, out: Dispatched | None = None,
                        use_workspace: bool = True, stream=None) -> tuple[Layout, Dispatched]:
    """moe_layout + moe_dispatch as one call (moe_layout_dispatch): one launch for the
    smallest batches (T * K * E <= 4096), else the count kernel and a dispatch that
    computes the offsets (its workgroup 0, or a workgroup launched before it for large
    batches) and places its own tokens.
    use_workspace=False passes no workspace, which asks for the one-launch form
    (T <= 512 and T * K <= 16384)."""
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 2 or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous int32 [T, K] tensor")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T, H] tensor")
    T, K = topk_idx.shape
    if topk_w.dtype != torch.float32 or not topk_w.is_contiguous() or tuple(topk_w.shape) != (T, K):
        raise ValueError("topk_w must be a contiguous fp32 [T, K] tensor")
    L = out_layout if out_layout is not None else Layout.empty(T, K, E, G, device=topk_idx.device)
    if (L.T, L.K, L.E, L.G) != (T, K, E, G):
        raise ValueError("layout buffers were made for other sizes")
    if x.shape[0] != T:
        raise ValueError("x must have one row per token of topk_idx")
    H = x.shape[1]
    D = out if out is not None else alloc_dispatch(L, H, mode, dtype, x.device)
    _check_dispatched(D, H, K, _dtype(dtype) == DTYPE_FP8, "out")
    ws, nb = (_ptr(L.workspace), L.workspace.numel()) if use_workspace else (None, 0)
    _check(_lib.moe_layout_dispatch(_ptr(topk_idx), L.ref(), ws, nb,
                                    _mode(mode), _dtype(dtype), H,
                                    _ptr(x), _ptr(topk_w), _ptr(D.recv_x), _ptr(D.recv_scale),
                                    _ptr(D.recv_topk_w), _ptr(D.recv_topk_idx), D.recv_x.shape[0],
                                    _stream(stream)), "moe_layout_dispatch")
    return L, D


NOALLOC_SCRATCH_BYTES = 8 << 20


def moe_layout_dispatch_noalloc(topk_idx: torch.Tensor, E: int, G: int, x: torch.Tensor,
                                topk_w: torch.Tensor, mode="expert", dtype="bf16", *,
                                out_layout: Layout, out: Dispatched, stream=None) -> tuple[Layout, Dispatched]:
    """moe_layout_dispatch without a workspace (moe_layout_dispatch_noalloc): the library's
    own fixed workspace is used, and nothing is allocated, here or in the library. The
    layout and receive arrays must be passed (out_layout, out). Calls overlapping on one
    GPU race on the library's workspace."""
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 2 or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous int32 [T, K] tensor")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T, H] tensor")
    T, K = topk_idx.shape
    if topk_w.dtype != torch.float32 or not topk_w.is_contiguous() or tuple(topk_w.shape) != (T, K):
        raise ValueError("topk_w must be a contiguous fp32 [T, K] tensor")
    L, D = out_layout, out
    if (L.T, L.K, L.E, L.G) != (T, K, E, G):
        raise ValueError("layout buffers were made for other sizes")
    if x.shape[0] != T:
        raise ValueError("x must have one row per token of topk_idx")
    H = x.shape[1]
    _check_dispatched(D, H, K, _dtype(dtype) == DTYPE_FP8, "out")
    _check(_lib.moe_layout_dispatch_noalloc(_ptr(topk_idx), L.ref(), _mode(mode), _dtype(dtype), H,
                                            _ptr(x), _ptr(topk_w), _ptr(D.recv_x), _ptr(D.recv_scale),
                                            _ptr(D.recv_topk_w), _ptr(D.recv_topk_idx), D.recv_x.shape[0],
                                            _stream(stream)), "moe_layout_dispatch_noalloc")
    return L, D


def moe_regroup(L: Layout, Dg: Dispatched, *, out: Dispatched | None = None,
                stream=None) -> Dispatched:
    """Per-group receive arrays -> per-expert receive arrays (moe_regroup)."""
    fp8 = Dg.recv_scale is not None
    if Dg.recv_x.dim() != 2:
        raise ValueError("the per-group receive rows must be a 2-D tensor")
    H = Dg.recv_x.shape[1]
    _check_dispatched(Dg, H, L.K, fp8, "Dg")
    De = out if out is not None else alloc_dispatch(L, H, "expert", "fp8" if fp8 else "bf16",
                                                    Dg.recv_x.device)
    _check_dispatched(De, H, L.K, fp8, "out")
    _check(_lib.moe_regroup(L.ref(), DTYPE_FP8 if fp8 else DTYPE_BF16, H, _ptr(Dg.recv_x),
                            _ptr(Dg.recv_scale), _ptr(Dg.recv_topk_w), _ptr(Dg.recv_topk_idx),
                            Dg.recv_x.shape[0], _ptr(De.recv_x), _ptr(De.recv_scale),
                            _ptr(De.recv_topk_w), _ptr(De.recv_topk_idx), De.recv_x.shape[0],
                            _stream(stream)), "moe_regroup")
    return De


@dataclasses.dataclass
class CastTransposed:
    c: torch.Tensor            # uint8 [rows, H]: e4m3 of x * scale[e] in the receive layout
    t: torch.Tensor            # uint8 [bytes]: T_e = [H, n_e padded to 16] at H * pad_offset[e]
    amax: torch.Tensor         # fp32 [E]
    pad_offset: torch.Tensor   # int32 [E + 1]

    def t_expert(self, e: int) -> torch.Tensor:
        """T_e as a [H, padded rows] uint8 view (synchronises to read pad_offset)."""
        po = self.pad_offset.cpu()
        H = self.c.shape[1]
        return self.t[H * int(po[e]):H * int(po[e + 1])].view(H, -1)


def moe_cast_transpose_fp8(L: Layout, x: torch.Tensor, scale: torch.Tensor, *,
                           amax: torch.Tensor | None = None, out: CastTransposed | None = None,
                           stream=None) -> CastTransposed:
    """Per-expert FP8 cast + padded transpose of per-expert bf16 rows (moe_cast_transpose_fp8)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [rows, H] tensor (per-expert layout)")
    rows, H = x.shape
    _need(scale, torch.float32, (L.E,), "scale")
    nb = _lib.moe_cast_transpose_t_bytes(L.T, L.K, L.E, H)
    if nb < 0:
        raise MoeError(int(nb), "moe_cast_transpose_t_bytes")
    if out is None:
        out = CastTransposed(torch.empty((rows, H), dtype=torch.uint8, device=x.device),
                             torch.empty(max(nb, 16), dtype=torch.uint8, device=x.device),
                             amax if amax is not None else torch.zeros(L.E, dtype=torch.float32, device=x.device),
                             torch.empty(L.E + 1, dtype=torch.int32, device=x.device))
    _need(out.c, torch.uint8, (rows, H), "out.c")
    if out.t.dtype != torch.uint8 or out.t.dim() != 1 or not out.t.is_contiguous():
        raise ValueError("out.t must be a contiguous 1-D uint8 tensor")
    _need(out.amax, torch.float32, (L.E,), "out.amax")
    _need(out.pad_offset, torch.int32, (L.E + 1,), "out.pad_offset")
    _check(_lib.moe_cast_transpose_fp8(L.ref(), H, _ptr(x), rows, _ptr(scale), _ptr(out.c), _ptr(out.t),
                                       out.t.numel(), _ptr(out.amax), _ptr(out.pad_offset),
                                       _stream(stream)), "moe_cast_transpose_fp8")
    return out


def moe_combine(L: Layout, y: torch.Tensor, topk_w: torch.Tensor, mode="expert", *,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Weighted top-k sum of expert outputs y (bf16 [rows, H]) per token (moe_combine)."""
    if y.dtype != torch.bfloat16 or y.dim() != 2 or not y.is_contiguous():
        raise ValueError("y must be a contiguous bf16 [rows, H] tensor")
    H = y.shape[1]
    _need(topk_w, torch.float32, (L.T, L.K), "topk_w")
    o = out if out is not None else torch.empty((L.T, H), dtype=torch.bfloat16, device=y.device)
    _need(o, torch.bfloat16, (L.T, H), "out")
    _check(_lib.moe_combine(L.ref(), _mode(mode), H, _ptr(y), y.shape[0], _ptr(topk_w),
                            _ptr(o), _stream(stream)), "moe_combine")
    return o


def moe_fp8_dequant(L: Layout, q: torch.Tensor, scale: torch.Tensor, mode="expert", *,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Identity expert on FP8 receive rows: bf16(decode(q) * scale) (moe_fp8_dequant)."""
    cap = _rows(q, "q")
    H = q.shape[1]
    _need(q, torch.uint8, (cap, H), "q")
    _need(scale, torch.float32, (cap, H // 128), "scale")
    y = out if out is not None else torch.empty((cap, H), dtype=torch.bfloat16, device=q.device)
    _need(y, torch.bfloat16, (cap, H), "out")
    _check(_lib.moe_fp8_dequant(L.ref(), _mode(mode), H, _ptr(q), _ptr(scale), _ptr(y),
                                cap, _stream(stream)), "moe_fp8_dequant")
    return y


def moe_ref_copy(dst: torch.Tensor, src: torch.Tensor, nbytes: int | None = None,
                 stream=None) -> None:
    """Plain 16-byte streaming copy (measurement reference, not part of the method)."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if not (src.is_contiguous() and dst.is_contiguous()) or n > min(src.numel() * src.element_size(),
                                                                      dst.numel() * dst.element_size()):
        raise ValueError("moe_ref_copy: contiguous src and dst of at least nbytes each")
    _check(_lib.moe_ref_copy(_ptr(dst), _ptr(src), n, _stream(stream)), "moe_ref_copy")


def moe_ref_mix(dst: torch.Tensor, src: torch.Tensor, row_bytes: int, nr: int, nw: int,
                stream=None) -> int:
    """Read/write-mix reference (measurement aid, not part of the method): nr rows of src
    read per nw rows of dst written, rows of row_bytes bytes, as many units as both
    buffers hold; returns the number of units."""
    nbs, nbd = src.numel() * src.element_size(), dst.numel() * dst.element_size()
    if not (src.is_contiguous() and dst.is_contiguous()) or row_bytes <= 0:
        raise ValueError("moe_ref_mix: contiguous src and dst and a positive row size")
    units = min(nbs // (row_bytes * nr), nbd // (row_bytes * nw))
    _check(_lib.moe_ref_mix(_ptr(dst), _ptr(src), row_bytes, units, nr, nw, _stream(stream)), "moe_ref_mix")
    return int(units)
