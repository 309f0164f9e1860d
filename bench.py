"""Benchmark of the MoE token path on one MI355X: layout -> dispatch -> combine.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t4096]

One step = one pass of the hot path over one batch of synthetic input already
resident in HBM: the routing layout (per-expert and per-group) and the dispatch
of bf16 rows into per-expert receive buffers, as one moe_layout_dispatch call
(for this batch: the layout's count kernel and a dispatch whose workgroup 0
computes the offsets while every workgroup places its own token), then
moe_combine (fp32 weighted top-k sum back to bf16; the experts are identities,
so combine reads the dispatched rows in place). Default workload: 4096 tokens x
7168 hidden bf16, 256 experts in 8 groups, top-8 uniform routing.

Prints ONE JSON line. `value` = algorithmic HBM bytes of a step (reads + writes,
each byte counted once) / wall time per step, the median over --processes
separate processes (this one and fresh children, one after another). Per-call
times come from HIP events recorded around every call of every 4th timed step,
on the stream the kernels run on; every timed step writes a status word of its
own, all checked after the timed region. The same line carries
the roofline of the dominant kernel (the combine), the CPU oracle timed on the
host cores (its single-thread canonical build and its OpenMP build on every
core, per call and per workload, asserted bit-identical), and secondary
measurements: the same step as three calls, the per-group layout, FP8 dispatch,
each call's read/write-mix ceiling and a plain copy, cold-cache timings, and
every call on every workload with its parity against the oracle.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
EVENT_EVERY = 4           # per-call events on every 4th timed step
WORKLOAD_NAMES = ("tiny", "t256", "t4096", "skew", "fp8")


# ------------------------------------------------------------------ algorithmic bytes

def layout_bytes(T, K, E, G, P):
    return T * K * 4 + (2 * E + 2 * G + 2) * 4 + T * 4 + 3 * T * K * 4 + T * G * 4 + P * 4


def dispatch_bytes(T, H, K, G, R, mode, fp8=False):
    reads = T * H * 2 + T * K * 8 + (T * K * 4 if mode == "expert" else T * G * 4)
    row = (H + (H // 128) * 4 if fp8 else H * 2) + K * 8
    return reads, R * row


def combine_bytes(T, H, K, R):
    return R * H * 2 + T * K * 4 + T * K * 4, T * H * 2


# ------------------------------------------------------------------ helpers

# Source files that define each timed kernel (plus the shared device helpers).
KERNEL_SOURCES = {
    "dispatch": ("dispatch.hip", "place.hpp", "common.hpp", "kernels.hpp"),
    "combine": ("combine.hip", "common.hpp", "kernels.hpp"),
    "layout": ("layout.hip", "layout_exchange.hip", "layout_tile.hpp", "common.hpp", "kernels.hpp"),
    "regroup": ("regroup.hip", "common.hpp", "kernels.hpp"),
    "cast_transpose": ("cast_transpose.hip", "common.hpp", "kernels.hpp"),
}


_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


def code_text(src: str) -> str:
    """The code of a C++ source with its comments and blank space removed, so that a
    comment edit leaves a kernel's hash (and its recorded counters) valid. The kernel
    sources hold no string literal containing comment markers."""
    return " ".join(_COMMENT.sub(" ", src).split())


def source_hash(kernel: str | None = None) -> str:
    """Hash of the code (comments and spacing aside) of the sources of one kernel, or
    of all kernel sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_moe_layout_amd", "csrc")
    files = KERNEL_SOURCES[kernel] if kernel else sorted(os.listdir(csrc))
    for fn in files:
        h.update(fn.encode())
        h.update(code_text(open(os.path.join(csrc, fn), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def load_counters(key: str):
    """The committed rocprofv3 --pmc record of one kernel instance, if it was taken on
    that kernel's current sources; None otherwise."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        k = json.load(open(p)).get("kernels", {}).get(key)
    except ValueError:
        return None
    if not k or k.get("source_hash") != source_hash(k.get("kernel", key.split("_")[0])):
        return None
    return k


def load_traffic(key: str):
    """HBM traffic (bytes per launch) of a kernel instance from the committed counters,
    or None (no record, or taken on other sources)."""
    k = load_counters(key)
    return None if k is None else k.get("traffic_bytes")


def stats(v):
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"median": float(np.median(a)), "mean": float(a.mean()), "std": float(a.std()),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "best": float(a.min())}


class Dev:
    """Device copies of one workload and its buffers."""

    def __init__(self, moe, d, modes=("expert",), dtype="bf16"):
        import numpy as np
        import torch
        wl = d["workload"]
        self.wl = wl
        self.x = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
        self.w = torch.from_numpy(d["topk_w"]).cuda()
        self.idx = torch.from_numpy(d["topk_idx"]).cuda()
        self.L = moe.Layout.empty(wl.T, wl.K, wl.E, wl.G)
        self.D = {m: moe.alloc_dispatch(self.L, wl.H, m, dtype) for m in modes}
        self.out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        self.y = {}


def time_calls(fns, iters, flush=None):
    """Median-able per-call times (µs) of each fn in fns, run in sequence per iteration,
    each bracketed by events on the current stream; optional flush outside the events."""
    import torch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in fns] for _ in range(iters)]
    for it in range(iters):
        for j, fn in enumerate(fns):
            if flush is not None:
                flush()
            a, b = ev[it][j]
            a.record()
            fn()
            b.record()
    torch.cuda.synchronize()
    return [[ev[it][j][0].elapsed_time(ev[it][j][1]) * 1e3 for it in range(iters)]
            for j in range(len(fns))]


def time_stream(fn, n=100, lead=20):
    """µs per call of fn issued n times back to back between two events, after `lead`
    calls that fill the queue (the host issues a call faster than the GPU runs it,
    so the GPU never waits for the host): what a call costs in a stream of work,
    without the fixed cost that a pair of events around each call adds."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(lead):
        fn()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def host_bits(t):
    """A device tensor's bytes on the host, as unsigned integers of its element size."""
    import numpy as np
    import torch
    t = t.contiguous()
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ CPU oracle leg

def _timed(fn, budget_s=0.4, max_reps=7):
    """(last result, median µs) of fn repeated until budget_s is spent (at least once)."""
    import numpy as np
    ts, r = [], None
    t_start = time.perf_counter()
    while len(ts) < max_reps:
        t0 = time.perf_counter()
        r = fn()
        ts.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    return r, float(np.median(ts)) * 1e6


def _prefilled(D):
    """Arrays shaped like a dispatch result, filled with a pattern (so their pages are
    touched before a timed call writes them and an unwritten element shows)."""
    import numpy as np
    out = {k: (np.full_like(v, 0x5A) if isinstance(v, np.ndarray) else v) for k, v in D.items()}
    return out


def oracle_leg(d, nthreads: int):
    """Both oracle builds on every call of one workload: the per-call times (the C call
    with its outputs already allocated and touched), the two builds' outputs compared
    byte for byte, and the OpenMP build's outputs for the GPU parity check."""
    import numpy as np
    import oracle
    wl = d["workload"]
    T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    x, w, idx = d["x"], d["topk_w"], d["topk_idx"]
    disp = oracle.dispatch_fp8 if wl.fp8 else oracle.dispatch_bf16
    us = {"openmp": {}, "serial": {}}
    res = {}
    # the OpenMP build first: its first call of each kind allocates and touches the arrays
    with oracle.variant("openmp"):
        oracle.set_threads(nthreads)
        threads = oracle.threads()
        L, us["openmp"]["layout"] = _timed(lambda: oracle.layout(idx, E, G))
        res["L"] = L
        for mode in ("expert", "group"):
            D0 = disp(L, mode, x, w, idx)
            D, us["openmp"][f"dispatch_{mode}"] = _timed(lambda: disp(L, mode, x, w, idx, out=D0))
            y = oracle.dequant_fp8(D["recv_q"], D["recv_scale"]) if wl.fp8 else D["recv_x"]
            c0 = oracle.combine(L, mode, y, w)
            c, us["openmp"][f"combine_{mode}"] = _timed(lambda: oracle.combine(L, mode, y, w, out=c0))
            res[mode] = {"D": D, "y": y, "out": c}
    identical = True
    with oracle.variant("serial"):
        Ls, us["serial"]["layout"] = _timed(lambda: oracle.layout(idx, E, G))
        identical &= all(np.array_equal(Ls[k], L[k]) for k in L if isinstance(L[k], np.ndarray))
        identical &= Ls["status"] == L["status"]
        for mode in ("expert", "group"):
            ref = res[mode]
            Dp = _prefilled(ref["D"])
            Ds, us["serial"][f"dispatch_{mode}"] = _timed(lambda: disp(Ls, mode, x, w, idx, out=Dp))
            identical &= all(Ds[k].tobytes() == ref["D"][k].tobytes() for k in ref["D"]["_names"])
            cp = np.full_like(ref["out"], 0x5A5A)
            cs, us["serial"][f"combine_{mode}"] = _timed(lambda: oracle.combine(Ls, mode, ref["y"], w, out=cp))
            identical &= cs.tobytes() == ref["out"].tobytes()
            del Ds, Dp, cs, cp
    if not identical:
        raise RuntimeError(f"{wl.name}: the OpenMP oracle build differs from the canonical build")
    nbytes = {"layout": layout_bytes(T, K, E, G, L["R_group"])}
    for mode, rows in (("expert", L["R_expert"]), ("group", L["R_group"])):
        nbytes[f"dispatch_{mode}"] = sum(dispatch_bytes(T, H, K, G, rows, mode, fp8=wl.fp8))
        nbytes[f"combine_{mode}"] = sum(combine_bytes(T, H, K, rows))
    calls = {c: {"us_1": round(us["serial"][c], 1), f"us_{threads}": round(us["openmp"][c], 1),
                 "gbs_1": round(nbytes[c] / us["serial"][c] / 1e3, 3),
                 f"gbs_{threads}": round(nbytes[c] / us["openmp"][c] / 1e3, 3)} for c in nbytes}
    return {"threads": threads, "builds_identical": True, "calls": calls, "bytes": nbytes,
            "us": us}, res


def _ulps(a_u16, b_u16):
    import numpy as np

    def key(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + (u & 0x7FFF))
    return np.abs(key(a_u16) - key(b_u16))


def parity_of(gpu: dict, ora: dict, fp8: bool) -> dict:
    """GPU arrays against the oracle's: layout arrays, receive rows, metadata and (FP8)
    scales bit-exact; combine within 1 bf16 ulp, with the count of differing elements."""
    import numpy as np
    L = ora["L"]
    R, P = L["R_expert"], L["R_group"]
    out = {}
    bad = [n for n in ("expert_count", "expert_offset", "group_count", "group_offset", "slot_e",
                       "slot_g", "slot_tg") if not np.array_equal(gpu["L"][n].view(np.int32), L[n])]
    if not np.array_equal(gpu["L"]["tok_group_mask"], L["tok_group_mask"]):
        bad.append("tok_group_mask")
    if not np.array_equal(gpu["L"]["recv_src_e"][:R].view(np.int32), L["recv_src_e"][:R]):
        bad.append("recv_src_e")
    if not np.array_equal(gpu["L"]["recv_src_g"][:P].view(np.int32), L["recv_src_g"][:P]):
        bad.append("recv_src_g")
    if int(gpu["L"]["status"][0]) & 7 != L["status"]:
        bad.append("status")
    out["layout"] = "bit-exact" if not bad else "MISMATCH: " + ", ".join(bad)
    for mode, rows in (("expert", R), ("group", P)):
        g, o = gpu[mode], ora[mode]
        names = ("recv_q", "recv_scale", "recv_w", "recv_idx") if fp8 else ("recv_x", "recv_w", "recv_idx")
        bad = [n for n in names if g[n][:rows].tobytes() != np.ascontiguousarray(o["D"][n][:rows]).tobytes()]
        out[f"dispatch_{mode}"] = "bit-exact" if not bad else "MISMATCH: " + ", ".join(bad)
        if fp8:
            out[f"dequant_{mode}"] = ("bit-exact" if g["y"][:rows].tobytes() == o["y"][:rows].tobytes()
                                      else "MISMATCH")
        d = _ulps(g["out"], o["out"])
        ndiff = int((g["out"] != o["out"]).sum())
        out[f"combine_{mode}"] = (f"{ndiff} of {g['out'].size} elements differ, max {int(d.max(initial=0))} ulp"
                                  if ndiff else "bit-exact")
    out["ok"] = all(v == "bit-exact" for k, v in out.items())
    return out


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="t4096")
    ap.add_argument("--no-extras", action="store_true", help="only the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the plain reference copy (256 MiB, 5 times): a known byte "
                         "count for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--mix-probes", action="store_true",
                    help="only run the read/write-mix references of the t4096 dispatch (1 row "
                         "read per 8 written) and combine (8 read per 1 written), 5 times each "
                         "back to back: for taking their counters")
    ap.add_argument("--profile", default=None, metavar="WORKLOAD:LAYOUT",
                    help="only the three calls moe_layout, moe_dispatch and moe_combine (and the "
                         "FP8 dequant between them) of one workload and receive layout, 5 times "
                         "in a row, e.g. t4096:group: for taking counters of those kernels")
    ap.add_argument("--processes", type=int, default=3,
                    help="time the step in this many separate processes in all (this one included; "
                         "run one after another); `value` is the median of their values")
    ap.add_argument("--table", default=None, metavar="NAMES",
                    help="only the per-workload table for these comma-separated workloads "
                         "(e.g. t4096): every call of the library on each, timed alone, printed "
                         "as one JSON object; for profiling one workload's kernels")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the expert groups of one EP rank live in one GPU's HBM)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_moe_layout_amd as moe
    import synth_inputs as si

    torch.cuda.init()
    # the GPU should be idle: record how much of its memory is already in use (mori's
    # benchmark script refuses to run above 15%)
    free_b, total_b = torch.cuda.mem_get_info()
    used_before = round(1 - free_b / total_b, 4)
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.full((n,), 3, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(5):
            moe.moe_ref_copy(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy": {"bytes_read": n, "bytes_written": n, "launches": 5}}))
        return
    if args.mix_probes:
        wl = si.WORKLOADS["t4096"]
        row = wl.H * 2
        xs = torch.full((wl.T * row,), 3, dtype=torch.uint8, device="cuda")
        a = torch.full((wl.T * wl.K * row,), 1, dtype=torch.uint8, device="cuda")
        b = torch.full((wl.T * row,), 2, dtype=torch.uint8, device="cuda")
        for _ in range(5):
            moe.moe_ref_mix(a, xs, row, 1, wl.K)   # the dispatch's mix: xs -> a
            moe.moe_ref_mix(b, a, row, wl.K, 1)    # the combine's mix: a -> b
        torch.cuda.synchronize()
        print(json.dumps({"mix_probes": {"row_bytes": row, "units": wl.T, "k": wl.K, "launches": 5}}))
        return
    if args.profile:
        name, mode = args.profile.split(":")
        d = si.make_workload(name)
        wl = d["workload"]
        dt = "fp8" if wl.fp8 else "bf16"
        dv = Dev(moe, d, modes=(mode,), dtype=dt)
        L, D = dv.L, dv.D[mode]
        for _ in range(5):
            moe.moe_layout(dv.idx, wl.E, wl.G, out=L)
            moe.moe_dispatch(L, dv.x, dv.w, dv.idx, mode, dt, out=D)
            y = moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode) if wl.fp8 else D.recv_x
            moe.moe_combine(L, y, dv.w, mode, out=dv.out)
        torch.cuda.synchronize()
        L.check_status()
        print(json.dumps({"profile": args.profile, "rows": int(L.rows(mode).item()),
                          "group_rows": int(L.group_offset[wl.G].item()), "launches": 5}))
        return
    if args.table:
        names = tuple(args.table.split(","))
        print(json.dumps({"workloads": workload_table(moe, names=names, oracle_threads=0)}))
        return
    d = si.make_workload(args.workload)
    wl = d["workload"]
    T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    dv = Dev(moe, d, modes=("expert",))
    L, D, out = dv.L, dv.D["expert"], dv.out
    # One status word per timed step: step s runs on a Layout that shares every array
    # of L but its status word, status_words[s] (each step's count kernel clears its
    # own word and the combine adds its bits), so every step's status is kept and
    # checked after the timed region without a kernel of its own inside it.
    status_words = torch.full((args.steps,), -1, dtype=torch.int32, device="cuda")
    Ls = [dataclasses.replace(L, status=status_words[s:s + 1]) for s in range(args.steps)]
    for Lx in Ls:
        Lx.ref()   # the C structs, built before the timed region

    # one step: routing layout + dispatch as one call (the library's form for this
    # batch: the count kernel, then a dispatch whose workgroup 0 computes the offsets
    # and whose workgroups place their own tokens), then the combine; the three
    # separate calls are timed in extras
    def step(Lx):
        moe.moe_layout_dispatch(dv.idx, E, G, dv.x, dv.w, "expert", "bf16", out_layout=Lx, out=D)
        moe.moe_combine(Lx, D.recv_x, dv.w, "expert", out=out)

    for _ in range(args.warmup):
        step(L)
    torch.cuda.synchronize()

    # Per-call HIP events on every EVENT_EVERY-th timed step: a sample of the timed
    # region for the per-call times, while most steps carry no event records (each
    # record is a command of its own, ~4 us here, which would otherwise inflate the
    # wall time the value is computed from).
    sampled = [s for s in range(args.steps) if s % EVENT_EVERY == 0]
    ev = {s: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for s in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev.get(s)
        Lx = Ls[s]
        if e:
            e[0].record()
        moe.moe_layout_dispatch(dv.idx, E, G, dv.x, dv.w, "expert", "bf16", out_layout=Lx, out=D)
        if e:
            e[1].record()
        moe.moe_combine(Lx, D.recv_x, dv.w, "expert", out=out)
        if e:
            e[2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / args.steps * 1e3
    us = {name: [ev[s][i].elapsed_time(ev[s][i + 1]) * 1e3 for s in sampled]
          for i, name in enumerate(("layout_dispatch", "combine"))}

    words = status_words.cpu().numpy()
    if (words == -1).any():
        raise RuntimeError("a timed step left its status word unwritten")
    step_status = int(np.bitwise_or.reduce(words))
    if step_status & moe.STATUS_ERRORS:
        raise RuntimeError(f"a timed step's status word reported bad data: {step_status:#x}")
    R = int(L.expert_offset[E].item())
    P = int(L.group_offset[G].item())
    b_layout = layout_bytes(T, K, E, G, P)
    d_r, d_w = dispatch_bytes(T, H, K, G, R, "expert")
    c_r, c_w = combine_bytes(T, H, K, R)
    step_bytes = b_layout + d_r + d_w + c_r + c_w
    value_here = step_bytes / (ms_per_step * 1e-3) / 1e9
    if args.processes > 1:
        procs = other_processes(args, value_here, ms_per_step)
        ms_med = procs["median_ms_per_step"]
    else:
        procs, ms_med = None, ms_per_step
    value = step_bytes / (ms_med * 1e-3) / 1e9

    avg = {k: float(np.mean(v)) for k, v in us.items()}
    # the dominant kernel: combine (the layout + dispatch call is two kernels)
    dom_bytes, dom_us = c_r + c_w, avg["combine"]
    ach = dom_bytes / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": load_traffic("combine_expert_bf16"),
                "kernel": "combine (per-expert bf16)", "algorithmic_bytes": dom_bytes,
                "avg_us": round(dom_us, 2)}

    result = {
        "metric": "dispatch & combine HBM GB/s (and % peak) at 4096 tok×7168 bf16 top-8, 1 GPU",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_med, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {T} tokens x {H} hidden bf16, {E} experts in {G} groups, "
                               f"top-{K} {wl.routing} routing, per-expert receive buffers",
                   "tokens": T, "hidden": H, "experts": E, "groups": G, "topk": K,
                   "routing": wl.routing, "receive_layout": "expert", "seed": wl.seed},
        "roofline": roofline,
        "step": "moe_layout_dispatch + moe_combine (per-expert layout)",
        "step_status_or": step_status,
        "kernels_us": {k: {kk: round(vv, 2) for kk, vv in stats(v).items()} for k, v in us.items()},
        "event_steps": len(sampled),
        "kernels_gbs": {
            "layout_dispatch": round((b_layout + d_r + d_w) / (avg["layout_dispatch"] * 1e-6) / 1e9, 1),
            "combine": round((c_r + c_w) / (avg["combine"] * 1e-6) / 1e9, 1),
            "combine_payload_gbs": round(R * H * 2 / (avg["combine"] * 1e-6) / 1e9, 1),
        },
        "bytes": {"layout": b_layout, "dispatch": d_r + d_w, "combine": c_r + c_w, "rows": R,
                  "group_rows": P},
        "source_hash": source_hash(),
        "gpu_memory_in_use_at_start": used_before,
    }
    if procs is not None:
        result["processes"] = procs

    nthreads = len(os.sched_getaffinity(0))
    table = None
    if not args.no_extras:
        result["extra"] = extras(moe, d, dv, args)
        table = workload_table(moe, oracle_threads=0 if args.no_cpu_baseline else nthreads)
        result["extra"]["workloads"] = table
        add_ceilings(result["extra"])
        result["parity"] = {n: r["parity"]["ok"] for n, r in table.items() if isinstance(r, dict)
                            and "parity" in r}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, nthreads, table)
    print(json.dumps(result), flush=True)


def other_processes(args, value, ms):
    """The timed step repeated in args.processes - 1 child processes (started one after
    another, each a fresh `python bench.py --no-extras --no-cpu-baseline --processes 1`),
    with this process's value: each value and ms per step, and their medians."""
    import subprocess
    import numpy as np
    vals, mss = [round(value, 1)], [ms]
    for _ in range(args.processes - 1):
        cmd = [sys.executable, os.path.abspath(__file__), "--steps", str(args.steps), "--warmup",
               str(args.warmup), "--workload", args.workload, "--no-extras", "--no-cpu-baseline",
               "--processes", "1"]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"child bench failed ({r.returncode}): {r.stderr[-2000:]}")
        line = json.loads(r.stdout.strip().splitlines()[-1])
        vals.append(line["value"])
        mss.append(line["ms_per_step"])
    return {"values": vals, "ms_per_step": [round(m, 4) for m in mss], "this_process": round(value, 1),
            "median": round(float(np.median(vals)), 1), "median_ms_per_step": float(np.median(mss))}


def cpu_baseline(d, nthreads, table):
    """The oracle (C, as it stands) on the headline workload: one layout, one per-expert
    dispatch and one combine per build, per call (the t4096 row of the workload table
    when it was made, else measured here), for the OpenMP build on every core (`value`)
    and the single-thread canonical build; the two builds' outputs are bit-identical."""
    wl = d["workload"]
    if table is not None and wl.name in table and "oracle" in table[wl.name]:
        orc = table[wl.name]["oracle"]
    else:
        orc, _ = oracle_leg(d, nthreads)
    n = orc["threads"]
    calls = ("layout", "dispatch_expert", "combine_expert")
    nbytes = sum(orc["bytes"][c] for c in calls)
    t_n = sum(orc["us"]["openmp"][c] for c in calls)
    t_1 = sum(orc["us"]["serial"][c] for c in calls)
    return {
        "value": round(nbytes / t_n / 1e3, 3), "unit": "GB/s", "cores": n, "kind": "oracle",
        "sample": (f"the {wl.name} workload once per call (layout, per-expert dispatch, combine) "
                   f"by the OpenMP build of the C oracle on {n} threads, its outputs preallocated; "
                   f"{t_n / 1e3:.0f} ms of calls (the single-thread build: {t_1 / 1e3:.0f} ms)"),
        "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0)),
        "ms_per_step": round(t_n / 1e3, 2),
        "per_call_ms": {c: round(orc["us"]["openmp"][c] / 1e3, 3) for c in calls},
        "builds_identical": orc["builds_identical"],
        "single_thread": {"value": round(nbytes / t_1 / 1e3, 3), "unit": "GB/s", "cores": 1,
                          "ms_per_step": round(t_1 / 1e3, 2),
                          "per_call_ms": {c: round(orc["us"]["serial"][c] / 1e3, 3) for c in calls}},
    }


def extras(moe, d, dv, args):
    """Secondary measurements (not part of `value`): the step as three calls, the GROUP
    layout, FP8 dispatch on the FP8 workload, flushed-cache timings, the read/write-mix
    ceilings of the dispatch and the combine, and a plain copy."""
    import numpy as np
    import torch
    import synth_inputs as si
    wl = dv.wl
    T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    it = 50     # timed calls per measurement (median, p10/p90 over these)
    res = {}
    L = dv.L
    moe.moe_layout(dv.idx, E, G, out=L)
    P = int(L.group_offset[G].item())
    R = int(L.expert_offset[E].item())

    # the same step as three separate calls (layout, dispatch, combine)
    De = dv.D["expert"]
    lay = lambda: moe.moe_layout(dv.idx, E, G, out=L)
    disp = lambda: moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "expert", "bf16", out=De)
    comb = lambda: moe.moe_combine(L, De.recv_x, dv.w, "expert", out=dv.out)
    lay(); disp(); comb()
    t3 = time_calls([lay, disp, comb], it)
    bl = layout_bytes(T, K, E, G, P)
    bd3, bc3 = sum(dispatch_bytes(T, H, K, G, R, "expert")), sum(combine_bytes(T, H, K, R))
    step3 = [a + b + c for a, b, c in zip(*t3)]
    m3 = [stats(v)["median"] for v in t3]
    res["three_call_step"] = {
        "layout_us": m3[0], "dispatch_us": m3[1], "combine_us": m3[2],
        "step_us": stats(step3)["median"],
        "step_gbs": round((bl + bd3 + bc3) / stats(step3)["median"] / 1e3, 1),
        "dispatch_gbs": round(bd3 / m3[1] / 1e3, 1), "combine_gbs": round(bc3 / m3[2] / 1e3, 1),
        "dispatch_frac": round(bd3 / m3[1] / 1e3 / PEAK_HBM_GBS, 4),
        "combine_frac": round(bc3 / m3[2] / 1e3 / PEAK_HBM_GBS, 4),
        "dispatch_payload_gbs": round(R * H * 2 / m3[1] / 1e3, 1),
        "combine_payload_gbs": round(R * H * 2 / m3[2] / 1e3, 1)}
    Dg = moe.alloc_dispatch(L, H, "group")
    disp_g = lambda: moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "group", "bf16", out=Dg)
    comb_g = lambda: moe.moe_combine(L, Dg.recv_x, dv.w, "group", out=dv.out)
    disp_g(); comb_g()
    tg = time_calls([disp_g, comb_g], it)
    bd, bc = sum(dispatch_bytes(T, H, K, G, P, "group")), sum(combine_bytes(T, H, K, P))
    res["group"] = {"rows": P, "dispatch_us": stats(tg[0])["median"], "combine_us": stats(tg[1])["median"],
                    "dispatch_gbs": round(bd / stats(tg[0])["median"] / 1e3, 1),
                    "combine_gbs": round(bc / stats(tg[1])["median"] / 1e3, 1)}
    del Dg

    De = dv.D["expert"]
    disp_e = lambda: moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "expert", "bf16", out=De)
    comb_e = lambda: moe.moe_combine(L, De.recv_x, dv.w, "expert", out=dv.out)
    bde, bce = sum(dispatch_bytes(T, H, K, G, R, "expert")), sum(combine_bytes(T, H, K, R))
    # each kernel repeated on its own (no other kernel's write-back in between)
    td = time_calls([disp_e], it)
    tcb = time_calls([comb_e], it)
    res["expert_alone"] = {"dispatch_us": stats(td[0])["median"], "combine_us": stats(tcb[0])["median"],
                           "dispatch_gbs": round(bde / stats(td[0])["median"] / 1e3, 1),
                           "combine_gbs": round(bce / stats(tcb[0])["median"] / 1e3, 1)}

    # cold-cache timing of the per-expert kernels: 1 GiB is read before every call
    # (outside the timed events), so the 256 MB last-level cache holds only clean,
    # unrelated lines when the kernel starts
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush = lambda: scratch.sum()
    tc = time_calls([disp_e, comb_e], 15, flush=flush)
    res["expert_flushed"] = {"dispatch_us": stats(tc[0])["median"], "combine_us": stats(tc[1])["median"],
                             "dispatch_gbs": round(bde / stats(tc[0])["median"] / 1e3, 1),
                             "combine_gbs": round(bce / stats(tc[1])["median"] / 1e3, 1)}

    # Read/write-mix ceilings: the dispatch's mix (one 14 KiB row read, K written) and
    # the combine's (K read, one written) over contiguous rows of the same size and
    # count, with the kernels' cache policy; back to back as in the step (the first
    # reads a buffer that nothing wrote recently, as the dispatch reads x, and writes the
    # rows the second reads; the second writes a third buffer), and alone.
    row = H * 2
    xs = torch.full((T * row,), 3, dtype=torch.uint8, device="cuda")
    a = torch.full((R * row,), 1, dtype=torch.uint8, device="cuda")
    b = torch.full((T * row,), 2, dtype=torch.uint8, device="cuda")
    mix_d = lambda: moe.moe_ref_mix(a, xs, row, 1, K)
    mix_c = lambda: moe.moe_ref_mix(b, a, row, K, 1)
    mix_d(); mix_c()
    tp = time_calls([mix_d, mix_c], it)
    tda, tca = time_calls([mix_d], it)[0], time_calls([mix_c], it)[0]
    mb_d, mb_c = (R + T) * row, (R + T) * row
    md, mc = stats(tp[0])["median"], stats(tp[1])["median"]
    res["mix_ceiling"] = {
        "bytes": mb_d, "row_bytes": row, "rows_read_per_write": {"dispatch": 1 / K, "combine": K},
        "pair": {"dispatch_us": md, "combine_us": mc, "dispatch_gbs": round(mb_d / md / 1e3, 1),
                 "combine_gbs": round(mb_c / mc / 1e3, 1),
                 "step_gbs": round((mb_d + mb_c) / stats([x + y for x, y in zip(*tp)])["median"] / 1e3, 1)},
        "alone": {"dispatch_us": stats(tda)["median"], "combine_us": stats(tca)["median"],
                  "dispatch_gbs": round(mb_d / stats(tda)["median"] / 1e3, 1),
                  "combine_gbs": round(mb_c / stats(tca)["median"] / 1e3, 1)}}
    del a, b, xs

    # plain copy ceiling: 2 x 512 MiB streaming copy (half reads, half writes)
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    cp = lambda: moe.moe_ref_copy(dst, src)
    cp()
    tcp = time_calls([cp], 20)
    res["copy_ceiling"] = {"bytes": 2 * n, "us": stats(tcp[0])["median"],
                           "gbs": round(2 * n / stats(tcp[0])["median"] / 1e3, 1)}
    del src, dst, scratch

    # FP8 dispatch on the FP8 workload (same shape, its own seed), both layouts
    d8 = si.make_workload("fp8")
    w8 = d8["workload"]
    dv8 = Dev(moe, d8, modes=("expert", "group"), dtype="fp8")
    moe.moe_layout(dv8.idx, w8.E, w8.G, out=dv8.L)
    R8 = int(dv8.L.expert_offset[w8.E].item())
    P8 = int(dv8.L.group_offset[w8.G].item())
    f8 = {}
    for mode, rows in (("expert", R8), ("group", P8)):
        D8 = dv8.D[mode]
        fn = lambda: moe.moe_dispatch(dv8.L, dv8.x, dv8.w, dv8.idx, mode, "fp8", out=D8)
        fn()
        t8 = time_calls([fn], it)
        b8 = sum(dispatch_bytes(w8.T, w8.H, w8.K, w8.G, rows, mode, fp8=True))
        f8[mode] = {"rows": rows, "dispatch_us": stats(t8[0])["median"],
                    "dispatch_gbs": round(b8 / stats(t8[0])["median"] / 1e3, 1)}
    res["fp8_dispatch"] = f8

    # the same step with layout + dispatch as one call (moe_layout_dispatch)
    fs = {}
    for mode in ("expert", "group"):
        Dm = dv.D["expert"] if mode == "expert" else moe.alloc_dispatch(L, H, "group")
        ld = lambda: moe.moe_layout_dispatch(dv.idx, E, G, dv.x, dv.w, mode, "bf16", out_layout=L, out=Dm)
        cb = lambda: moe.moe_combine(L, Dm.recv_x, dv.w, mode, out=dv.out)
        ld(); cb()
        tf = time_calls([ld, cb], it)
        rows = R if mode == "expert" else P
        nb = (layout_bytes(T, K, E, G, P) + sum(dispatch_bytes(T, H, K, G, rows, mode))
              + sum(combine_bytes(T, H, K, rows)))
        step = [a + b for a, b in zip(tf[0], tf[1])]
        fs[mode] = {"layout_dispatch_us": stats(tf[0])["median"], "combine_us": stats(tf[1])["median"],
                    "step_us": stats(step)["median"], "step_gbs": round(nb / stats(step)["median"] / 1e3, 1)}
    res["fused_step"] = fs
    del dv8
    torch.cuda.synchronize()

    t3 = res["three_call_step"]
    mx = res["mix_ceiling"]["pair"]
    res["of_copy_ceiling"] = {
        # each call against the reference with its own read/write mix, run back to back
        "dispatch_vs_mix": round(t3["dispatch_gbs"] / mx["dispatch_gbs"], 3),
        "combine_vs_mix": round(t3["combine_gbs"] / mx["combine_gbs"], 3),
        "fused_step_vs_mix": round(res["fused_step"]["expert"]["step_gbs"] / mx["step_gbs"], 3),
        # and against the plain half-read, half-write copy
        "fused_step_vs_copy": round(res["fused_step"]["expert"]["step_gbs"] / res["copy_ceiling"]["gbs"], 3)}
    props = torch.cuda.get_device_properties(0)
    res["env"] = {"device": torch.cuda.get_device_name(0),
                  "arch": getattr(props, "gcnArchName", None),
                  "compute_units": props.multi_processor_count,
                  "hbm_gib": round(props.total_memory / 2**30, 1),
                  **device_clocks(),
                  "hip": torch.version.hip, "torch": torch.__version__,
                  "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    return res


def add_ceilings(extra):
    """Each workload report row's share of the measured ceiling of the same run: the
    read/write-mix reference of its call (the dispatch's or the combine's mix); none for
    the latency-bound layout."""
    mix = extra["mix_ceiling"]["pair"]
    for name, r in extra["workloads"].items():
        if not isinstance(r, dict):
            continue
        for row in r.get("report", []):
            if row["call"] == "layout":      # latency-bound: no bandwidth ceiling applies
                row["of_ceiling"] = None
                continue
            ref = mix["dispatch_gbs"] if row["call"] == "dispatch" else mix["combine_gbs"]
            row["of_ceiling"] = round(row["gbs"] / ref, 3)


def device_clocks():
    """Peak engine and memory clocks (MHz) and memory bus width (bits) of device 0, from
    the HIP runtime (hipDeviceGetAttribute; attribute numbers of hip_runtime_api.h:
    ClockRate 5, MemoryClockRate 60, MemoryBusWidth 59); None where unavailable."""
    import ctypes
    out = {"engine_clock_mhz": None, "memory_clock_mhz": None, "memory_bus_bits": None}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return out
    for key, attr, scale in (("engine_clock_mhz", 5, 1000), ("memory_clock_mhz", 60, 1000),
                             ("memory_bus_bits", 59, 1)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0:
            out[key] = v.value // scale
    return out


def _layout_host(L):
    return {n: host_bits(getattr(L, n)) for n in (
        "expert_count", "expert_offset", "group_count", "group_offset", "tok_group_mask", "slot_e",
        "slot_g", "slot_tg", "recv_src_e", "recv_src_g", "status")}


def workload_table(moe, names=WORKLOAD_NAMES, it=50, oracle_threads=0):
    """Per-workload timings of every call in both receive layouts (median µs over `it`
    event-timed calls; GB/s = algorithmic bytes / median; for the layout, and for the
    dispatch and combine of batches of at most 256 tokens, also the µs per call in a
    stream of back-to-back calls, `*_us_stream`, since a pair of events around one
    short call adds a fixed cost of its own), the per-expert step
    replayed from a captured HIP graph (no host launch cost), and, with
    oracle_threads > 0, both oracle builds timed per call on the same inputs and the
    GPU's outputs of every call checked against the oracle's (`parity`). Each workload
    also gets `report`: one row per (layout, call) with the survey's columns."""
    import numpy as np
    import torch
    import synth_inputs as si
    out = {}
    for name in names:
        d = si.make_workload(name)
        wl = d["workload"]
        T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
        dt = "fp8" if wl.fp8 else "bf16"
        dv = Dev(moe, d, modes=("expert", "group"), dtype=dt)
        L = dv.L
        lay = lambda: moe.moe_layout(dv.idx, E, G, out=L)
        lay()
        torch.cuda.synchronize()
        R, P = int(L.expert_offset[E].item()), int(L.group_offset[G].item())
        t_lay = time_calls([lay], it)[0]
        row = {"T": T, "H": H, "E": E, "G": G, "K": K, "routing": wl.routing, "dtype": dt,
               "layout_us": round(stats(t_lay)["median"], 2),
               "layout_us_stream": round(min(time_stream(lay) for _ in range(3)), 2)}
        gpu = {"L": _layout_host(L)}
        cstats = {"layout": (stats(t_lay), layout_bytes(T, K, E, G, P))}
        for mode, nrows in (("expert", R), ("group", P)):
            D = dv.D[mode]
            disp = lambda: moe.moe_dispatch(L, dv.x, dv.w, dv.idx, mode, dt, out=D)
            disp()
            y = moe.moe_fp8_dequant(L, D.recv_x, D.recv_scale, mode) if wl.fp8 else D.recv_x
            comb = lambda: moe.moe_combine(L, y, dv.w, mode, out=dv.out)
            comb()
            td, tc = time_calls([disp, comb], it)
            bd = sum(dispatch_bytes(T, H, K, G, nrows, mode, fp8=wl.fp8))
            bc = sum(combine_bytes(T, H, K, nrows))
            md, mc = stats(td)["median"], stats(tc)["median"]
            cstats[f"dispatch_{mode}"] = (stats(td), bd)
            cstats[f"combine_{mode}"] = (stats(tc), bc)
            row[mode] = {"rows": nrows, "dispatch_us": round(md, 2), "combine_us": round(mc, 2),
                         "dispatch_gbs": round(bd / md / 1e3, 1), "combine_gbs": round(bc / mc / 1e3, 1),
                         "dispatch_frac": round(bd / md / 1e3 / PEAK_HBM_GBS, 4),
                         "combine_frac": round(bc / mc / 1e3 / PEAK_HBM_GBS, 4),
                         "dispatch_payload_gbs": round(nrows * H * (1 if wl.fp8 else 2) / md / 1e3, 1),
                         "combine_payload_gbs": round(nrows * H * 2 / mc / 1e3, 1)}
            if T <= 256:   # launch-bound calls: also what each costs in a stream of calls
                row[mode]["dispatch_us_stream"] = round(min(time_stream(disp) for _ in range(3)), 2)
                row[mode]["combine_us_stream"] = round(min(time_stream(comb) for _ in range(3)), 2)
            if oracle_threads:
                torch.cuda.synchronize()
                g = {"out": host_bits(dv.out)}
                if wl.fp8:
                    g.update(recv_q=host_bits(D.recv_x[:nrows]), recv_scale=host_bits(D.recv_scale[:nrows]),
                             y=host_bits(y[:nrows]))
                else:
                    g["recv_x"] = host_bits(D.recv_x[:nrows])
                g.update(recv_w=host_bits(D.recv_topk_w[:nrows]), recv_idx=host_bits(D.recv_topk_idx[:nrows]))
                gpu[mode] = g
        # receive-side regroup: the per-group arrays -> the per-expert layout
        Dg, De = dv.D["group"], dv.D["expert"]
        moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "group", dt, out=Dg)
        rg = lambda: moe.moe_regroup(L, Dg, out=De)
        rg()
        mr = stats(time_calls([rg], it)[0])["median"]
        row_b = H if wl.fp8 else 2 * H
        meta = K * 8 + ((H // 128) * 4 if wl.fp8 else 0)
        br = P * (row_b + meta) + T * (G + 2 * K) * 4 + R * (row_b + meta)
        row["regroup"] = {"us": round(mr, 2), "gbs": round(br / mr / 1e3, 1),
                          "frac": round(br / mr / 1e3 / PEAK_HBM_GBS, 4)}
        # per-expert FP8 cast + padded transpose of the per-expert rows (bf16 workloads)
        if not wl.fp8 and H % 64 == 0:
            moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "expert", dt, out=De)
            sc = torch.full((E,), 64.0, dtype=torch.float32, device="cuda")
            am = torch.zeros(E, dtype=torch.float32, device="cuda")
            CT = moe.moe_cast_transpose_fp8(L, De.recv_x, sc, amax=am)
            ctf = lambda: moe.moe_cast_transpose_fp8(L, De.recv_x, sc, out=CT)
            torch.cuda.synchronize()
            mct = stats(time_calls([ctf], it)[0])["median"]
            npad = int(CT.pad_offset[E].item())
            bct = R * H * 2 + R * H + npad * H + (E + 1) * 4 * 2 + E * 8
            row["cast_transpose"] = {"us": round(mct, 2), "gbs": round(bct / mct / 1e3, 1),
                                     "frac": round(bct / mct / 1e3 / PEAK_HBM_GBS, 4)}
            del CT
        # HIP-graph replay of the per-expert step
        De = dv.D["expert"]
        ye = De.recv_x if not wl.fp8 else None
        if not wl.fp8:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(2):
                    lay(); moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "expert", dt, out=De)
                    moe.moe_combine(L, ye, dv.w, "expert", out=dv.out)
            torch.cuda.current_stream().wait_stream(s)
            with torch.cuda.graph(g):
                lay()
                moe.moe_dispatch(L, dv.x, dv.w, dv.idx, "expert", dt, out=De)
                moe.moe_combine(L, ye, dv.w, "expert", out=dv.out)
            g.replay()
            torch.cuda.synchronize()
            row["graph_step_us"] = round(stats(time_calls([g.replay], it)[0])["median"], 2)
            del g
            # layout + dispatch as one call (one launch for the smallest batches)
            fused = lambda: moe.moe_layout_dispatch(dv.idx, E, G, dv.x, dv.w, "expert", dt,
                                                    out_layout=L, out=De)
            fused()
            row["fused_layout_dispatch_us"] = round(stats(time_calls([fused], it)[0])["median"], 2)
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(2):
                    fused(); moe.moe_combine(L, ye, dv.w, "expert", out=dv.out)
            torch.cuda.current_stream().wait_stream(s)
            with torch.cuda.graph(g):
                fused()
                moe.moe_combine(L, ye, dv.w, "expert", out=dv.out)
            g.replay()
            torch.cuda.synchronize()
            row["graph_step_fused_us"] = round(stats(time_calls([g.replay], it)[0])["median"], 2)
            del g
        del dv, D, De, Dg
        torch.cuda.synchronize()
        orc = None
        if oracle_threads:
            orc, ora = oracle_leg(d, oracle_threads)
            row["oracle"] = orc
            row["parity"] = parity_of(gpu, ora, wl.fp8)
            del ora, gpu
        # report rows: workload | layout | dtype | call | GPU µs (median, p10-p90) | GB/s |
        # share of 8 TB/s | share of the call's ceiling | payload GB/s | oracle µs | parity
        rep = []
        for key, (st, nb) in cstats.items():
            call, _, mode = key.partition("_")
            rows_here = R if mode == "expert" else P
            r = {"workload": name, "receive_layout": mode or "both", "dtype": dt if call == "dispatch" else "bf16",
                 "call": call, "us_median": round(st["median"], 2),
                 "us_p10_p90": [round(st["p10"], 2), round(st["p90"], 2)],
                 "gbs": round(nb / st["median"] / 1e3, 1),
                 "of_peak": round(nb / st["median"] / 1e3 / PEAK_HBM_GBS, 4),
                 "payload_gbs": (round(rows_here * H * (1 if wl.fp8 and call == "dispatch" else 2)
                                       / st["median"] / 1e3, 1) if call != "layout" else None)}
            # HBM traffic per launch from the committed counters (None unless they were
            # taken on this kernel's current sources), and its ratio to the algorithmic bytes
            if call != "layout":
                tk = f"{name}.{call}_{mode}_{'fp8' if wl.fp8 and call == 'dispatch' else 'bf16'}"
                tb = load_traffic(tk)
                r["traffic_bytes"] = tb
                r["traffic_over_algorithmic"] = None if tb is None else round(tb / nb, 4)
            if orc is not None:
                n = orc["threads"]
                r["oracle_us"] = {"1": orc["calls"][key]["us_1"], str(n): orc["calls"][key][f"us_{n}"]}
                r["parity"] = row["parity"].get(key, row["parity"]["layout"])
            rep.append(r)
        row["report"] = rep
        out[name] = row
    steps = [v["layout_us"] + v["expert"]["dispatch_us"] + v["expert"]["combine_us"] for v in out.values()]
    out["geomean_step_us_expert"] = round(float(np.exp(np.mean(np.log(steps)))), 2)
    return out


if __name__ == "__main__":
    main()
