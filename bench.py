"""Benchmark of the MoE token path on one MI355X: layout -> dispatch -> combine.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t4096]

One step = one pass of the hot path over one batch of synthetic input already
resident in HBM: the routing layout (per-expert and per-group) and the dispatch
of bf16 rows into per-expert receive buffers, as one moe_layout_dispatch call
(for this batch: the layout's count kernel, one offsets workgroup, and a
dispatch whose workgroups place their own tokens), then moe_combine (fp32
weighted top-k sum back to bf16; the experts are identities, so combine reads
the dispatched rows in place). Default workload: 4096 tokens x 7168 hidden
bf16, 256 experts in 8 groups, top-8 uniform routing.

Prints ONE JSON line. `value` = algorithmic HBM bytes of a step (reads + writes,
each byte counted once) / wall time per step. Per-call times come from HIP
events recorded around every call of every 4th step of the timed region, on
the stream the kernels run on. The same line carries the roofline of the dominant kernel, the
CPU oracle timed on host cores (a bounded sample of the same workload), and
secondary measurements (the same step as three calls moe_layout, moe_dispatch,
moe_combine with per-call rates, the deduplicated per-group layout, FP8
dispatch on the FP8 workload, a plain copy ceiling, each kernel repeated alone,
cold-cache timings, every call on every workload).
"""
from __future__ import annotations

import argparse
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
    "layout": ("layout.hip", "common.hpp", "kernels.hpp"),
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


def load_traffic(kernel: str, key: str):
    """HBM traffic (bytes per launch) of a kernel from the committed rocprofv3 --pmc
    counters, if they were taken on that kernel's current sources; None otherwise."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        k = json.load(open(p)).get("kernels", {}).get(key)
    except ValueError:
        return None
    if not k or k.get("source_hash") != source_hash(kernel):
        return None
    return k.get("traffic_bytes")


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


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(d, budget_s=12.0):
    """The oracle (single-threaded C, as it stands) on the same workload: whole steps
    (layout + EXPERT dispatch + combine) repeated until the time budget is spent."""
    import oracle
    wl = d["workload"]
    T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    steps, t_layout, t_disp, t_comb, nbytes = 0, 0.0, 0.0, 0.0, 0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        Lo = oracle.layout(d["topk_idx"], E, G)
        t1 = time.perf_counter()
        Do = oracle.dispatch_bf16(Lo, "expert", d["x"], d["topk_w"], d["topk_idx"])
        t2 = time.perf_counter()
        oracle.combine(Lo, "expert", Do["recv_x"], d["topk_w"])
        t3 = time.perf_counter()
        steps += 1
        t_layout += t1 - t0
        t_disp += t2 - t1
        t_comb += t3 - t2
        R = Lo["R_expert"]
        nbytes += (layout_bytes(T, K, E, G, Lo["R_group"]) + sum(dispatch_bytes(T, H, K, G, R, "expert"))
                   + sum(combine_bytes(T, H, K, R)))
        del Do
        if time.perf_counter() - t_start > budget_s or steps >= 50:
            break
    total = t_layout + t_disp + t_comb
    return {
        "value": nbytes / total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{steps} whole step(s) of the {wl.name} workload (layout + per-expert "
                   f"dispatch + combine) by the single-threaded C oracle, {total:.1f} s"),
        "ms_per_step": total / steps * 1e3,
        "ms_layout": t_layout / steps * 1e3, "ms_dispatch": t_disp / steps * 1e3,
        "ms_combine": t_comb / steps * 1e3,
        "host_cores_available": len(os.sched_getaffinity(0)),
    }


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="t4096")
    ap.add_argument("--no-extras", action="store_true", help="only the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the plain reference copy (256 MiB, 5 times): a known byte "
                         "count for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--processes", type=int, default=3,
                    help="also time the step in this many separate processes in all (this one "
                         "included; run one after another) and report each value and their median "
                         "in extra.processes; `value` stays this process's")
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
    if args.table:
        print(json.dumps({"workloads": workload_table(moe, names=tuple(args.table.split(",")))}))
        return
    d = si.make_workload(args.workload)
    wl = d["workload"]
    T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    dv = Dev(moe, d, modes=("expert",))
    L, D, out = dv.L, dv.D["expert"], dv.out

    # one step: routing layout + dispatch as one call (the library's form for this
    # batch: the count kernel, one offsets workgroup, and a dispatch that places its
    # own tokens), then the combine; the three separate calls are timed in extras
    fns = [
        lambda: moe.moe_layout_dispatch(dv.idx, E, G, dv.x, dv.w, "expert", "bf16", out_layout=L, out=D),
        lambda: moe.moe_combine(L, D.recv_x, dv.w, "expert", out=out),
    ]
    for _ in range(args.warmup):
        for f in fns:
            f()
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
        if e:
            e[0].record()
        fns[0]()
        if e:
            e[1].record()
        fns[1]()
        if e:
            e[2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / args.steps * 1e3
    us = {name: [ev[s][i].elapsed_time(ev[s][i + 1]) * 1e3 for s in sampled]
          for i, name in enumerate(("layout_dispatch", "combine"))}

    assert int(L.status.item()) == 0
    R = int(L.expert_offset[E].item())
    P = int(L.group_offset[G].item())
    b_layout = layout_bytes(T, K, E, G, P)
    d_r, d_w = dispatch_bytes(T, H, K, G, R, "expert")
    c_r, c_w = combine_bytes(T, H, K, R)
    step_bytes = b_layout + d_r + d_w + c_r + c_w
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    avg = {k: float(np.mean(v)) for k, v in us.items()}
    # the dominant kernel: combine (the layout + dispatch call is several kernels)
    kern = {"combine": (c_r + c_w, avg["combine"])}
    dom = "combine"
    ach = kern[dom][0] / (kern[dom][1] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": load_traffic(dom, f"{dom}_expert_bf16"),
                "kernel": f"{dom} (per-expert bf16)", "algorithmic_bytes": kern[dom][0],
                "avg_us": round(kern[dom][1], 2)}

    result = {
        "metric": "dispatch & combine HBM GB/s (and % peak) at 4096 tok×7168 bf16 top-8, 1 GPU",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {T} tokens x {H} hidden bf16, {E} experts in {G} groups, "
                               f"top-{K} {wl.routing} routing, per-expert receive buffers",
                   "tokens": T, "hidden": H, "experts": E, "groups": G, "topk": K,
                   "routing": wl.routing, "receive_layout": "expert", "seed": wl.seed},
        "roofline": roofline,
        "step": "moe_layout_dispatch + moe_combine (per-expert layout)",
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
    }

    if not args.no_extras:
        result["extra"] = extras(moe, d, dv, args)
        if args.processes > 1:
            result["extra"]["processes"] = other_processes(args, value)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, args.cpu_budget)
    print(json.dumps(result), flush=True)


def other_processes(args, value):
    """The timed step repeated in args.processes - 1 child processes (started one after
    another, each a fresh `python bench.py --no-extras --no-cpu-baseline`), with this
    process's value: each value, and their median."""
    import subprocess
    import numpy as np
    vals = [round(value, 1)]
    for _ in range(args.processes - 1):
        cmd = [sys.executable, os.path.abspath(__file__), "--steps", str(args.steps), "--warmup",
               str(args.warmup), "--workload", args.workload, "--no-extras", "--no-cpu-baseline"]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"child bench failed ({r.returncode}): {r.stderr[-2000:]}")
        vals.append(json.loads(r.stdout.strip().splitlines()[-1])["value"])
    return {"values": vals, "median": round(float(np.median(vals)), 1)}


def extras(moe, d, dv, args):
    """Secondary measurements (not part of `value`): GROUP layout, FP8 dispatch on
    the FP8 workload, flushed-cache timings, and a plain copy ceiling."""
    import numpy as np
    import torch
    import synth_inputs as si
    wl = dv.wl
    T, H, E, G, K = wl.T, wl.H, wl.E, wl.G, wl.K
    it = 30
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

    # plain copy ceiling: 2 x 512 MiB streaming copy
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

    # the same step with layout + dispatch as one call (moe_layout_dispatch: the count
    # kernel, one offsets workgroup, and a dispatch that places its own tokens)
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
    res["workloads"] = workload_table(moe)

    # rates against the plain copy of the same run (mixed read/write traffic's achievable rate)
    cg = res["copy_ceiling"]["gbs"]
    t3 = res["three_call_step"]
    res["of_copy_ceiling"] = {"dispatch": round(t3["dispatch_gbs"] / cg, 3),
                              "combine": round(t3["combine_gbs"] / cg, 3),
                              "fused_step": round(res["fused_step"]["expert"]["step_gbs"] / cg, 3)}
    props = torch.cuda.get_device_properties(0)
    res["env"] = {"device": torch.cuda.get_device_name(0),
                  "arch": getattr(props, "gcnArchName", None),
                  "compute_units": props.multi_processor_count,
                  "hbm_gib": round(props.total_memory / 2**30, 1),
                  **device_clocks(),
                  "hip": torch.version.hip, "torch": torch.__version__,
                  "host_cores_available": len(os.sched_getaffinity(0))}
    return res


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


def workload_table(moe, names=("tiny", "t256", "t4096", "skew", "fp8"), it=30):
    """Per-workload timings of every call in both receive layouts (median µs over `it`
    event-timed calls; GB/s = algorithmic bytes / median), plus, for each workload, the
    per-expert step (layout + dispatch + combine) replayed from a captured HIP graph,
    which removes the host's launch cost from small workloads."""
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
        row = {"T": T, "H": H, "E": E, "G": G, "K": K, "routing": wl.routing, "dtype": dt,
               "layout_us": round(stats(time_calls([lay], it)[0])["median"], 2)}
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
            row[mode] = {"rows": nrows, "dispatch_us": round(md, 2), "combine_us": round(mc, 2),
                         "dispatch_gbs": round(bd / md / 1e3, 1), "combine_gbs": round(bc / mc / 1e3, 1),
                         "dispatch_frac": round(bd / md / 1e3 / PEAK_HBM_GBS, 4),
                         "combine_frac": round(bc / mc / 1e3 / PEAK_HBM_GBS, 4),
                         "dispatch_payload_gbs": round(nrows * H * (1 if wl.fp8 else 2) / md / 1e3, 1),
                         "combine_payload_gbs": round(nrows * H * 2 / mc / 1e3, 1)}
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
            if True:
                # layout + dispatch as one call (one launch for T <= 512)
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
        out[name] = row
        del dv, D, De
        torch.cuda.synchronize()
    steps = [v["layout_us"] + v["expert"]["dispatch_us"] + v["expert"]["combine_us"] for v in out.values()]
    out["geomean_step_us_expert"] = round(float(np.exp(np.mean(np.log(steps)))), 2)
    return out


if __name__ == "__main__":
    main()
