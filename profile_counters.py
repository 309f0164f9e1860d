"""rocprofv3 kernel traces and HBM counters of the library's kernels -> profiles/.

    python3 profile_counters.py OUTDIR [--only NAMES]     (on a GPU machine)
    python3 profile_counters.py OUTDIR --from-raw          (anywhere: re-read OUTDIR)

From the repository root. Runs rocprofv3 over bench.py targets, each pass a process
of its own (rocprofv3 does not split counters over passes): a kernel trace
(durations), FETCH_SIZE, WRITE_SIZE and TCC_HIT_sum + TCC_MISS_sum, and for the step
and the mix references two passes of memory-side request and stall counters.
Targets (NAMES for --only, comma-separated):

  copy    bench.py --calibrate-copy: the plain 256 MiB reference copy, whose known
          bytes scale the counters (FETCH_SIZE counts half of what a copy reads)
  step    bench.py --steps 20 --warmup 3 --no-extras --no-cpu-baseline --processes 1:
          the headline step (the layout's count kernel, the placing dispatch, combine)
  W:L     bench.py --profile W:L for W in t4096, skew, fp8 and L in expert, group:
          moe_layout, moe_dispatch, (FP8) moe_fp8_dequant and moe_combine, 5 times each
  mix     bench.py --mix-probes: the read/write-mix references of the dispatch and combine
  table   bench.py --table t4096: the regroup and the cast-transpose among every call
  tables  bench.py --table tiny,t256,t4096,skew,fp8: every call on every workload
          (kernel trace only)

Each kernel instance gets the median over its launches of the bytes per launch
(counter KiB x 1024 x the copy's ratio of known to counted bytes), their ratio to
the algorithmic bytes where bench.py defines them, the L2 hit rate, the average
duration from the trace, and the hash of its kernel's code (bench.py's
source_hash: comments and spacing aside) as it was when the passes ran. bench.py
reports `traffic` only while that hash matches the current sources. Writes
profiles/counters.json and markdown summaries into profiles/, and copies of them
into OUTDIR beside the raw rocprofv3 output; --from-raw rebuilds them from that
output alone (with the hashes stored beside it).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (no GPU use at import)
import synth_inputs as si  # noqa: E402

PASS_FLAGS = {
    "trace": ["--kernel-trace", "--stats"],
    "fetch": ["--pmc", "FETCH_SIZE"],
    "write": ["--pmc", "WRITE_SIZE"],
    "tcc": ["--pmc", "TCC_HIT_sum", "TCC_MISS_sum"],
    "wrreq": ["--pmc", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_STALL_sum",
              "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "GRBM_GUI_ACTIVE"],
    "rdreq": ["--pmc", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_BUSY_sum",
              "GRBM_GUI_ACTIVE"],
}
BASIC = ("trace", "fetch", "write", "tcc")
PROFILE_TARGETS = [f"{w}:{m}" for w in ("t4096", "skew", "fp8") for m in ("expert", "group")]
ALL_TARGETS = ["copy", "step", *PROFILE_TARGETS, "mix", "table", "tables"]
TABLES = "tiny,t256,t4096,skew,fp8"
REQUESTS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_STALL_sum",
            "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_BUSY_sum",
            "GRBM_GUI_ACTIVE")


def passes_of(name: str) -> tuple:
    if name in ("step", "mix"):
        return BASIC + ("wrreq", "rdreq")
    if name == "tables":
        return ("trace",)
    return BASIC


def target_args(name: str) -> list[str]:
    if name == "copy":
        return ["--calibrate-copy"]
    if name == "step":
        return ["--steps", "20", "--warmup", "3", "--no-extras", "--no-cpu-baseline", "--processes", "1"]
    if name == "mix":
        return ["--mix-probes"]
    if name == "table":
        return ["--table", "t4096"]
    if name == "tables":
        return ["--table", TABLES]
    return ["--profile", name]


def command(name: str, kind: str) -> str:
    """The rocprofv3 command of one pass, as run from the repository root."""
    return " ".join(["rocprofv3", *PASS_FLAGS[kind], "-f csv -d <out> -o k --", "python3 bench.py",
                     *target_args(name)])


def pass_dir(out: str, name: str, kind: str) -> str:
    return os.path.join(out, f"{name.replace(':', '_')}_{kind}")


def run_pass(out: str, name: str, kind: str) -> None:
    d = pass_dir(out, name, kind)
    cmd = ["timeout", "-s", "KILL", "300", "rocprofv3", *PASS_FLAGS[kind], "-f", "csv", "-d", d, "-o", "k", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *target_args(name)]
    env = dict(os.environ, TMPDIR="/tmp")
    t0 = time.time()
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(d + ".log", "w") as f:
        f.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    print(f"{name} {kind}: exit {r.returncode} in {time.time() - t0:.0f} s", flush=True)
    if r.returncode != 0:
        raise SystemExit(f"rocprofv3 failed for {name} {kind}; see {d}.log")


def per_dispatch(d: str) -> dict:
    """{kernel name: [{counter: value} per dispatch]} from a counter-collection run
    (summed over the counter's instances), or {kernel name: [{"ns": duration}]} from
    a trace."""
    out = collections.defaultdict(list)
    cc = os.path.join(d, "k_counter_collection.csv")
    if os.path.exists(cc):
        by = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(cc)):
            by[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for disp, vals in by.items():
            out[names[disp]].append(dict(vals))
        return out
    for r in csv.DictReader(open(os.path.join(d, "k_kernel_trace.csv"))):
        out[r["Kernel_Name"]].append({"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
    return out


def base_name(kernel_name: str) -> str:
    """A kernel's name with its template arguments, without namespaces and parameters."""
    n = kernel_name.replace("(anonymous namespace)::", "").split("(")[0]
    n = n[5:] if n.startswith("void ") else n
    return n.replace("moe::", "").replace("at::native::", "").strip()


def collect(out: str, name: str) -> dict:
    """{kernel: {"ns": [...], counter: [...]}} from the passes of one target."""
    res = collections.defaultdict(lambda: collections.defaultdict(list))
    for kind in passes_of(name):
        d = pass_dir(out, name, kind)
        if not os.path.isdir(d):   # (--from-raw over an output without this pass)
            continue
        for k, vals in per_dispatch(d).items():
            for v in vals:
                for q, x in v.items():
                    res[base_name(k)][q].append(x)
    return res


def pick(r: dict, prefix: str) -> dict:
    """The lists of every kernel whose name starts with prefix, merged."""
    out = collections.defaultdict(list)
    for k, v in r.items():
        if k.startswith(prefix):
            for q, vals in v.items():
                out[q] += vals
    if not out:
        raise SystemExit(f"no kernel {prefix} in {sorted(r)}")
    return out


def median_top(vals: list[float], n: int | None) -> float:
    """Median of the n largest values (a kernel name shared by calls of other sizes in
    one run, e.g. the table's, keeps its full-size launches), or of all."""
    v = sorted(vals)
    return statistics.median(v[-n:] if n else v)


def record(kernel: str, c: dict, scale: tuple, alg: tuple | None, hashes: dict, note: str | None = None,
           top=None) -> dict:
    fs, ws = scale
    fb = median_top(c["FETCH_SIZE"], top) * 1024 * fs
    wb = median_top(c["WRITE_SIZE"], top) * 1024 * ws
    r = {"kernel": kernel, "source_hash": hashes[kernel], "fetch_bytes": fb, "write_bytes": wb,
         "traffic_bytes": fb + wb, "avg_us": median_top(c["ns"], top) / 1e3 if c["ns"] else None}
    if c["TCC_HIT_sum"]:
        h, m = median_top(c["TCC_HIT_sum"], top), median_top(c["TCC_MISS_sum"], top)
        r["tcc_hit_rate"] = h / (h + m) if h + m else None
    for q in REQUESTS:
        if c.get(q):
            r.setdefault("requests", {})[q] = median_top(c[q], top)
    if alg:
        r.update(algorithmic_read=alg[0], algorithmic_write=alg[1], ratio=(fb + wb) / (alg[0] + alg[1]),
                 fetch_ratio=fb / alg[0], write_ratio=wb / alg[1])
    if note:
        r["note"] = note
    return r


def counts(wl) -> tuple:
    """(R, P, expert counts) of a synthetic workload (every entry valid)."""
    import numpy as np
    d = si.make_workload(wl.name)
    idx = d["topk_idx"]
    ne = np.bincount(idx.ravel(), minlength=wl.E)
    groups = idx // (wl.E // wl.G)
    P = sum(len(set(row)) for row in groups.tolist())
    return int(idx.size), int(P), ne


def bench_line(out: str, name: str) -> dict | None:
    """The JSON line bench.py printed in the trace pass of a target, if any."""
    try:
        for line in open(pass_dir(out, name, "trace") + ".log"):
            if line.startswith("{"):
                return json.loads(line)
    except (OSError, ValueError):
        pass
    return None


# ------------------------------------------------------------------ markdown summaries

def trace_table(r: dict) -> list[str]:
    """Markdown rows of per-kernel trace statistics (µs), busiest first."""
    rows = [(k, v["ns"]) for k, v in r.items() if v.get("ns")]
    total = sum(sum(ns) for _, ns in rows)
    rows.sort(key=lambda kv: -sum(kv[1]))
    lines = ["| Kernel | Calls | Average (µs) | Median (µs) | Min (µs) | Max (µs) | Share of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for k, ns in rows:
        lines.append(f"| `{k}` | {len(ns)} | {statistics.mean(ns) / 1e3:.2f} | {statistics.median(ns) / 1e3:.2f} | "
                     f"{min(ns) / 1e3:.2f} | {max(ns) / 1e3:.2f} | {100 * sum(ns) / total:.1f}% |")
    return lines


def mb(x) -> str:
    return f"{x / 1e6:.1f}"


def traffic_rows(items: list[tuple[str, dict]]) -> list[str]:
    lines = ["| Where | Kernel | trace median (µs) | read (MB) | written (MB) | algorithmic read (MB) | "
             "algorithmic write (MB) | read ratio | write ratio | total ratio | L2 hit rate |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for where, v in items:
        us = f"{v['avg_us']:.2f}" if v.get("avg_us") else "-"
        hit = f"{v['tcc_hit_rate']:.3f}" if v.get("tcc_hit_rate") is not None else "-"
        if "algorithmic_read" in v:
            alg = (f"{mb(v['algorithmic_read'])} | {mb(v['algorithmic_write'])} | {v['fetch_ratio']:.3f} | "
                   f"{v['write_ratio']:.3f} | {v['ratio']:.3f}")
        else:
            alg = "- | - | - | - | -"
        lines.append(f"| {where} | `{v['kernel_name']}` | {us} | {mb(v['fetch_bytes'])} | {mb(v['write_bytes'])} | "
                     f"{alg} | {hit} |")
    return lines


def request_rows(items: list[tuple[str, dict]]) -> list[str]:
    lines = ["| Kernel | read requests | write requests (of them 64 B) | read DRAM-credit stall cycles | "
             "write stall cycles | GRBM_GUI_ACTIVE |", "|---|---|---|---|---|---|"]
    for where, v in items:
        q = v.get("requests", {})

        def g(k):
            return f"{q[k]:.0f}" if k in q else "-"
        lines.append(f"| {where} | {g('TCC_EA0_RDREQ_sum')} | {g('TCC_EA0_WRREQ_sum')} "
                     f"({g('TCC_EA0_WRREQ_64B_sum')}) | {g('TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum')} | "
                     f"{g('TCC_EA0_WRREQ_STALL_sum')} | {g('GRBM_GUI_ACTIVE')} |")
    return lines


def write_md(dirs: list[str], fname: str, lines: list[str]) -> None:
    for d in dirs:
        with open(os.path.join(d, fname), "w") as f:
            f.write("\n".join(lines).rstrip() + "\n")


def calibration_text(cal: dict) -> str:
    return (f"Calibration: the same counters on the plain reference copy of 256 MiB (`python3 bench.py "
            f"--calibrate-copy`, kernel `ref_copy_kernel`, 256 MiB read and 256 MiB written): FETCH_SIZE = "
            f"{cal['FETCH_SIZE_KiB']:.0f} KiB, WRITE_SIZE = {cal['WRITE_SIZE_KiB']:.0f} KiB per launch, so bytes "
            f"read = FETCH_SIZE x 1024 x {cal['fetch_scale']:.4f} and bytes written = WRITE_SIZE x 1024 x "
            f"{cal['write_scale']:.4f}. Figures are medians per launch; durations are the medians of the same "
            f"target's trace pass.")


HEAD = ("Written by `python3 profile_counters.py <out>` (repository root, one MI355X) from the rocprofv3 passes "
        "listed, each run from the repository root; `<out>` holds their raw output.")


def summaries(out: str, res: dict, K: dict, cal: dict, dirs: list[str]) -> None:
    """The markdown summaries of what was collected."""
    wl = si.WORKLOADS["t4096"]
    wdesc = (f"{wl.T} tokens x {wl.H} hidden bf16, {wl.E} experts in {wl.G} groups, top-{wl.K} "
             f"{wl.routing} routing (seed {wl.seed})")
    if "step" in res:
        b = bench_line(out, "step") or {}
        ku = b.get("kernels_us", {})
        lines = ["# Kernel trace: t4096 per-expert step", "", HEAD, "",
                 f"Workload: {wdesc}, per-expert receive buffers. A step is `moe_layout_dispatch` (the layout's "
                 "count kernel, then the bf16 dispatch whose workgroup 0 computes the offsets and per-tile bases "
                 "while every workgroup places its own token) and `moe_combine`; each timed step keeps a status "
                 "word of its own.", "",
                 "    " + command("step", "trace"), "",
                 "Per-kernel statistics over the run (3 warm-up + 20 timed steps, and torch's own set-up copies "
                 "and fills):", ""] + trace_table(res["step"])
        if ku:
            lines += ["", "The bench line of the same run, with HIP events in its timed region: the layout + "
                      f"dispatch call {ku['layout_dispatch']['mean']:.2f} µs (mean; the count kernel, the dispatch "
                      f"and the gap between them), the combine {ku['combine']['mean']:.2f} µs (mean); "
                      f"{b['value']:.1f} GB/s for the step ({b['ms_per_step'] * 1e3:.2f} µs per step by the wall "
                      "clock, the profiler attached). Events bracket the host call, so they also hold the launch gap "
                      "before the kernel and the event commands themselves (a few µs, more with the profiler "
                      "attached); the trace's durations are the kernels' alone."]
        write_md(dirs, "t4096_expert_step_kernel_trace.md", lines)
        items = [("step", K[k]) for k in ("dispatch_expert_bf16", "combine_expert_bf16", "layout_count_t4096")]
        lines = ["# HBM traffic counters: t4096 per-expert step", "", HEAD, "",
                 f"The step of `t4096_expert_step_kernel_trace.md` ({wdesc}). One pass per counter set:", ""]
        lines += ["    " + command("step", k) for k in ("fetch", "write", "tcc", "wrreq", "rdreq")]
        lines += ["", calibration_text(cal), ""] + traffic_rows(items)
        lines += ["", "Memory-side requests (summed over the L2 channels of the 8 XCDs; GRBM_GUI_ACTIVE summed "
                  "over the XCDs):", ""]
        lines += request_rows([(f"`{v['kernel_name']}`", v) for _, v in items[:2]])
        write_md(dirs, "t4096_expert_step_hbm_counters.md", lines)
    wl_items = []
    for n, v in K.items():
        w, _, rest = n.partition(".")
        if w in ("t4096", "skew", "fp8") and rest.split("_")[0] in ("dispatch", "combine", "dequant"):
            wl_items.append((f"{w}:{rest.split('_')[1]}", v))
    if wl_items:
        lines = ["# HBM traffic counters per workload and receive layout", "", HEAD, "",
                 "`bench.py --profile WORKLOAD:LAYOUT` runs only `moe_layout`, `moe_dispatch`, (FP8: "
                 "`moe_fp8_dequant`) and `moe_combine` of one workload and receive layout, 5 times in a row. For "
                 "each of " + ", ".join(PROFILE_TARGETS) + ":", ""]
        lines += ["    " + command("WORKLOAD:LAYOUT", k) for k in BASIC]
        lines += ["", "and for the regroup and the cast-transpose, the table of t4096 (each call timed alone; "
                  "the median of the 51 full-size launches):", ""]
        lines += ["    " + command("table", k) for k in BASIC]
        lines += ["", calibration_text(cal), ""]
        tab = [("t4096 (table)", K[k]) for k in ("t4096.regroup_bf16", "t4096.cast_transpose") if k in K]
        lines += traffic_rows(wl_items + tab)
        lay = [f"{n.split('.')[0]} `{v['kernel_name']}` {v['avg_us']:.2f} µs" for n, v in K.items()
               if ".layout_" in n and v.get("avg_us")]
        if lay:
            lines += ["", "Layout kernels (latency-bound, about 1.5 MB moved each), trace medians: "
                      + "; ".join(lay) + "."]
        write_md(dirs, "per_workload_hbm_counters.md", lines)
    if "mix_dispatch_like" in K and "dispatch_expert_bf16" in K:
        md, mc = K["mix_dispatch_like"], K["mix_combine_like"]
        sd, sc = K["dispatch_expert_bf16"], K["combine_expert_bf16"]
        lines = ["# Read/write-mix references of the dispatch and the combine (t4096 shape)", "", HEAD, "",
                 "`moe_ref_mix` (a measurement aid of the library, not part of the method) moves the bytes of a "
                 "t4096 dispatch or combine over contiguous rows of 14,336 bytes with the kernels' cache policy "
                 "(non-temporal loads, plain stores) and shape (one workgroup per unit, one 16-byte vector per "
                 "lane): the dispatch's mix reads one row and writes it to 8 rows; the combine's mix reads those "
                 "8 rows and writes their XOR to one row. `bench.py --mix-probes` runs the pair back to back 5 "
                 "times, as the step runs dispatch then combine:", ""]
        lines += ["    " + command("mix", k) for k in passes_of("mix")]
        lines += ["", calibration_text(cal), "",
                  "| Reference | trace median (µs) | read (MB) | written (MB) | GB/s | the library's kernel in the "
                  "step (µs) | kernel / reference time |", "|---|---|---|---|---|---|---|"]
        for label, ref, lib in (("dispatch's mix (1 read : 8 written)", md, sd),
                                ("combine's mix (8 read : 1 written)", mc, sc)):
            gbs = ref["traffic_bytes"] / (ref["avg_us"] * 1e-6) / 1e9
            lines.append(f"| {label} | {ref['avg_us']:.2f} | {mb(ref['fetch_bytes'])} | {mb(ref['write_bytes'])} | "
                         f"{gbs:.0f} | {lib['avg_us']:.2f} | {lib['avg_us'] / ref['avg_us']:.3f} |")
        lines += ["", "Memory-side requests, the references against the step's kernels:", ""]
        lines += request_rows([("dispatch's mix", md), (f"`{sd['kernel_name']}` (step)", sd),
                               ("combine's mix", mc), (f"`{sc['kernel_name']}` (step)", sc)])
        write_md(dirs, "rw_mix_ceilings.md", lines)
    if "tables" in res:
        lines = ["# Kernel trace: every call on every workload", "", HEAD, "",
                 f"`bench.py --table {TABLES}` runs every call of the library on each named workload, each call "
                 "timed alone (51 calls per kernel and workload; layout, dispatch and combine in both receive "
                 "layouts, regroup, cast-transpose on the bf16 workloads, and graph replays of the step):", "",
                 "    " + command("tables", "trace"), "",
                 "Per-kernel statistics over all five workloads (an instance serves several workloads and "
                 "layouts; per-workload times are in the bench line's `extra.workloads`, event-timed):", ""]
        lines += trace_table(res["tables"])
        write_md(dirs, "workload_tables_kernel_trace.md", lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out")
    ap.add_argument("--only", default=None)
    ap.add_argument("--from-raw", action="store_true",
                    help="rebuild counters.json and the summaries from OUTDIR's raw output")
    ap.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"),
                    help="where counters.json and the summaries go (default: the repository's profiles/)")
    args = ap.parse_args()
    args.out = os.path.abspath(args.out)   # the passes run from /tmp
    os.makedirs(args.out, exist_ok=True)
    hpath = os.path.join(args.out, "source_hashes.json")
    if args.from_raw:
        names = [n for n in ALL_TARGETS if os.path.isdir(pass_dir(args.out, n, passes_of(n)[0]))]
        hashes = json.load(open(hpath))
    else:
        names = args.only.split(",") if args.only else ALL_TARGETS
        hashes = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
        with open(hpath, "w") as f:
            json.dump(hashes, f, indent=1)
        for n in names:
            for kind in passes_of(n):
                run_pass(args.out, n, kind)
    os.makedirs(args.profiles_dir, exist_ok=True)
    path = os.path.join(args.profiles_dir, "counters.json")
    doc = json.load(open(path)) if os.path.exists(path) else {"kernels": {}}
    if not args.only:
        doc["kernels"] = {}   # every target again: no record of a kernel that no longer runs stays
    res = {n: collect(args.out, n) for n in names}
    if "copy" in res:
        c = pick(res["copy"], "ref_copy_kernel")
        n = 256 << 20
        doc["calibration"] = {"copy_bytes_read": n, "copy_bytes_written": n,
                              "FETCH_SIZE_KiB": statistics.median(c["FETCH_SIZE"]),
                              "WRITE_SIZE_KiB": statistics.median(c["WRITE_SIZE"]),
                              "fetch_scale": n / 1024 / statistics.median(c["FETCH_SIZE"]),
                              "write_scale": n / 1024 / statistics.median(c["WRITE_SIZE"])}
    cal = doc["calibration"]
    scale = (cal["fetch_scale"], cal["write_scale"])
    K = doc.setdefault("kernels", {})
    W = si.WORKLOADS

    def rec(key, kernel, r, prefix, alg, note=None, top=None):
        K[key] = record(kernel, pick(r, prefix), scale, alg, hashes, note, top)
        K[key]["kernel_name"] = next(k for k in sorted(r) if k.startswith(prefix))

    if "step" in res:
        wl = W["t4096"]
        R, P, _ = counts(wl)
        r = res["step"]
        rec("dispatch_expert_bf16", "dispatch", r, "dispatch_bf16_kernel",
            bench.dispatch_bytes(wl.T, wl.H, wl.K, wl.G, R, "expert"),
            "the placing form (moe_layout_dispatch), offsets in workgroup 0")
        rec("combine_expert_bf16", "combine", r, "combine_kernel", bench.combine_bytes(wl.T, wl.H, wl.K, R))
        rec("layout_count_t4096", "layout", r, "layout_count_kernel", None)
    for name in PROFILE_TARGETS:
        if name not in res:
            continue
        w, mode = name.split(":")
        wl = W[w]
        R, P, _ = counts(wl)
        rows = R if mode == "expert" else P
        r = res[name]
        dt = "fp8" if wl.fp8 else "bf16"
        dk = "dispatch_fp8_wave_kernel" if wl.fp8 else "dispatch_bf16_kernel"
        rec(f"{w}.dispatch_{mode}_{dt}", "dispatch", r, dk,
            bench.dispatch_bytes(wl.T, wl.H, wl.K, wl.G, rows, mode, fp8=wl.fp8))
        rec(f"{w}.combine_{mode}_bf16", "combine", r, "combine_kernel", bench.combine_bytes(wl.T, wl.H, wl.K, rows))
        if wl.fp8:
            rec(f"{w}.dequant_{mode}", "combine", r, "fp8_dequant_kernel",
                (rows * (wl.H + wl.H // 128 * 4), rows * wl.H * 2))
        for lk in ("layout_exchange_kernel", "layout_count_kernel", "layout_place_kernel", "layout_onepass_kernel"):
            if any(k.startswith(lk) for k in r):
                rec(f"{w}.{lk.replace('_kernel', '')}", "layout", r, lk, None)
    if "mix" in res:
        wl = W["t4096"]
        row = wl.H * 2
        # the dispatch's mix (1 row read : K written) and the combine's (K read : 1 written)
        rec("mix_dispatch_like", "combine", res["mix"], f"ref_mix_kernel<1, {wl.K}>",
            (wl.T * row, wl.T * wl.K * row))
        rec("mix_combine_like", "combine", res["mix"], f"ref_mix_kernel<{wl.K}, 1>",
            (wl.T * wl.K * row, wl.T * row))
    if "table" in res:
        wl = W["t4096"]
        R, P, ne = counts(wl)
        r = res["table"]
        row_b, meta = 2 * wl.H, wl.K * 8
        rec("t4096.regroup_bf16", "regroup", r, "regroup_kernel",
            (P * (row_b + meta) + wl.T * (wl.G + 2 * wl.K) * 4, R * (row_b + meta)), top=51)
        npad = int(sum((int(n) + 15) // 16 * 16 for n in ne))
        rec("t4096.cast_transpose", "cast_transpose", r, "cast_transpose_cols_kernel",
            (R * wl.H * 2, R * wl.H + npad * wl.H), top=51)
    doc["taken"] = time.strftime("%Y-%m-%d", time.localtime(os.path.getmtime(hpath)))
    dirs = [args.profiles_dir, args.out]
    for d in dirs:
        with open(os.path.join(d, "counters.json"), "w") as f:
            json.dump(doc, f, indent=1)
    summaries(args.out, res, K, cal, dirs)
    print("| kernel instance | avg us | read MB | written MB | read ratio | write ratio | total ratio | L2 hit |")
    print("|---|---|---|---|---|---|---|---|")
    for k, v in K.items():
        fr = f"{v['fetch_ratio']:.3f}" if "fetch_ratio" in v else "-"
        wr = f"{v['write_ratio']:.3f}" if "write_ratio" in v else "-"
        tr = f"{v['ratio']:.3f}" if "ratio" in v else "-"
        hit = f"{v['tcc_hit_rate']:.3f}" if v.get("tcc_hit_rate") is not None else "-"
        us = f"{v['avg_us']:.2f}" if v.get("avg_us") else "-"
        print(f"| {k} | {us} | {v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.1f} | {fr} | {wr} | {tr} | {hit} |")


if __name__ == "__main__":
    main()
