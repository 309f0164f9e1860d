"""HBM traffic counters of the library's kernels -> profiles/counters.json.

    python3 profile_counters.py OUTDIR [--only NAMES]

From the repository root on a GPU machine. Runs rocprofv3 over bench.py targets,
each pass a process of its own (rocprofv3 does not split counters over passes):
a kernel trace (durations), then FETCH_SIZE, WRITE_SIZE and TCC_HIT_sum +
TCC_MISS_sum as separate --pmc runs. Targets (NAMES for --only, comma-separated):

  copy    bench.py --calibrate-copy: the plain 256 MiB reference copy, whose known
          bytes scale the counters (FETCH_SIZE counts half of what a copy reads)
  step    bench.py --steps 20 --warmup 3 --no-extras --no-cpu-baseline --processes 1:
          the headline step (the layout's count kernel, the placing dispatch, combine)
  W:L     bench.py --profile W:L for W in t4096, skew, fp8 and L in expert, group:
          moe_layout, moe_dispatch, (FP8) moe_fp8_dequant and moe_combine, 5 times each
  mix     bench.py --mix-probes: the read/write-mix references of the dispatch and combine
  table   bench.py --table t4096: the regroup and the cast-transpose among every call

Each kernel instance gets the median over its launches of the bytes per launch
(counter KiB x 1024 x the copy's ratio of known to counted bytes), their ratio to
the algorithmic bytes where bench.py defines them, the L2 hit rate, the average
duration from the trace, and the hash of its kernel's code (bench.py's
source_hash: comments and spacing aside). bench.py reports `traffic` only while
that hash matches the current sources. Raw rocprofv3 output stays in OUTDIR, with a
copy of the resulting counters.json; a markdown table of the result is printed.
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

PASSES = (("trace", ["--kernel-trace", "--stats"]), ("fetch", ["--pmc", "FETCH_SIZE"]),
          ("write", ["--pmc", "WRITE_SIZE"]), ("tcc", ["--pmc", "TCC_HIT_sum", "TCC_MISS_sum"]))
PROFILE_TARGETS = [f"{w}:{m}" for w in ("t4096", "skew", "fp8") for m in ("expert", "group")]


def target_args(name: str) -> list[str]:
    if name == "copy":
        return ["--calibrate-copy"]
    if name == "step":
        return ["--steps", "20", "--warmup", "3", "--no-extras", "--no-cpu-baseline", "--processes", "1"]
    if name == "mix":
        return ["--mix-probes"]
    if name == "table":
        return ["--table", "t4096"]
    return ["--profile", name]


def run_pass(out: str, name: str, kind: str, flags: list[str]) -> str:
    """One rocprofv3 run; returns its output directory."""
    d = os.path.join(out, f"{name.replace(':', '_')}_{kind}")
    cmd = ["timeout", "-s", "KILL", "300", "rocprofv3", *flags, "-f", "csv", "-d", d, "-o", "k", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *target_args(name)]
    env = dict(os.environ, TMPDIR="/tmp")
    t0 = time.time()
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(d + ".log", "w") as f:
        f.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    print(f"{name} {kind}: exit {r.returncode} in {time.time() - t0:.0f} s", flush=True)
    if r.returncode != 0:
        raise SystemExit(f"rocprofv3 failed for {name} {kind}; see {d}.log")
    return d


def per_dispatch(d: str) -> dict:
    """{kernel name: [value per dispatch]} from a counter-collection run (summed over
    the counter's instances), or {kernel name: [duration ns]} from a trace."""
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
        out[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def base_name(kernel_name: str) -> str:
    """A kernel's name with its template arguments, without namespaces and parameters."""
    n = kernel_name.replace("(anonymous namespace)::", "").split("(")[0]
    n = n[5:] if n.startswith("void ") else n
    return n.replace("moe::", "").strip()


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


def collect(out: str, name: str) -> dict:
    """{kernel: {"ns": [...], "fetch": [...], "write": [...], "hit": [...], "miss": [...]}}"""
    res = collections.defaultdict(lambda: collections.defaultdict(list))
    for kind, flags in PASSES:
        d = run_pass(out, name, kind, flags)
        for k, vals in per_dispatch(d).items():
            kb = base_name(k)
            if kind == "trace":
                res[kb]["ns"] += vals
            else:
                for v in vals:
                    if "FETCH_SIZE" in v:
                        res[kb]["fetch"].append(v["FETCH_SIZE"])
                    if "WRITE_SIZE" in v:
                        res[kb]["write"].append(v["WRITE_SIZE"])
                    if "TCC_HIT_sum" in v:
                        res[kb]["hit"].append(v["TCC_HIT_sum"])
                        res[kb]["miss"].append(v["TCC_MISS_sum"])
    return res


def median_top(vals: list[float], n: int | None) -> float:
    """Median of the n largest values (a kernel name shared by calls of other sizes in
    one run, e.g. the table's, keeps its full-size launches), or of all."""
    v = sorted(vals)
    return statistics.median(v[-n:] if n else v)


def record(kernel: str, c: dict, scale: tuple, alg: tuple | None, note: str | None = None, top=None) -> dict:
    fs, ws = scale
    fb = median_top(c["fetch"], top) * 1024 * fs
    wb = median_top(c["write"], top) * 1024 * ws
    r = {"kernel": kernel, "source_hash": bench.source_hash(kernel), "fetch_bytes": fb, "write_bytes": wb,
         "traffic_bytes": fb + wb, "avg_us": median_top(c["ns"], top) / 1e3 if c["ns"] else None}
    if c["hit"]:
        h, m = median_top(c["hit"], top), median_top(c["miss"], top)
        r["tcc_hit_rate"] = h / (h + m) if h + m else None
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out")
    ap.add_argument("--only", default=None)
    args = ap.parse_args()
    args.out = os.path.abspath(args.out)   # the passes run from /tmp
    os.makedirs(args.out, exist_ok=True)
    names = args.only.split(",") if args.only else ["copy", "step", *PROFILE_TARGETS, "mix", "table"]
    path = os.path.join(ROOT, "profiles", "counters.json")
    doc = json.load(open(path)) if os.path.exists(path) else {"kernels": {}}
    if not args.only:
        doc["kernels"] = {}   # every target again: no record of a kernel that no longer runs stays
    res = {n: collect(args.out, n) for n in names}
    if "copy" in res:
        c = pick(res["copy"], "ref_copy_kernel")
        n = 256 << 20
        doc["calibration"] = {"copy_bytes_read": n, "copy_bytes_written": n,
                              "FETCH_SIZE_KiB": statistics.median(c["fetch"]),
                              "WRITE_SIZE_KiB": statistics.median(c["write"]),
                              "fetch_scale": n / 1024 / statistics.median(c["fetch"]),
                              "write_scale": n / 1024 / statistics.median(c["write"])}
    cal = doc["calibration"]
    scale = (cal["fetch_scale"], cal["write_scale"])
    K = doc.setdefault("kernels", {})
    W = si.WORKLOADS
    if "step" in res:
        wl = W["t4096"]
        R, P, _ = counts(wl)
        r = res["step"]
        K["dispatch_expert_bf16"] = record("dispatch", pick(r, "dispatch_bf16_kernel"), scale,
                                           bench.dispatch_bytes(wl.T, wl.H, wl.K, wl.G, R, "expert"),
                                           "the placing form (moe_layout_dispatch), offsets in workgroup 0")
        K["combine_expert_bf16"] = record("combine", pick(r, "combine_kernel"), scale,
                                          bench.combine_bytes(wl.T, wl.H, wl.K, R))
        K["layout_count_t4096"] = record("layout", pick(r, "layout_count_kernel"), scale, None)
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
        K[f"{w}.dispatch_{mode}_{dt}"] = record(
            "dispatch", pick(r, dk), scale, bench.dispatch_bytes(wl.T, wl.H, wl.K, wl.G, rows, mode, fp8=wl.fp8))
        K[f"{w}.combine_{mode}_bf16"] = record("combine", pick(r, "combine_kernel"), scale,
                                               bench.combine_bytes(wl.T, wl.H, wl.K, rows))
        if wl.fp8:
            K[f"{w}.dequant_{mode}"] = record("combine", pick(r, "fp8_dequant_kernel"), scale,
                                              (rows * (wl.H + wl.H // 128 * 4), rows * wl.H * 2))
        for lk in ("layout_exchange_kernel", "layout_count_kernel", "layout_place_kernel", "layout_onepass_kernel"):
            if any(k.startswith(lk) for k in r):
                K[f"{w}.{lk.replace('_kernel', '')}"] = record("layout", pick(r, lk), scale, None)
    if "mix" in res:
        wl = W["t4096"]
        row = wl.H * 2
        # the dispatch's mix (1 row read : K written) and the combine's (K read : 1 written)
        K["mix_dispatch_like"] = record("combine", pick(res["mix"], f"ref_mix_kernel<1, {wl.K}>"), scale,
                                        (wl.T * row, wl.T * wl.K * row))
        K["mix_combine_like"] = record("combine", pick(res["mix"], f"ref_mix_kernel<{wl.K}, 1>"), scale,
                                       (wl.T * wl.K * row, wl.T * row))
    if "table" in res:
        wl = W["t4096"]
        R, P, ne = counts(wl)
        r = res["table"]
        row_b, meta = 2 * wl.H, wl.K * 8
        K["t4096.regroup_bf16"] = record("regroup", pick(r, "regroup_kernel"), scale,
                                         (P * (row_b + meta) + wl.T * (wl.G + 2 * wl.K) * 4, R * (row_b + meta)),
                                         top=51)
        npad = int(sum((int(n) + 15) // 16 * 16 for n in ne))
        K["t4096.cast_transpose"] = record("cast_transpose", pick(r, "cast_transpose_cols_kernel"), scale,
                                           (R * wl.H * 2, R * wl.H + npad * wl.H), top=51)
    doc["taken"] = time.strftime("%Y-%m-%d")
    for p in (path, os.path.join(args.out, "counters.json")):   # the second beside the raw output
        with open(p, "w") as f:
            json.dump(doc, f, indent=1)
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
