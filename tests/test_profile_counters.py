"""profile_counters.py's arithmetic, on a synthetic raw rocprofv3 output (no GPU):
the copy calibration (bytes = counter KiB x 1024 x the copy's ratio of known to
counted bytes, a dispatch's counter instances summed), the ratios to algorithmic
bytes, the L2 hit rate and the trace median of a kernel, as `--from-raw` rebuilds
them into a directory of their own."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY = "void moe::(anonymous namespace)::ref_copy_kernel(unsigned int __vector(4) const*, unsigned int __vector(4)*, long)"
MIX81 = "void moe::(anonymous namespace)::ref_mix_kernel<8, 1>(unsigned int __vector(4) const*, unsigned int __vector(4)*, int)"
MIX18 = "void moe::(anonymous namespace)::ref_mix_kernel<1, 8>(unsigned int __vector(4) const*, unsigned int __vector(4)*, int)"


def _counters(d, rows):
    """rows: (dispatch id, kernel, counter, value); several rows of one dispatch and
    counter are its instances."""
    os.makedirs(d)
    with open(os.path.join(d, "k_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def _trace(d, rows):
    os.makedirs(d)
    with open(os.path.join(d, "k_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)


def test_from_raw_arithmetic(tmp_path):
    out, prof = tmp_path / "raw", tmp_path / "profiles"
    out.mkdir()
    (out / "source_hashes.json").write_text(json.dumps({k: "h-" + k for k in (
        "dispatch", "combine", "layout", "regroup", "cast_transpose")}))
    # the copy: 256 MiB each way; FETCH_SIZE counts half of it, in two instances
    _trace(str(out / "copy_trace"), [(COPY, 0, 100000)])
    _counters(str(out / "copy_fetch"), [(1, COPY, "FETCH_SIZE", 65536.0), (1, COPY, "FETCH_SIZE", 65536.0)])
    _counters(str(out / "copy_write"), [(1, COPY, "WRITE_SIZE", 262144.0)])
    _counters(str(out / "copy_tcc"), [(1, COPY, "TCC_HIT_sum", 1.0), (1, COPY, "TCC_MISS_sum", 3.0)])
    # the mix references at the t4096 shape (4096 rows of 14336 bytes, top-8)
    row, T, K = 14336, 4096, 8
    rd81, wr81 = T * K * row, T * row
    _trace(str(out / "mix_trace"), [(MIX81, 0, 88000), (MIX81, 0, 92000), (MIX81, 0, 90000),
                                    (MIX18, 0, 70000)])
    _counters(str(out / "mix_fetch"), [(1, MIX81, "FETCH_SIZE", rd81 * 1.01 / 1024 / 2), (2, MIX18, "FETCH_SIZE",
                                                                                          wr81 / 1024 / 2)])
    _counters(str(out / "mix_write"), [(1, MIX81, "WRITE_SIZE", wr81 / 1024), (2, MIX18, "WRITE_SIZE",
                                                                              rd81 / 1024)])
    _counters(str(out / "mix_tcc"), [(1, MIX81, "TCC_HIT_sum", 10.0), (1, MIX81, "TCC_MISS_sum", 90.0),
                                     (2, MIX18, "TCC_HIT_sum", 0.0), (2, MIX18, "TCC_MISS_sum", 1.0)])
    r = subprocess.run([sys.executable, os.path.join(ROOT, "profile_counters.py"), str(out), "--from-raw",
                        "--profiles-dir", str(prof)], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
    doc = json.load(open(prof / "counters.json"))
    cal = doc["calibration"]
    assert cal["FETCH_SIZE_KiB"] == 131072 and cal["fetch_scale"] == 2.0 and cal["write_scale"] == 1.0
    m = doc["kernels"]["mix_combine_like"]
    assert m["kernel_name"] == "ref_mix_kernel<8, 1>" and m["source_hash"] == "h-combine"
    assert m["fetch_bytes"] == pytest.approx(rd81 * 1.01) and m["write_bytes"] == pytest.approx(wr81)
    assert m["fetch_ratio"] == pytest.approx(1.01) and m["write_ratio"] == pytest.approx(1.0)
    assert m["ratio"] == pytest.approx((rd81 * 1.01 + wr81) / (rd81 + wr81))
    assert m["avg_us"] == pytest.approx(90.0) and m["tcc_hit_rate"] == pytest.approx(0.1)
    d = doc["kernels"]["mix_dispatch_like"]
    assert d["fetch_ratio"] == pytest.approx(1.0) and d["write_ratio"] == pytest.approx(1.0)
    assert d["avg_us"] == pytest.approx(70.0)
    # the copy beside the raw output equals the one in the profiles directory
    assert json.load(open(out / "counters.json")) == doc
