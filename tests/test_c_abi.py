"""The C boundary used from plain C: tests/c_abi/roundtrip.c includes only
include/moe_ep.h (and the HIP runtime's C API for device memory), links
libmoe_ep.so, and checks layout, dispatch and combine in both receive layouts
against definitions (counts and offsets, receive rows equal to their source rows,
the identity round trip through combine, argument error codes)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "roundtrip")


def test_c_caller_is_built():
    assert os.access(BIN, os.X_OK), "tests/c_abi/roundtrip is built by __graft_entry__.build()"
    r = subprocess.run(["readelf", "-d", BIN], capture_output=True, text=True)
    assert "libmoe_ep.so" in r.stdout


@pytest.mark.gpu
def test_c_caller_round_trip():
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
