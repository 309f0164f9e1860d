"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code):
oracle/sanitize_check.c drives every oracle function over edge shapes (no tokens,
K = E, one group, up to 1024 experts, invalid and repeated entries, empty experts)
and special values with exactly sized buffers; any out-of-bounds access, leak or
undefined behaviour aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    src = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c")]
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", *src, "-lm", "-o", str(exe)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
