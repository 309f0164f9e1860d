"""bench.py's command line on the CPU: more than one GPU is refused with a message, before
torch or the library is imported (one GPU holds the whole path's share)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_kernel_hash_ignores_comments_but_not_code():
    sys.path.insert(0, ROOT)
    import bench
    a = "int f(int x)\n{\n    return x + 1;   // one more\n}\n/* note */\n"
    b = "int f(int x) { /* the next integer */\n  return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
