"""Host-side checks of bench.py (no GPU): the kernel-source hash that keys the
stored traffic counters follows the code and not its comments, and asking for
more than one GPU is refused with a message."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* the\n result */\n}\n"
    b = "// f doubles its argument\nint f(int x) {\n\n    return 2 * x;\n}"
    assert bench._code_only(a) == bench._code_only(b)


def test_code_only_follows_code_changes():
    a = "int f(int x) { return 2 * x; }"
    b = "int f(int x) { return 3 * x; }"
    assert bench._code_only(a) != bench._code_only(b)


def test_source_sha_is_stable_and_distinct_per_kernel():
    assert bench.source_sha("gate_up") == bench.source_sha("gate_up")
    assert bench.source_sha("gate_up") != bench.source_sha("gate_up_gemm")
    assert len(bench.source_sha("gate_up_gemm")) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
