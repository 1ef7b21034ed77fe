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


def test_dtype_follows_the_workload():
    from workloads import get_config
    assert bench.compute_dtype(get_config("tiny")) == "f32"
    assert bench.compute_dtype(get_config("decode_e48")) == "bf16"
    # fp8 weights are converted to bf16 for bf16 MFMA
    assert bench.compute_dtype(get_config("prefill_ub_fp8")) == "bf16"
    # ... unless the gate/up GEMM runs on the fp8 MFMA
    assert bench.compute_dtype(get_config("prefill_ub_fp8"), fp8_mfma=True) == "fp8+bf16"
    assert bench.compute_dtype(get_config("decode_e48"), fp8_mfma=True) == "bf16"


def test_nested_workload_names_resolve():
    """Every nested workload name strips to a configured base workload, and
    the fp8-MFMA variants are fp8-weight layers."""
    from workloads import get_config
    for name in bench.NESTED:
        base = name
        for suffix in (bench.SIGNALED, bench.ONE_LAUNCH, bench.FP8_MFMA):
            if base.endswith(suffix):
                base = base[:-len(suffix)]
        base = "prefill_ub_fp8" if base in bench.PREFILL_SPLITS or base == "prefill_unsplit" else base
        cfg = get_config(base)
        if name.endswith(bench.FP8_MFMA):
            assert cfg.w == "fp8"


def test_host_info_names_the_cpu():
    info = bench.host_info()
    assert info["nproc"] >= 1 and info["usable_cpus"] >= 1
    assert isinstance(info["cpu_model"], str)


def test_unknown_config_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "nope"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and r.stdout == ""


def test_algorithmic_work_counts_touched_experts_and_valid_rows():
    """decode_e48-shaped counts by hand: 2 touched experts of I = 640, H = 7168,
    bf16, 3 valid rows of 5, top-3."""
    import numpy as np
    from workloads import get_config
    cfg = get_config("decode_e48").with_(T=5)
    ids = np.array([[0, 5, 5], [5, 0, 0], [-1, -1, -1], [0, 0, 5], [-1, -1, -1]])
    w = bench.algorithmic_work(cfg, ids, 3)
    H, I = 7168, 640
    assert w["touched_experts"] == 2
    assert w["gate_up_bytes"] == 2 * 2 * I * H * 2 + 3 * H * 2
    assert w["gate_up_flops"] == 2.0 * 3 * 3 * H * 2 * I
    assert w["step_bytes"] == 2 * 3 * I * H * 2 + 3 * H * 2 + 5 * H * 2 + 48 * H * 2
