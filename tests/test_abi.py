"""CPU-side checks of the C ABI: the library loads, exports every entry point
declared in include/moe.h, and rejects bad arguments before any launch (no
GPU needed: nothing below reaches a HIP call)."""
import ctypes
import os
import re

import pytest

import expert_layer_moe_amd as moe
from expert_layer_moe_amd.binding import EXPORTS, LIB_PATH, moe_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    declared = _declared_functions()
    assert set(declared) == set(EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_nm_shows_c_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in EXPORTS:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def _d(**kw):
    base = dict(T=256, H=7168, E=48, n_shared=0, I=640, act_dtype=moe.MOE_BF16,
                w_dtype=moe.MOE_BF16, w13_scale=None, w2_scale=None, block_m=0, w_layout=0)
    base.update(kw)
    return moe_desc(**base)


def test_header_compiles_as_c_and_links(tmp_path):
    """A C99 program (tests/c_abi/abi_smoke.c) includes moe.h with strict
    warnings as errors, links libmoe_amd.so and calls the host-side entry
    points (nothing is launched)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = LIB_PATH
    src = os.path.join(os.path.dirname(__file__), "c_abi", "abi_smoke.c")
    exe = str(tmp_path / "abi_smoke")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.dirname(HEADER), src, "-o", exe, lib,
                        "-Wl,-rpath," + os.path.dirname(lib)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "abi smoke: ok" in r.stdout, r.stdout + r.stderr


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert moe.moe_status_str(s)
    assert moe.moe_status_str(-99) == "unknown status"


@pytest.mark.parametrize("kw,topk,status", [
    (dict(), 3, 0),
    (dict(T=0), 3, -1),
    (dict(E=0), 1, -1),
    (dict(E=257), 3, -1),
    (dict(), 0, -1),
    (dict(), 49, -1),
    (dict(n_shared=2), 3, -1),
    (dict(H=7200), 3, -2),
    (dict(I=650), 3, -2),
    (dict(act_dtype=moe.MOE_F32), 3, -2),
    (dict(w_dtype=moe.MOE_FP8_E4M3), 3, -1),     # fp8 without scales
    (dict(w_dtype=moe.MOE_FP8_E4M3, I=704, w13_scale=FAKE, w2_scale=FAKE), 3, -2),
    (dict(block_m=48), 3, -1),
    (dict(block_m=8), 3, -1),
    (dict(block_m=16), 3, 0),
    (dict(block_m=32), 3, 0),
    (dict(block_m=64), 3, 0),
    (dict(block_m=128), 3, 0),
    (dict(block_m=256), 3, 0),
    # sorted rows x I at 2^32 and above: past the tiled down GEMM's 32-bit
    # element offsets of h rows
    (dict(T=1 << 20, E=48, I=1024), 8, -2),
    (dict(T=1 << 19, E=48, I=1024), 8, -2),
    (dict(T=1 << 19, E=48, I=512), 8, 0),
    (dict(w_layout=moe.MOE_LAYOUT_FRAG16), 3, 0),
    (dict(w_layout=2), 3, -1),
    (dict(w_layout=moe.MOE_LAYOUT_FRAG16, H=256, I=64, act_dtype=moe.MOE_F32,
          w_dtype=moe.MOE_F32), 3, -2),
])
def test_descriptor_validation(kw, topk, status):
    lib = moe.load_library()
    d = _d(**kw)
    n = lib.moe_workspace_size(ctypes.byref(d), topk)
    assert (n > 0) == (status == 0)
    st = lib.moe_forward(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, topk, FAKE,
                         FAKE, 0, None)
    # valid descriptors fail on the (zero) workspace size instead
    assert st == (status if status != 0 else -3)


def test_null_pointers_rejected():
    lib = moe.load_library()
    d = _d()
    big = lib.moe_workspace_size(ctypes.byref(d), 3)
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        x, r, w13, w2, out = args
        assert lib.moe_forward(ctypes.byref(d), x, None, r, w13, w2, 3, out, FAKE,
                               big, None) == -1
    assert lib.moe_forward(None, FAKE, None, FAKE, FAKE, FAKE, 3, FAKE, FAKE, big, None) == -1
    assert lib.moe_route(ctypes.byref(d), FAKE, None, FAKE, 3, None, FAKE, None, FAKE,
                         big, None) == -1
    assert lib.moe_route(ctypes.byref(d), FAKE, None, FAKE, 3, FAKE, FAKE, None, FAKE,
                         big - 1, None) == -3


def test_align_validation():
    lib = moe.load_library()
    d = _d()
    A = lambda desc, ids, k, bm, ws=None, nbytes=0: lib.moe_align(
        ctypes.byref(desc) if desc is not None else None, ids, k, bm, FAKE, FAKE, FAKE, FAKE,
        ws, nbytes, None)
    assert A(d, FAKE, 3, 0) == -1
    assert A(d, FAKE, 3, 257) == -1
    assert A(d, FAKE, 49, 32) == -1
    assert A(d, None, 3, 32) == -1
    assert A(None, FAKE, 3, 32) == -1
    assert A(_d(n_shared=2), FAKE, 3, 32) == -1
    # more than 8192 assignments with a workspace below 4 ceil(n / 4096) (E + ns)
    # bytes: rejected before any launch
    big = _d(T=4096, E=48, n_shared=1)
    need = 4 * ((4096 * 4 + 4095) // 4096) * 49
    assert A(big, FAKE, 3, 16, FAKE, need - 1) == -3


def test_pack_weights_validation():
    lib = moe.load_library()
    assert lib.moe_pack_weights(None, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_pack_weights(ctypes.byref(_d()), None, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_pack_weights(ctypes.byref(_d()), FAKE, FAKE, FAKE, None, None) == -1
    f32 = _d(H=256, I=64, act_dtype=moe.MOE_F32, w_dtype=moe.MOE_F32)
    assert lib.moe_pack_weights(ctypes.byref(f32), FAKE, FAKE, FAKE, FAKE, None) == -2
    assert lib.moe_pack_weights(ctypes.byref(_d(I=650)), FAKE, FAKE, FAKE, FAKE, None) == -2


def test_path_thresholds_validation():
    lib = moe.load_library()
    assert lib.moe_set_path_thresholds(-1, -1) == -1
    assert lib.moe_set_path_thresholds(16, -2) == -1
    assert lib.moe_set_path_thresholds(16, 1) == 0
    assert lib.moe_set_path_thresholds(128, -1) == 0


def test_workspace_grows_with_batch():
    lib = moe.load_library()
    a = lib.moe_workspace_size(ctypes.byref(_d(T=128)), 3)
    b = lib.moe_workspace_size(ctypes.byref(_d(T=8192)), 3)
    assert 0 < a < b


def test_profile_hooks_without_records():
    assert moe.stage_names() == ["route_logits", "route_topk", "align", "pack_x", "gate_up",
                                 "gate_up_gemm", "down", "down_gemm", "combine", "x_split",
                                 "combine_wait", "expert_mlp"]
    rec = moe.moe_profile_read()
    assert all(v == (0.0, 0) for v in rec.values())


def test_noalloc_validation_before_any_launch():
    """Bad descriptors, null pointers and layers whose workspace exceeds the
    fixed scratch are rejected before the scratch is looked up."""
    lib = moe.load_library()
    F = lambda d, k=3, x=FAKE: lib.moe_forward_noalloc(
        ctypes.byref(d) if d is not None else None, x, None, FAKE, FAKE, FAKE, k, FAKE, None)
    assert F(None) == -1
    assert F(_d(T=0)) == -1
    assert F(_d(H=7200)) == -2
    assert F(_d(), x=None) == -1
    assert F(_d(), k=0) == -1
    big = _d(T=8192)
    assert lib.moe_workspace_size(ctypes.byref(big), 3) > moe.SCRATCH_BYTES
    assert F(big) == -3


def test_signaled_validation_before_any_launch():
    """moe_forward_signaled: bad descriptors, null pointers (the counters
    included), fp32 layers and short workspaces are rejected before any
    launch; the counter count is (E + n_shared) ceil(T / 64)."""
    lib = moe.load_library()
    d = _d()
    big = lib.moe_workspace_size(ctypes.byref(d), 3)
    S = lambda desc, sig=FAKE, ws_bytes=big, x=FAKE, k=3: lib.moe_forward_signaled(
        ctypes.byref(desc) if desc is not None else None, x, None, FAKE, FAKE, FAKE, k, FAKE,
        FAKE, ws_bytes, sig, None, None)
    assert S(None) == -1
    assert S(_d(T=0)) == -1
    assert S(d, sig=None) == -1
    assert S(d, x=None) == -1
    assert S(d, k=0) == -1
    assert S(d, ws_bytes=big - 1) == -3
    f32 = _d(H=256, I=64, act_dtype=moe.MOE_F32, w_dtype=moe.MOE_F32)
    assert S(f32, ws_bytes=lib.moe_workspace_size(ctypes.byref(f32), 3)) == -2
    C = lambda desc: lib.moe_block_signal_count(ctypes.byref(desc) if desc else None)
    assert C(None) == 0
    assert C(_d(T=1, E=48)) == 48
    assert C(_d(T=64, E=48)) == 48
    assert C(_d(T=65, E=48, n_shared=1)) == 2 * 49
    assert C(_d(T=8192, E=256)) == 256 * 128


def test_signal_wait_bound_validation():
    lib = moe.load_library()
    assert lib.moe_set_signal_wait_us(-1) == -1
    assert lib.moe_set_signal_wait_us(1000001) == -1
    assert lib.moe_set_signal_wait_us(0) == 0
    assert lib.moe_set_signal_wait_us(10000) == 0


def test_one_launch_switch_validation():
    lib = moe.load_library()
    assert lib.moe_set_one_launch(2) == -1 and lib.moe_set_one_launch(-1) == -1
    d = _d()
    base = lib.moe_workspace_size(ctypes.byref(d), 3)
    assert lib.moe_set_one_launch(1) == 0
    try:
        # the counters' room is always in the workspace
        assert lib.moe_workspace_size(ctypes.byref(d), 3) == base
    finally:
        assert lib.moe_set_one_launch(0) == 0


def test_scratch_bytes_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define MOE_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == moe.SCRATCH_BYTES


def test_fp8_mfma_switch_and_workspace():
    """The fp8 gate/up GEMM's arithmetic is process-wide; the two-term token
    codes (2 T H + 4 T bytes) are in the workspace only when that path can
    run (fp8 weights, a batch large enough for the tiled GEMM)."""
    lib = moe.load_library()
    assert lib.moe_set_fp8_mfma(2) == -1 and lib.moe_set_fp8_mfma(-1) == -1
    d = _d(T=8192, E=256, I=256, w_dtype=moe.MOE_FP8_E4M3, w13_scale=FAKE, w2_scale=FAKE)
    try:
        assert lib.moe_set_fp8_mfma(0) == 0
        off = lib.moe_workspace_size(ctypes.byref(d), 8)
        assert lib.moe_set_fp8_mfma(1) == 0
        on = lib.moe_workspace_size(ctypes.byref(d), 8)
        assert on - off >= 2 * 8192 * 7168 + 4 * 8192
        # the size does not depend on the path thresholds
        assert lib.moe_set_path_thresholds(16, 1) == 0
        assert lib.moe_workspace_size(ctypes.byref(d), 8) == on
        bf16 = _d(T=8192, E=256, I=256)
        b = lib.moe_workspace_size(ctypes.byref(bf16), 8)
        assert lib.moe_set_fp8_mfma(0) == 0
        assert lib.moe_workspace_size(ctypes.byref(bf16), 8) == b   # bf16 weights: no codes
    finally:
        lib.moe_set_fp8_mfma(0)
        lib.moe_set_path_thresholds(128, -1)


@pytest.mark.skip(reason="one-launch expert MLP switched off (its first GPU run hung, "
                         "cause not found): moe_set_one_stage is not exported")
def test_one_stage_switch_and_workspace():
    """The one-launch expert MLP is process-wide; it needs its own copy of the
    packed token rows and sync words, only for batches that can stream every
    segment (no tiled GEMM)."""
    lib = moe.load_library()
    assert lib.moe_set_one_stage(2) == -1
    d = _d()   # the 48-expert decode share
    try:
        assert lib.moe_set_one_stage(0) == 0
        off = lib.moe_workspace_size(ctypes.byref(d), 3)
        assert lib.moe_set_one_stage(1) == 0
        on = lib.moe_workspace_size(ctypes.byref(d), 3)
        assert on > off
        big = _d(T=8192)   # may take the tiled GEMM: never one launch
        a = lib.moe_workspace_size(ctypes.byref(big), 3)
        assert lib.moe_set_one_stage(0) == 0
        assert lib.moe_workspace_size(ctypes.byref(big), 3) == a
    finally:
        lib.moe_set_one_stage(0)
