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
    (dict(block_m=48), 3, -2),
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
    assert lib.moe_align(ctypes.byref(d), FAKE, 3, 0, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_align(ctypes.byref(d), FAKE, 3, 257, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_align(ctypes.byref(d), FAKE, 49, 32, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_align(ctypes.byref(d), None, 3, 32, FAKE, FAKE, FAKE, FAKE, None) == -1


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
                                 "gate_up_gemm", "down", "down_gemm", "combine"]
    rec = moe.moe_profile_read()
    assert all(v == (0.0, 0) for v in rec.values())
