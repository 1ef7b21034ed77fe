"""ctypes binding of libmoe_amd.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels; this module only
checks tensor shapes / dtypes / devices and passes raw device pointers and the
current HIP stream.  PyTorch provides device memory and streams.  There is no
fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe_amd.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_LAYOUT_ROW_MAJOR, MOE_LAYOUT_FRAG16 = 0, 1
_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
           -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP"}

EXPORTS = ["moe_workspace_size", "moe_route", "moe_align", "moe_forward",
           "moe_forward_noalloc", "moe_forward_signaled", "moe_block_signal_count", "moe_set_signal_wait_us", "moe_set_one_launch",
           "moe_pack_weights", "moe_set_path_thresholds", "moe_set_fp8_mfma", "moe_status_str", "moe_num_stages", "moe_stage_name",
           "moe_profile_enable", "moe_profile_read"]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class moe_desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("I", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("block_m", ctypes.c_int32), ("w_layout", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(the MoE layer has no fallback path)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(moe_desc)
    lib.moe_workspace_size.argtypes = [D, I32]
    lib.moe_workspace_size.restype = SZ
    lib.moe_route.argtypes = [D, P, P, P, I32, P, P, P, P, SZ, P]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_align.argtypes = [D, P, I32, I32, P, P, P, P, P, SZ, P]
    lib.moe_align.restype = ctypes.c_int
    lib.moe_forward.argtypes = [D, P, P, P, P, P, I32, P, P, SZ, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [D, P, P, P, P, P, I32, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_signaled.argtypes = [D, P, P, P, P, P, I32, P, P, SZ, P, P, P]
    lib.moe_forward_signaled.restype = ctypes.c_int
    lib.moe_block_signal_count.argtypes = [D]
    lib.moe_block_signal_count.restype = SZ
    lib.moe_set_signal_wait_us.argtypes = [I32]
    lib.moe_set_signal_wait_us.restype = ctypes.c_int
    lib.moe_set_one_launch.argtypes = [I32]
    lib.moe_set_one_launch.restype = ctypes.c_int
    lib.moe_pack_weights.argtypes = [D, P, P, P, P, P]
    lib.moe_pack_weights.restype = ctypes.c_int
    lib.moe_set_fp8_mfma.argtypes = [I32]
    lib.moe_set_fp8_mfma.restype = ctypes.c_int
    lib.moe_set_path_thresholds.argtypes = [I32, I32]
    lib.moe_set_path_thresholds.restype = ctypes.c_int
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_num_stages.argtypes = []
    lib.moe_num_stages.restype = ctypes.c_int
    lib.moe_stage_name.argtypes = [ctypes.c_int]
    lib.moe_stage_name.restype = ctypes.c_char_p
    lib.moe_profile_enable.argtypes = [ctypes.c_int]
    lib.moe_profile_enable.restype = ctypes.c_int
    lib.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int32), I32]
    lib.moe_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, load_library().moe_status_str(status).decode())


_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_FP8_E4M3}


def make_desc(T, H, E, I, n_shared=0, act_dtype=MOE_BF16, w_dtype=MOE_BF16,
              w13_scale: Optional[torch.Tensor] = None,
              w2_scale: Optional[torch.Tensor] = None, block_m=0,
              w_layout=MOE_LAYOUT_ROW_MAJOR) -> moe_desc:
    return moe_desc(T, H, E, n_shared, I, act_dtype, w_dtype,
                    _ptr(w13_scale), _ptr(w2_scale), block_m, w_layout)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _act(desc):
    return torch.float32 if desc.act_dtype == MOE_F32 else torch.bfloat16


def _w(desc):
    return {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16,
            MOE_FP8_E4M3: torch.uint8}[desc.w_dtype]


def moe_workspace_size(desc: moe_desc, topk: int) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(desc), topk))


def alloc_workspace(desc: moe_desc, topk: int, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(desc, topk)
    if n == 0:
        raise MoeError(-1, "invalid descriptor")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(desc, x, valid_rows, router_w, topk, topk_ids, topk_w, logits=None,
              workspace=None, stream=None):
    T, H, E = desc.T, desc.H, desc.E
    ws = workspace if workspace is not None else alloc_workspace(desc, topk, x.device)
    _check(load_library().moe_route(
        ctypes.byref(desc), _dev(x, "x", _act(desc), (T, H)),
        _dev(valid_rows, "valid_rows", torch.uint8, (T,)),
        _dev(router_w, "router_w", _act(desc), (E, H)), topk,
        _dev(topk_ids, "topk_ids", torch.int32, (T, topk)),
        _dev(topk_w, "topk_w", torch.float32, (T, topk)),
        _dev(logits, "logits", torch.float32, (T, E)),
        _dev(ws, "workspace", torch.uint8), ws.numel(), _stream(stream)))
    return ws


def moe_align(desc, topk_ids, topk, block_m, sorted_ids, block_expert,
              expert_offsets, n_post_padded, workspace=None, stream=None):
    T, E, ns = desc.T, desc.E, desc.n_shared
    cap = T * (topk + ns) + (E + ns) * (block_m - 1)
    if sorted_ids.numel() < cap or block_expert.numel() < (cap + block_m - 1) // block_m:
        raise ValueError("sorted_ids / block_expert below the documented capacity")
    if expert_offsets.numel() < E + ns + 1:
        raise ValueError("expert_offsets holds E + n_shared + 1 entries")
    _check(load_library().moe_align(
        ctypes.byref(desc), _dev(topk_ids, "topk_ids", torch.int32, (T, topk)), topk,
        block_m, _dev(sorted_ids, "sorted_ids", torch.int32),
        _dev(block_expert, "block_expert", torch.int32),
        _dev(expert_offsets, "expert_offsets", torch.int32),
        _dev(n_post_padded, "n_post_padded", torch.int32, (1,)),
        _dev(workspace, "workspace", torch.uint8),
        0 if workspace is None else workspace.numel(), _stream(stream)))


def moe_forward(desc, x, valid_rows, router_w, w13, w2, topk, out, workspace,
                stream=None):
    T, H, E, I, ns = desc.T, desc.H, desc.E, desc.I, desc.n_shared
    _check(load_library().moe_forward(
        ctypes.byref(desc), _dev(x, "x", _act(desc), (T, H)),
        _dev(valid_rows, "valid_rows", torch.uint8, (T,)),
        _dev(router_w, "router_w", _act(desc), (E, H)),
        _dev(w13, "w13", _w(desc), (E + ns, 2 * I, H)),
        _dev(w2, "w2", _w(desc), (E + ns, H, I)), topk,
        _dev(out, "out", _act(desc), (T, H)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)))


def moe_forward_noalloc(desc, x, valid_rows, router_w, w13, w2, topk, out, stream=None):
    """moe_forward in the library's fixed device scratch (no workspace)."""
    T, H, E, I, ns = desc.T, desc.H, desc.E, desc.I, desc.n_shared
    _check(load_library().moe_forward_noalloc(
        ctypes.byref(desc), _dev(x, "x", _act(desc), (T, H)),
        _dev(valid_rows, "valid_rows", torch.uint8, (T,)),
        _dev(router_w, "router_w", _act(desc), (E, H)),
        _dev(w13, "w13", _w(desc), (E + ns, 2 * I, H)),
        _dev(w2, "w2", _w(desc), (E + ns, H, I)), topk,
        _dev(out, "out", _act(desc), (T, H)), _stream(stream)))


def moe_block_signal_count(desc: moe_desc) -> int:
    """Entries of moe_forward_signaled's completion counters."""
    return int(load_library().moe_block_signal_count(ctypes.byref(desc)))


def moe_forward_signaled(desc, x, valid_rows, router_w, w13, w2, topk, out, workspace,
                         block_signal, stream=None, consumer_stream=None):
    """moe_forward with per-(expert, 64-row block) completion counters
    (block_signal, int32 [E + n_shared, ceil(T / 64)]) and the combine waiting
    on them on consumer_stream (None: the current stream, like `stream`)."""
    T, H, E, I, ns = desc.T, desc.H, desc.E, desc.I, desc.n_shared
    _check(load_library().moe_forward_signaled(
        ctypes.byref(desc), _dev(x, "x", _act(desc), (T, H)),
        _dev(valid_rows, "valid_rows", torch.uint8, (T,)),
        _dev(router_w, "router_w", _act(desc), (E, H)),
        _dev(w13, "w13", _w(desc), (E + ns, 2 * I, H)),
        _dev(w2, "w2", _w(desc), (E + ns, H, I)), topk,
        _dev(out, "out", _act(desc), (T, H)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _dev(block_signal, "block_signal", torch.int32, (E + ns, (T + 63) // 64)),
        _stream(stream), _stream(consumer_stream)))


def moe_set_signal_wait_us(us: int = 10000):
    """Time bound of each wait of the signaled combine (process-wide)."""
    _check(load_library().moe_set_signal_wait_us(us))


def moe_set_one_launch(enable: bool = False):
    """Calls where every segment streams: gate/up and down in one launch
    (True) or two (False, the default).  Process-wide."""
    _check(load_library().moe_set_one_launch(1 if enable else 0))


SCRATCH_BYTES = 64 << 20   # MOE_SCRATCH_BYTES


def moe_pack_weights(desc, w13, w2, w13_packed=None, w2_packed=None, stream=None):
    """Row-major w13 / w2 -> the MFMA fragment layout (MOE_LAYOUT_FRAG16).
    Returns the packed tensors (allocated here when not given)."""
    ne, H, I = desc.E + desc.n_shared, desc.H, desc.I
    w13_packed = torch.empty_like(w13) if w13_packed is None else w13_packed
    w2_packed = torch.empty_like(w2) if w2_packed is None else w2_packed
    wd = _w(desc)
    _check(load_library().moe_pack_weights(
        ctypes.byref(desc), _dev(w13, "w13", wd, (ne, 2 * I, H)),
        _dev(w2, "w2", wd, (ne, H, I)),
        _dev(w13_packed, "w13_packed", wd, (ne, 2 * I, H)),
        _dev(w2_packed, "w2_packed", wd, (ne, H, I)), _stream(stream)))
    return w13_packed, w2_packed


def moe_set_path_thresholds(gemm_min_rows: int = 128, gemm_min_tiles: int = -1):
    """Segments above gemm_min_rows rows use the tiled GEMM kernels once their
    tiles number gemm_min_tiles (-1 = fill the chip).  Process-wide."""
    _check(load_library().moe_set_path_thresholds(gemm_min_rows, gemm_min_tiles))


def moe_set_fp8_mfma(enable: bool = False):
    """fp8 weights on the tiled gate/up GEMM: fp8 MFMA on two-term token
    codes (True) or bf16 MFMA on dequantised weights (False, the default).
    Process-wide; size workspaces after choosing."""
    _check(load_library().moe_set_fp8_mfma(1 if enable else 0))


def moe_status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


# ---- measurement hooks -------------------------------------------------------
def stage_names():
    lib = load_library()
    return [lib.moe_stage_name(i).decode() for i in range(lib.moe_num_stages())]


def moe_profile_enable(stages=None):
    """Time the named stages (None or [] = off, "all" = every stage)."""
    if stages == "all":
        mask = -1
    else:
        names = stage_names()
        mask = 0
        for s in stages or []:
            mask |= 1 << names.index(s)
    _check(load_library().moe_profile_enable(mask))


def moe_profile_read():
    lib = load_library()
    n = lib.moe_num_stages()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib.moe_profile_read(ms, cnt, n))
    return {name: (ms[i], cnt[i]) for i, name in enumerate(stage_names())}
