"""MI355X-native MoE expert-layer forward: hand-written gfx950 HIP kernels
behind a C ABI (include/moe.h), with a thin ctypes binding."""
from .binding import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_LAYOUT_FRAG16,
                      MOE_LAYOUT_ROW_MAJOR, MoeError, alloc_workspace,
                      load_library, make_desc, moe_align, moe_desc, moe_forward,
                      moe_forward_noalloc, moe_forward_signaled, moe_block_signal_count,
                      moe_set_signal_wait_us, moe_set_one_launch, SCRATCH_BYTES,
                      moe_pack_weights, moe_set_fp8_mfma, moe_set_path_thresholds,
                      moe_profile_enable, moe_profile_read, moe_route,
                      moe_status_str, moe_workspace_size, stage_names)
from .layer import DeviceLayer

__all__ = [
    "MOE_BF16", "MOE_F32", "MOE_FP8_E4M3", "MOE_LAYOUT_FRAG16", "MOE_LAYOUT_ROW_MAJOR",
    "MoeError", "alloc_workspace", "load_library", "make_desc", "moe_align", "moe_desc",
    "moe_forward", "moe_forward_noalloc", "moe_forward_signaled", "moe_block_signal_count",
    "moe_set_signal_wait_us", "moe_set_one_launch", "SCRATCH_BYTES", "moe_pack_weights", "moe_set_fp8_mfma", "moe_set_path_thresholds",
    "moe_profile_enable", "moe_profile_read", "moe_route", "moe_status_str",
    "moe_workspace_size", "stage_names", "DeviceLayer",
]
