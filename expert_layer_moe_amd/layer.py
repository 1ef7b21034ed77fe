"""Device-resident layer: weights, descriptor and workspace for repeated
moe_forward calls (memory management only; the math is in the kernels)."""
from __future__ import annotations

from typing import Optional

import torch

from .binding import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_LAYOUT_FRAG16,
                      MOE_LAYOUT_ROW_MAJOR, alloc_workspace, make_desc, moe_forward,
                      moe_forward_signaled, moe_pack_weights, moe_route)

_ACT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
_W = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_FP8_E4M3}


class DeviceLayer:
    """Holds one layer's router / expert weights on the GPU.

    router [E, H], w13 [E+ns, 2I, H], w2 [E+ns, H, I] (uint8 = fp8 e4m3fn codes
    with fp32 block scales s13 [E+ns, 2I/128, H/128], s2 [E+ns, H/128, I/128]).
    packed=True re-lays the expert weights out once with moe_pack_weights and
    keeps only that copy (bf16 / fp8 weights).  block_m: the descriptor's
    segment padding (0 = library default).
    """

    def __init__(self, router, w13, w2, topk: int, n_shared: int = 0,
                 s13: Optional[torch.Tensor] = None, s2: Optional[torch.Tensor] = None,
                 device="cuda", packed: bool = False, block_m: int = 0):
        self.router = router.to(device).contiguous()
        self.w13 = w13.to(device).contiguous()
        self.w2 = w2.to(device).contiguous()
        self.s13 = None if s13 is None else s13.to(device, torch.float32).contiguous()
        self.s2 = None if s2 is None else s2.to(device, torch.float32).contiguous()
        self.E, self.H = self.router.shape
        self.n_shared = n_shared
        self.I = self.w13.shape[1] // 2
        self.topk = topk
        self.act = _ACT[self.router.dtype]
        self.wd = _W[self.w13.dtype]
        if self.wd == MOE_FP8_E4M3:
            ne, I, H = self.E + n_shared, self.I, self.H
            if self.s13 is None or tuple(self.s13.shape) != (ne, 2 * I // 128, H // 128):
                raise ValueError("fp8 weights need s13 [E+ns, 2I/128, H/128]")
            if self.s2 is None or tuple(self.s2.shape) != (ne, H // 128, I // 128):
                raise ValueError("fp8 weights need s2 [E+ns, H/128, I/128]")
        self.device = device
        self.block_m = block_m
        self._ws = {}
        self.layout = MOE_LAYOUT_ROW_MAJOR
        if packed:
            self.w13, self.w2 = moe_pack_weights(self.desc(1), self.w13, self.w2)
            self.layout = MOE_LAYOUT_FRAG16

    def desc(self, T: int):
        return make_desc(T, self.H, self.E, self.I, self.n_shared, self.act, self.wd,
                         self.s13, self.s2, block_m=self.block_m, w_layout=self.layout)

    def workspace(self, T: int) -> torch.Tensor:
        if T not in self._ws:
            self._ws[T] = alloc_workspace(self.desc(T), self.topk, self.device)
        return self._ws[T]

    def forward(self, x, valid=None, out=None, workspace=None, stream=None):
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        ws = workspace if workspace is not None else self.workspace(T)
        moe_forward(self.desc(T), x, valid, self.router, self.w13, self.w2, self.topk,
                    out, ws, stream)
        return out

    def block_signals(self, T: int) -> torch.Tensor:
        """Completion counters for forward_signaled: int32 [E+ns, ceil(T/64)]."""
        return torch.empty((self.E + self.n_shared, (T + 63) // 64), dtype=torch.int32,
                           device=self.device)

    def forward_signaled(self, x, valid=None, out=None, workspace=None, block_signal=None,
                         stream=None, consumer_stream=None):
        """forward with per-(expert, 64-row block) completion counters and the
        combine waiting on them on consumer_stream.  Returns (out, block_signal)."""
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        ws = workspace if workspace is not None else self.workspace(T)
        sig = block_signal if block_signal is not None else self.block_signals(T)
        moe_forward_signaled(self.desc(T), x, valid, self.router, self.w13, self.w2, self.topk,
                             out, ws, sig, stream, consumer_stream)
        return out, sig

    def route(self, x, valid=None, logits=False, stream=None):
        T = x.shape[0]
        ids = torch.empty((T, self.topk), dtype=torch.int32, device=x.device)
        w = torch.empty((T, self.topk), dtype=torch.float32, device=x.device)
        lg = torch.empty((T, self.E), dtype=torch.float32, device=x.device) if logits else None
        moe_route(self.desc(T), x, valid, self.router, self.topk, ids, w, lg,
                  self.workspace(T), stream)
        return ids, w, lg
