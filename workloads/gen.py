"""Seeded synthetic inputs for the MoE layer (host tensors, CPU generator).

Recipe (every tensor has its own torch.Generator so that two workloads sharing
a layer share its weights bit for bit, whatever their batch size):

* x      ~ N(0, 1), drawn in fp32, rounded to the activation dtype (RNE).
* router ~ N(0, 0.02) or U(-sqrt(3)*0.02, +sqrt(3)*0.02) (same std).
* w13, w2 ~ N(0, 0.02), drawn expert by expert in fp32, then rounded to bf16,
  or quantised to fp8 e4m3fn per 128x128 block: s = max(amax, 1e-12)/448,
  q = RNE(w/s).  The pair (q, s) *is* the weight from then on.
* routing-bias channel (bias_max set): the last hidden column of x is 1 and the
  last column of the router holds b_e, a seeded permutation of
  linspace(0, bias_max, E); the logits then carry an additive per-expert bias,
  which skews expert loads (bias_max 1.15 gives a max/min load of about 4).
* padding rows of a gathered batch hold N(0,1) garbage (or NaN on request);
  the layer must never read them.

Layouts (row-major, K contiguous):
  x [T, H], router [E, H], w13 [E+ns, 2I, H] (gate rows 0..I-1 then up rows
  I..2I-1), w2 [E+ns, H, I], s13 [E+ns, 2I/128, H/128], s2 [E+ns, H/128, I/128].
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import LayerConfig, valid_mask

FP8_MAX = 448.0

_TAG = {"x": 0, "router": 1, "w13": 2, "w2": 3, "bias": 4}


def _gen(seed: int, tag: str) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 16 + _TAG[tag])


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def quantize_fp8_blocks(w: torch.Tensor, block: int = 128):
    """fp32 [R, C] -> (codes uint8 [R, C], scales fp32 [R/block, C/block])."""
    R, C = w.shape
    assert R % block == 0 and C % block == 0
    wb = w.reshape(R // block, block, C // block, block)
    amax = wb.abs().amax(dim=(1, 3))
    s = torch.clamp(amax, min=1e-12) / FP8_MAX
    q = (wb / s[:, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    q = q.reshape(R, C).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, s.to(torch.float32)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor                  # [T, H] act dtype
    valid: Optional[torch.Tensor]    # [T] uint8, None = all rows valid
    router: torch.Tensor             # [E, H] act dtype
    w13: torch.Tensor                # [E+ns, 2I, H] f32 / bf16 / uint8 (fp8 codes)
    w2: torch.Tensor                 # [E+ns, H, I]
    s13: Optional[torch.Tensor] = None   # fp8 block scales
    s2: Optional[torch.Tensor] = None

    @property
    def n_valid(self) -> int:
        return self.cfg.T if self.valid is None else int(self.valid.sum())


def _draw_weights(cfg: LayerConfig, tag: str, shape_per_expert):
    g = _gen(cfg.layer_seed, tag)
    n_exp = cfg.E + cfg.n_shared
    codes, scales = [], []
    for _ in range(n_exp):
        w = torch.randn(shape_per_expert, generator=g, dtype=torch.float32) * 0.02
        if cfg.w == "fp8":
            q, s = quantize_fp8_blocks(w)
            codes.append(q)
            scales.append(s)
        else:
            codes.append(w.to(_torch_dtype(cfg.w)))
    out = torch.stack(codes)
    sc = torch.stack(scales) if scales else None
    return out, sc


_LAYER_CACHE = {}


def layer_weights(cfg: LayerConfig):
    """Router and expert weights of a layer (cached per layer identity)."""
    key = (cfg.layer_seed, cfg.H, cfg.E, cfg.I, cfg.n_shared, cfg.act, cfg.w,
           cfg.router, cfg.bias_max)
    if key in _LAYER_CACHE:
        return _LAYER_CACHE[key]
    H, E = cfg.H, cfg.E
    g = _gen(cfg.layer_seed, "router")
    if cfg.router == "uniform":
        a = math.sqrt(3.0) * 0.02
        R = (torch.rand((E, H), generator=g, dtype=torch.float32) * 2 - 1) * a
    else:
        R = torch.randn((E, H), generator=g, dtype=torch.float32) * 0.02
    if cfg.bias_max is not None:
        gb = _gen(cfg.layer_seed, "bias")
        b = torch.linspace(0.0, cfg.bias_max, E)[torch.randperm(E, generator=gb)]
        R[:, H - 1] = b
    R = R.to(_torch_dtype(cfg.act))
    w13, s13 = _draw_weights(cfg, "w13", (2 * cfg.I, H))
    w2, s2 = _draw_weights(cfg, "w2", (H, cfg.I))
    res = (R, w13, s13, w2, s2)
    _LAYER_CACHE.clear()   # keep at most one layer resident (they are GBs)
    _LAYER_CACHE[key] = res
    return res


def make_x(cfg: LayerConfig, pad_fill: str = "randn"):
    """Token rows of the (sub-)batch and its validity mask."""
    full_T = cfg.full_T
    g = _gen(cfg.x_seed, "x")
    x = torch.randn((full_T, cfg.H), generator=g, dtype=torch.float32)
    if cfg.bias_max is not None:
        x[:, cfg.H - 1] = 1.0
    m = valid_mask(cfg)
    valid = None
    if m is not None:
        valid = torch.tensor(m, dtype=torch.uint8)
        if pad_fill == "nan":
            x[valid == 0] = float("nan")
    if cfg.ub is not None:
        lo = 0 if cfg.ub == 0 else full_T // 2
        hi = full_T // 2 if cfg.ub == 0 else full_T
        x = x[lo:hi]
        if valid is not None:
            valid = valid[lo:hi]
    assert x.shape[0] == cfg.T, (x.shape, cfg.T)
    return x.to(_torch_dtype(cfg.act)).contiguous(), valid


def make_inputs(cfg: LayerConfig, pad_fill: str = "randn") -> LayerInputs:
    R, w13, s13, w2, s2 = layer_weights(cfg)
    x, valid = make_x(cfg, pad_fill)
    return LayerInputs(cfg=cfg, x=x, valid=valid, router=R, w13=w13, w2=w2,
                       s13=s13, s2=s2)


def random_small(T, H, E, k, I, n_shared=0, act="bf16", w="bf16", seed=0,
                 valid_frac=1.0, router="normal", name="small") -> LayerInputs:
    """Small seeded layer for parity tests (any shape the ABI accepts)."""
    cfg = LayerConfig(name=name, T=T, H=H, E=E, k=k, I=I, n_shared=n_shared,
                      act=act, w=w, router=router, layer_seed=seed, x_seed=seed)
    R, w13, s13, w2, s2 = layer_weights(cfg)
    g = _gen(seed, "x")
    x = torch.randn((T, H), generator=g, dtype=torch.float32)
    valid = None
    if valid_frac < 1.0:
        valid = (torch.rand((T,), generator=g) < valid_frac).to(torch.uint8)
    return LayerInputs(cfg=cfg, x=x.to(_torch_dtype(act)).contiguous(), valid=valid,
                       router=R, w13=w13, w2=w2, s13=s13, s2=s2)
