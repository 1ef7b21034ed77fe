"""Helpers for GPU-vs-oracle parity: run the HIP layer, run the oracle on the
same seeded inputs, and compare under the documented rules.

Routing: ids must equal the oracle's bitwise on every valid row whose top-k+1
logits are farther apart than the fp32 re-ordering threshold; on near-tie rows
the GPU's set must be one of the oracle's admissible sets, and that row's
output is compared with the oracle's output for that same set.
Outputs: max |gpu - oracle| and nL1 = sum|gpu - oracle| / sum|oracle| over
valid rows within the tolerance of the weight dtype; padding rows exactly 0.
"""
from __future__ import annotations

import sys
import contextlib
from dataclasses import dataclass

import numpy as np
import torch

import oracle

TOL = {  # (max-abs, nL1)
    "bf16": (2e-2, 5e-3),
    "fp8": (6e-2, 1.5e-2),
    "f32": (1e-5, 1e-5),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_layer(inp, device="cuda", packed=False, block_m=0):
    from expert_layer_moe_amd import DeviceLayer
    cfg = inp.cfg
    return DeviceLayer(inp.router, inp.w13, inp.w2, cfg.k, cfg.n_shared,
                       inp.s13, inp.s2, device=device, packed=packed, block_m=block_m)


@contextlib.contextmanager
def gemm_path(min_rows=16, min_tiles=1):
    """Send segments above min_rows rows to the tiled GEMM kernels (at any
    tile count) for the duration; restores the defaults."""
    import expert_layer_moe_amd as moe
    moe.moe_set_path_thresholds(min_rows, min_tiles)
    try:
        yield
    finally:
        moe.moe_set_path_thresholds()


@contextlib.contextmanager
def fp8_mfma(enable):
    """fp8 weights on the tiled gate/up GEMM: fp8 MFMA on two-term token
    codes (True) or bf16 MFMA on dequantised weights (False), for the
    duration; restores the default.  Layers made inside size their
    workspaces for the setting."""
    import expert_layer_moe_amd as moe
    moe.moe_set_fp8_mfma(enable)
    try:
        yield
    finally:
        moe.moe_set_fp8_mfma(False)


@contextlib.contextmanager
def one_stage(enable):
    """Decode-sized batches: gate/up and down in one launch (True) or two, for
    the duration; restores the default.  Layers made inside size their
    workspaces for the setting.  (The path is switched off and the library
    does not export the switch: only skipped tests use this.)"""
    import expert_layer_moe_amd as moe
    moe.moe_set_one_stage(enable)
    try:
        yield
    finally:
        moe.moe_set_one_stage(False)


def run_gpu(inp, layer=None, x=None, valid=None):
    layer = layer or device_layer(inp)
    xd = (inp.x if x is None else x).cuda()
    vd = inp.valid if valid is None else valid
    vd = None if vd is None else vd.cuda()
    out = layer.forward(xd, vd)
    ids, w, lg = layer.route(xd, vd, logits=True)
    torch.cuda.synchronize()
    return dict(out=out.float().cpu().double().numpy(), ids=ids.cpu().numpy(),
                w=w.cpu().double().numpy(), logits=lg.cpu().double().numpy(), layer=layer)


@dataclass
class Report:
    max_abs: float
    nl1: float
    near_ties: int
    id_mismatch_rows: int
    rows: int


def compare(inp, gpu, ref=None, tol=None, strict_ids=False):
    """Full comparison; returns a Report, asserts the bars."""
    cfg = inp.cfg
    if ref is None:
        ref = oracle.moe_forward(inp, return_routing=True)
    out_ref, r = ref
    T = cfg.T
    valid = np.ones(T, bool) if inp.valid is None else inp.valid.numpy().astype(bool)
    ids_g, ids_o = gpu["ids"], r["ids"]
    delta = oracle.tie_threshold(r["x64"], r["R64"])
    if strict_ids:
        delta = np.zeros_like(delta)
    ties = set(oracle.near_tie_rows(r["logits"], cfg.k, delta, valid).tolist())
    # padding rows
    assert (ids_g[~valid] == -1).all(), "padding rows must get id -1"
    assert (gpu["w"][~valid] == 0).all()
    assert (gpu["out"][~valid] == 0).all(), "padding rows of out must be exactly 0"
    expect = out_ref.copy()
    mism = 0
    alt_rows, alt_sets = [], []
    for t in np.nonzero(valid)[0]:
        if np.array_equal(ids_g[t], ids_o[t]):
            continue
        mism += 1
        assert t in ties, f"row {t}: ids {ids_g[t]} vs oracle {ids_o[t]} outside a near tie"
        gs = tuple(sorted(ids_g[t].tolist()))
        adm = oracle.admissible_sets(r["logits"][t], cfg.k, delta[t])
        assert gs in adm, f"row {t}: gpu set {gs} not admissible {adm}"
        if gs != tuple(sorted(ids_o[t].tolist())):
            alt_rows.append(int(t))
            alt_sets.append(gs)
    if alt_rows:
        expect[alt_rows] = oracle.forward_rows_with_sets(inp, r["x64"], r["logits"],
                                                         alt_rows, alt_sets)
    # the premise of the near-tie rule: the GPU's fp32 logits lie within the
    # tie threshold of the exact ones on every valid row
    if "logits" in gpu and valid.any():
        dl_all = np.abs(gpu["logits"][valid] - r["logits"][valid]).max(axis=1)
        full_delta = oracle.tie_threshold(r["x64"], r["R64"])[valid]
        assert (dl_all <= full_delta).all(), \
            f"logit error {dl_all.max():.3e} above the tie threshold"
    # routing weights: softmax of the selected logits.  A softmax's Jacobian
    # rows sum (in absolute value) to 2 w (1 - w) <= 1/2, so |dw| <= 0.5 max
    # |dl| over the selected logits, dl being the GPU's measured logit error;
    # 2e-6 covers the fp32 exp and divide.
    same = valid & (ids_g == ids_o).all(axis=1)
    if same.any():
        rows = np.nonzero(same)[0]
        werr = np.abs(gpu["w"][rows] - r["w"][rows]).max(axis=1)
        if "logits" in gpu:
            sel = ids_o[rows]
            dl = np.abs(np.take_along_axis(gpu["logits"][rows], sel, 1) -
                        np.take_along_axis(r["logits"][rows], sel, 1)).max(axis=1)
        else:
            dl = oracle.tie_threshold(r["x64"], r["R64"])[rows]
        bound = 0.5 * dl + 2e-6
        assert (werr <= bound).all(), f"routing weights differ by {werr.max()}"
    d = np.abs(gpu["out"][valid] - expect[valid])
    max_abs = float(d.max()) if d.size else 0.0
    den = np.abs(expect[valid]).sum()
    nl1 = float(d.sum() / den) if den > 0 else 0.0
    tol = tol or TOL[cfg.w]
    rep = Report(max_abs, nl1, len(ties), mism, int(valid.sum()))
    log(f"[parity] {cfg.name} T={T} valid={rep.rows} max_abs={max_abs:.3e} "
        f"nL1={nl1:.3e} near_ties={rep.near_ties} id_mismatch_rows={mism}")
    assert max_abs <= tol[0], rep
    assert nl1 <= tol[1], rep
    return rep
