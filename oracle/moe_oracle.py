"""Plain, slow, fp64 CPU oracle of one MoE expert-layer forward pass.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the benchmark's CPU
baseline leg may call it; the HIP product path never does, and this module
shares no code with it (only the seeded input generators in `workloads/`).

What the layer computes.  The source pages name the pieces but never write the
arithmetic down, so the oracle takes the plainest reading they support:

* "Step3 Inference Optimization on AMD Instinct MI308X" (Moreh), Background:
  each MoE layer picks 3 of 48 experts per token (top-k routing).
  Optimisation list: a shared-expert MLP fused into the MoE layer (an always-on
  expert), mixed BF16 / FP8-blockscale weights, a MoE kernel tuned on the
  expert intermediate dimension ("inter_dim").
* "AMD Instinct MI355X: ATOM, kernels fusionnes et montee en charge": sparse
  MoE experts, block-scale GEMMs, fused MoE execution.
* "[SGLang] Single Batch Overlap for MoE models": the down-projection GEMM and
  the combine that sums expert outputs back per token; combine progress is
  tracked per 64-token block.
* "DP Attention and TBO for DeepSeek-V4 on MI355X" (summary), opening section:
  DP attention + TP MoE, so each GPU holds a 1/TP slice of every expert's
  intermediate dimension and its output is a partial sum for reduce_scatter;
  PrefillDelayer section: the gathered batch is padded to the largest rank.

Reading taken (each point also listed in the design notes):
  1. logits l[t,e] = sum_h x[t,h] * R[e,h]; R is [E, H] (out x in); no bias.
  2. selection on the logits rounded to fp32 (the kernel's decision precision),
     key (-l, e): descending logit, ties to the lower expert id; slots in that
     order.  weights = softmax over the k selected logits, i.e. "softmax, top-k,
     renormalise".
  3. rows with valid == 0 are never read: ids -1, weights 0, out row 0.
  4. expert e: [g; u] = W13[e] x (W13 is [2I, H], gate rows first),
     h = SiLU(g) * u with SiLU(z) = z / (1 + exp(-z)), y = W2[e] h (W2 [H, I]).
  5. out[t] = sum_j w[t,j] * y_{ids[t,j]}(x_t) + sum_s y_{E+s}(x_t) (shared
     experts always on, weight 1).
  6. fp8 weights are OCP e4m3fn codes q with one fp32 scale per 128x128 block:
     W = q * s.
Everything is computed in fp64 (library matmul as the GEMM step, no blocking
or reordering beyond it); only the routing decision is taken on fp32 logits.
"""
from __future__ import annotations

import itertools
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "e4m3fn_table", "e4m3fn_decode", "dequant_block_scaled", "to_f64",
    "router_logits", "select_topk", "topk_weights", "route", "align",
    "silu", "expert_ffn", "expert_weights_f64", "moe_forward", "near_tie_rows",
    "admissible_sets", "forward_rows_with_sets", "tie_threshold",
]


# ---------------------------------------------------------------- formats --
def e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3FN codes (NaN for the two NaNs).

    Layout s.eeee.mmm, exponent bias 7; e == 0 encodes subnormals m/8 * 2^-6;
    e == 15 with m == 7 is NaN; there is no infinity (max finite 448).
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3fn_table()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def dequant_block_scaled(codes: np.ndarray, scales: np.ndarray,
                         block: int = 128) -> np.ndarray:
    """W[r, c] = q[r, c] * s[r // block, c // block], in fp64."""
    q = e4m3fn_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    return q * np.repeat(np.repeat(s, block, axis=0), block, axis=1)


def to_f64(t) -> np.ndarray:
    """Exact widening of an fp32 / bf16 tensor (or array) to fp64."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


# ---------------------------------------------------------------- routing --
def router_logits(x64: np.ndarray, R64: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] R[e, h] (fp64)."""
    return x64 @ R64.T


def select_topk(l32_row: np.ndarray, k: int) -> List[int]:
    """The k experts with the largest logit; ties go to the lower expert id.
    Returned in slot order: descending logit, then ascending id."""
    E = l32_row.shape[0]
    order = sorted(range(E), key=lambda e: (-float(l32_row[e]), e))
    return order[:k]


def topk_weights(l_sel: Sequence[float]) -> np.ndarray:
    """Softmax over the selected logits (= softmax over all E, keep the
    top-k, renormalise to sum 1)."""
    l = np.asarray(l_sel, dtype=np.float64)
    u = np.exp(l - l.max())
    return u / u.sum()


def route(x64: np.ndarray, valid: Optional[np.ndarray], R64: np.ndarray, k: int):
    """Routing of every row: ids [T,k] int32 (-1 on padding rows), weights
    [T,k] fp64 (0 on padding rows), fp64 logits [T,E] (NaN on padding)."""
    T = x64.shape[0]
    E = R64.shape[0]
    ids = np.full((T, k), -1, dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    logits = np.full((T, E), np.nan, dtype=np.float64)
    rows = np.arange(T) if valid is None else np.nonzero(np.asarray(valid))[0]
    if rows.size:
        logits[rows] = router_logits(x64[rows], R64)
    l32 = logits.astype(np.float32)
    for t in rows:
        sel = select_topk(l32[t], k)
        ids[t] = sel
        w[t] = topk_weights(logits[t, sel])
    return ids, w, logits


# ------------------------------------------------------------------ align --
def align(ids: np.ndarray, E: int, block_m: int):
    """Stable counting sort of the flat assignments a = t*k + j by expert.

    Expert segments in ascending expert order; inside a segment, ascending a
    (= ascending token).  Each segment is padded with -1 up to a multiple of
    block_m; an expert with no assignment gets no block.  Ids of -1 (padding
    rows) are skipped.  Returns (sorted_ids, block_expert, expert_offsets
    [E+1], n_post_padded).
    """
    T, k = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e >= 0:
                counts[e] += 1
    padded = ((counts + block_m - 1) // block_m) * block_m
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    total = int(offsets[E])
    sorted_ids = np.full(total, -1, dtype=np.int32)
    cursor = offsets[:E].copy()
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e >= 0:
                sorted_ids[cursor[e]] = t * k + j
                cursor[e] += 1
    block_expert = np.repeat(np.arange(E, dtype=np.int32), padded // block_m)
    return sorted_ids, block_expert, offsets.astype(np.int32), total


# ---------------------------------------------------------------- experts --
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X: np.ndarray, W13: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """Y = W2 (SiLU(W_gate X) * (W_up X)) for a batch of rows X [n, H]."""
    I = W13.shape[0] // 2
    G = X @ W13[:I].T
    U = X @ W13[I:].T
    return (silu(G) * U) @ W2.T


def expert_weights_f64(inp, e: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 copies of expert e's W13 [2I, H] and W2 [H, I]."""
    if inp.s13 is not None:
        W13 = dequant_block_scaled(inp.w13[e].numpy(), inp.s13[e].numpy())
        W2 = dequant_block_scaled(inp.w2[e].numpy(), inp.s2[e].numpy())
    else:
        W13 = to_f64(inp.w13[e])
        W2 = to_f64(inp.w2[e])
    return W13, W2


def _valid_np(inp) -> Optional[np.ndarray]:
    return None if inp.valid is None else inp.valid.numpy().astype(bool)


def moe_forward(inp, return_routing: bool = False):
    """Full layer: out [T, H] fp64 (padding rows exactly 0)."""
    cfg = inp.cfg
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    valid = _valid_np(inp)
    rows = np.arange(T) if valid is None else np.nonzero(valid)[0]
    x64 = np.zeros((T, H), dtype=np.float64)
    if rows.size:
        x64[rows] = to_f64(inp.x[torch.from_numpy(rows)])
    R64 = to_f64(inp.router)
    ids, w, logits = route(x64, valid, R64, k)
    out = np.zeros((T, H), dtype=np.float64)
    for e in range(E + cfg.n_shared):
        if e < E:
            tok, slot = np.nonzero(ids == e)
            if tok.size == 0:
                continue
            coef = w[tok, slot]
        else:
            tok = rows
            if tok.size == 0:
                continue
            coef = np.ones(tok.size)
        W13, W2 = expert_weights_f64(inp, e)
        Y = expert_ffn(x64[tok], W13, W2)
        # a token meets a given expert at most once, so `tok` has no repeats
        out[tok] += coef[:, None] * Y
    if return_routing:
        return out, dict(ids=ids, w=w, logits=logits, x64=x64, R64=R64)
    return out


# ------------------------------------------------- several correct answers --
def tie_threshold(x64: np.ndarray, R64: np.ndarray) -> np.ndarray:
    """Per-row logit distance under which two fp32 evaluations of the logits in
    different summation orders may legitimately order two experts either way:
    2^-20 * ||x_t||_2 * max_e ||R_e||_2 (Cauchy-Schwarz bounds sum|x*R| by the
    product of norms; 2^-20 is 16 units of fp32 rounding)."""
    rn = np.sqrt((R64 * R64).sum(axis=1)).max()
    xn = np.sqrt((x64 * x64).sum(axis=1))
    return (2.0 ** -20) * xn * rn


def near_tie_rows(logits64: np.ndarray, k: int, delta: np.ndarray,
                  valid: Optional[np.ndarray] = None) -> np.ndarray:
    """Rows where two of the k+1 largest logits lie within delta of each other
    (selection or slot order may then legitimately differ)."""
    T, E = logits64.shape
    out = []
    for t in range(T):
        if valid is not None and not valid[t]:
            continue
        srt = np.sort(logits64[t])[::-1][: min(k + 1, E)]
        if np.any(np.diff(-srt) < delta[t]):
            out.append(t)
    return np.asarray(out, dtype=np.int64)


def admissible_sets(logits64_row: np.ndarray, k: int, delta: float) -> List[Tuple[int, ...]]:
    """Every k-subset that a correct fp32 evaluation could select: each
    selected logit >= each unselected one - delta.  Sorted tuples."""
    E = logits64_row.shape[0]
    l = logits64_row
    order = np.argsort(-l, kind="stable")
    kth = l[order[k - 1]]
    sure = [int(e) for e in range(E) if l[e] > kth + delta]
    cand = [int(e) for e in range(E) if abs(l[e] - kth) <= delta]
    need = k - len(sure)
    res = []
    for c in itertools.combinations(cand, need):
        s = sure + list(c)
        sel_min = min(l[s])
        uns_max = max([l[e] for e in range(E) if e not in s], default=-np.inf)
        if sel_min >= uns_max - delta:
            res.append(tuple(sorted(s)))
    return res


def forward_rows_with_sets(inp, x64: np.ndarray, logits64: np.ndarray,
                           rows: Sequence[int], sets: Sequence[Sequence[int]]) -> np.ndarray:
    """Layer output of the given rows, each routed to the given expert set
    (weights = softmax over that set's logits) plus the shared experts."""
    cfg = inp.cfg
    res = np.zeros((len(rows), cfg.H), dtype=np.float64)
    for i, (t, s) in enumerate(zip(rows, sets)):
        s = list(s)
        wts = topk_weights(logits64[t, s])
        for e, c in zip(s + list(range(cfg.E, cfg.E + cfg.n_shared)),
                        list(wts) + [1.0] * cfg.n_shared):
            W13, W2 = expert_weights_f64(inp, e)
            res[i] += c * expert_ffn(x64[t:t + 1], W13, W2)[0]
    return res
