"""Layer shapes of the five synthetic workloads and their row masks / splits.

The shapes stand in for the workloads the source pages describe:

* "AMD ROCm DP Attention and TBO for DeepSeek-V4 on MI355X" (summary page),
  section on PrefillDelayer: one DP rank prefills about 1024 tokens while
  seven ranks decode about 16 each, and the all_gather pads every rank to the
  largest, wasting about 86% of the gathered rows.  Section on the micro-batch
  split: 16384 tokens from requests of 7003, 6928 and 2453 tokens split at the
  request boundary give 7003 / 9381; split at the token midpoint they give
  8192 / 8192.
* "Step3 inference optimization on AMD Instinct MI308X", background section:
  56 MoE layers selecting 3 of 48 experts; results section: concurrency 256 on
  DP8 (32 decode tokens per rank).

Nothing here computes any part of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # gathered rows, padding included
    H: int                 # hidden size
    E: int                 # routed experts
    k: int                 # experts per token
    I: int                 # per-GPU (TP-sliced) expert intermediate size
    n_shared: int = 0      # always-on shared experts (0 or 1)
    act: str = "bf16"      # x / router / out dtype: "f32" | "bf16"
    w: str = "bf16"        # expert weight dtype: "f32" | "bf16" | "fp8"
    router: str = "normal"  # "normal": N(0, 0.02); "uniform": U(+-sqrt(3)*0.02)
    bias_max: Optional[float] = None  # routing-bias channel (see gen.py)
    layer_seed: int = 0
    x_seed: int = 0
    mask: str = "all"      # "all" | "dp_gather"
    dp_ranks: int = 8
    rows_per_rank: int = 0
    prefill_rank: int = 4
    decode_rows: int = 16
    requests: Tuple[int, ...] = ()   # prefill request lengths (full batch)
    ub: Optional[int] = None         # which midpoint micro-batch (0/1); None = whole batch
    description: str = ""

    @property
    def full_T(self) -> int:
        """Rows of the whole batch before any micro-batch split."""
        return sum(self.requests) if self.requests else self.T

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": LayerConfig(
        name="tiny", T=64, H=256, E=8, k=2, I=128, act="f32", w="f32",
        layer_seed=1001, x_seed=1001,
        description="T=64 H=256 E=8 top-2 I=128 fp32, all rows valid"),
    "decode_e48": LayerConfig(
        name="decode_e48", T=256, H=7168, E=48, k=3, I=640, bias_max=1.15,
        layer_seed=1002, x_seed=1002,
        description="decode share, 8 DP ranks x 32 rows, 48 experts top-3, "
                    "I=5120/8, bf16, routing bias so expert loads vary ~4x"),
    "decode_e256_shared": LayerConfig(
        name="decode_e256_shared", T=128, H=7168, E=256, k=8, I=256, n_shared=1,
        router="uniform", layer_seed=1003, x_seed=1003,
        description="decode share, 8 ranks x 16 rows, 256 experts top-8 + 1 "
                    "shared, I=2048/8, bf16"),
    "gather_padded_e48": LayerConfig(
        name="gather_padded_e48", T=8192, H=7168, E=48, k=3, I=640, bias_max=1.15,
        layer_seed=1002, x_seed=1004, mask="dp_gather", dp_ranks=8,
        rows_per_rank=1024, prefill_rank=4, decode_rows=16,
        description="mixed-phase gather: 8 ranks x 1024 padded rows, rank 4 "
                    "holds 1024 real rows, the others 16 each (1136 valid)"),
    "prefill_ub_fp8": LayerConfig(
        name="prefill_ub_fp8", T=8192, H=7168, E=256, k=8, I=256, w="fp8",
        layer_seed=1005, x_seed=1005, requests=(7003, 6928, 2453), ub=0,
        description="prefill micro-batch: 16384 tokens of requests "
                    "[7003, 6928, 2453] split at the midpoint; one 8192-row ub; "
                    "fp8 e4m3 weights with 128x128 fp32 block scales, bf16 x"),
}

# order used for reports
CONFIG_ORDER = ["tiny", "decode_e48", "decode_e256_shared", "gather_padded_e48",
                "prefill_ub_fp8"]


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]


def valid_mask(cfg: LayerConfig) -> Optional[List[int]]:
    """Row validity of the gathered batch (None = every row valid).

    dp_gather: rank r owns rows [r*R, (r+1)*R).  The prefill rank fills all R of
    its rows; every other rank fills only its first `decode_rows` rows, and the
    rest of its rows are the all_gather's padding.
    """
    if cfg.mask == "all":
        return None
    if cfg.mask == "dp_gather":
        R = cfg.rows_per_rank
        assert cfg.T == cfg.dp_ranks * R
        m = []
        for r in range(cfg.dp_ranks):
            n_real = R if r == cfg.prefill_rank else cfg.decode_rows
            m.extend([1] * n_real + [0] * (R - n_real))
        return m
    raise ValueError(cfg.mask)


def midpoint_split(total: int) -> Tuple[int, int]:
    """Two micro-batches cut at the token midpoint (first gets the floor)."""
    a = total // 2
    return a, total - a


def boundary_split(requests) -> Tuple[int, int]:
    """Prior behaviour: cut only at a request boundary, as close to the
    midpoint as possible without splitting a request, the first micro-batch
    taking whole requests until the next one would cross the midpoint."""
    total = sum(requests)
    half = total / 2
    acc = 0
    for r in requests:
        if acc + r > half and acc > 0:
            break
        acc += r
    return acc, total - acc
