"""Benchmark of the MoE expert-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one moe_forward (router, top-k, align, gate/up GEMM + SiLU*mul,
down GEMM, combine) over one batch of synthetic input already resident in
HBM.  The headline workload is the 48-expert top-3 decode share (256
gathered tokens, hidden 7168, inter 5120/8, bf16): its K timed steps give the
top-level figures.  By default (--config all) the same run then measures
every other workload with its own step count and nests the results under
"workloads": the 256-expert decode share with a shared expert, the padded
mixed-phase gather, the 8192-row prefill micro-batch with fp8 weights (the
MFMA-bound half of the metric), the two micro-batches on two HIP streams,
the unsplit 16384-row batch and the request-boundary split (7003 / 9381),
the tiny fp32 correctness layer, the gather and the prefill micro-batch
through moe_forward_signaled (per-(expert, 64-row block) completion counters
from the down kernels, the combine consuming them on a second stream), and
the two decode workloads with the gate/up and the down in one launch, and the
prefill micro-batch with its gate/up GEMM on the fp8 MFMA (token rows as two
e4m3 terms, moe_set_fp8_mfma).
Prints one JSON line.

Other modes (profiling runs; the default run takes none of them):
  --config NAME       only that workload (tiny, decode_e48, decode_e256_shared,
                      gather_padded_e48, prefill_ub_fp8, prefill_pair_fp8,
                      prefill_unsplit, prefill_boundary_split,
                      gather_padded_e48_signaled, prefill_ub_fp8_signaled,
                      decode_e48_one_launch, decode_e256_shared_one_launch,
                      prefill_ub_fp8_fp8_mfma)
  --no-cpu-baseline   skip the oracle timing
  --copy-calibrate    time a plain 1 GiB device copy (for counter scaling)
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import re
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s per MI355X + % of HBM-BW (decode) / MFMA peak (prefill)"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
CSRC = os.path.join(ROOT, "expert_layer_moe_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

# the headline workload, and the others measured in the same run
HEADLINE = "decode_e48"
NESTED = ["decode_e256_shared", "gather_padded_e48", "prefill_ub_fp8", "prefill_pair_fp8",
          "prefill_unsplit", "prefill_boundary_split", "tiny",
          "gather_padded_e48_signaled", "prefill_ub_fp8_signaled",
          "decode_e48_one_launch", "decode_e256_shared_one_launch", "prefill_ub_fp8_fp8_mfma"]
# workloads run through moe_forward_signaled: the down kernels raise
# per-(expert, 64-row block) completion counters and the combine consumes
# them on a second stream
SIGNALED = "_signaled"
# workloads run with the gate/up and down in one launch (moe_set_one_launch)
ONE_LAUNCH = "_one_launch"
# fp8-weight workloads whose gate/up GEMM runs on the fp8 MFMA with the token
# rows as two e4m3 terms (moe_set_fp8_mfma)
FP8_MFMA = "_fp8_mfma"
# the fp8-MFMA switch as the command line sets it for the whole run (a
# workload that turns it on for its own calls turns it back to this)
RUN_FP8_MFMA = [False]
# two-call variants of the prefill workload: (first rows, second rows)
PREFILL_SPLITS = {"prefill_pair_fp8": "midpoint", "prefill_boundary_split": "boundary"}


# sources that define each timed kernel (counter records name this hash)
KERNEL_SOURCES = {"gate_up": ("experts.hip", "moe_common.h"),
                  "gate_up_gemm": ("gemm.hip", "moe_common.h")}


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed, so
    that the hash follows the code and not its commentary."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(kernel: str = "gate_up") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def compute_dtype(cfg, fp8_mfma=False) -> str:
    """The arithmetic type of the expert GEMMs: fp32 FMA for fp32 layers,
    bf16 MFMA (fp32 accumulation) otherwise; fp8 weights are converted to
    bf16 on the way in, except with fp8_mfma, where the gate/up GEMM runs on
    the fp8 MFMA (two e4m3 token terms) and the rest in bf16."""
    if cfg.act == "f32":
        return "f32"
    return "fp8+bf16" if fp8_mfma and cfg.w == "fp8" else "bf16"


def algorithmic_work(cfg, ids, n_valid):
    """Per-call algorithmic bytes / flops of the expert kernels and of the
    whole step: weights of touched experts only, valid rows only."""
    import numpy as np
    E, H, I, ns = cfg.E, cfg.H, cfg.I, cfg.n_shared
    wb = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.w]
    ab = 4 if cfg.act == "f32" else 2
    touched = len(set(int(e) for e in np.unique(ids) if e >= 0)) + (ns if n_valid else 0)
    n_assign = n_valid * (cfg.k + ns)
    sc13 = sc2 = 0
    if cfg.w == "fp8":
        sc13 = touched * (2 * I // 128) * (H // 128) * 4
        sc2 = touched * (H // 128) * (I // 128) * 4
    w13 = touched * 2 * I * H * wb + sc13
    w2 = touched * H * I * wb + sc2
    x_bytes = n_valid * H * ab
    out_bytes = cfg.T * H * ab
    r_bytes = E * H * ab
    return dict(
        touched_experts=touched,
        gate_up_bytes=w13 + x_bytes,
        gate_up_flops=2.0 * n_assign * H * 2 * I,
        down_bytes=w2,
        down_flops=2.0 * n_assign * I * H,
        step_bytes=w13 + w2 + x_bytes + out_bytes + r_bytes,
        step_flops=2.0 * n_valid * H * E + 2.0 * n_assign * 3 * H * I,
    )


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": affinity, "cpu_model": model,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(inp, min_s=10.0, max_s=30.0):
    """The oracle, as it stands, on the host cores (bounded sample)."""
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    cfg = inp.cfg
    sample = inp
    desc = f"whole {cfg.name} batch ({inp.n_valid} valid rows)"
    if cfg.T > 1024:
        from workloads.gen import LayerInputs
        n = 512
        sample = LayerInputs(cfg=cfg.with_(T=n), x=inp.x[:n],
                             valid=None if inp.valid is None else inp.valid[:n],
                             router=inp.router, w13=inp.w13, w2=inp.w2,
                             s13=inp.s13, s2=inp.s2)
        desc = f"first {n} rows of the {cfg.name} batch ({sample.n_valid} valid)"
    # repeated runs for about 10-30 s of host work (at least 3 runs)
    times = []
    start = time.time()
    while True:
        t0 = time.perf_counter()
        oracle.moe_forward(sample)
        times.append(time.perf_counter() - t0)
        spent = time.time() - start
        if (spent >= min_s and len(times) >= 3) or spent + times[-1] > max_s:
            break
    t = sorted(times)[len(times) // 2]
    res = {"value": round(sample.n_valid / t, 2), "unit": "tokens/s",
           "cores": int(threads), "kind": "oracle",
           "sample": f"{desc}; median of {len(times)} runs, {t:.2f} s each; "
                     f"fp64 numpy oracle, its BLAS pool on {threads} threads"}
    res.update(host_info())
    return res


def traffic_for(kernel: str, workload: str):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kernel}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_steps(step, n):
    """Milliseconds per step over n steps, between synchronisations."""
    import torch
    a, b = _events()
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


class Workload:
    """One workload made resident on the GPU: the layer (weights re-laid out
    once at load time unless row_major), its inputs, outputs, workspaces and
    the step that the timed region repeats."""

    def __init__(self, name, row_major=False):
        import torch
        import expert_layer_moe_amd as moe
        from workloads import get_config, make_inputs
        from workloads.configs import boundary_split, midpoint_split

        self.name = name
        self.signaled = name.endswith(SIGNALED)
        self.one_launch = name.endswith(ONE_LAUNCH)
        self.fp8_mfma = name.endswith(FP8_MFMA)
        bname = name[:-len(SIGNALED)] if self.signaled else name
        bname = bname[:-len(ONE_LAUNCH)] if self.one_launch else bname
        bname = bname[:-len(FP8_MFMA)] if self.fp8_mfma else bname
        self.split = PREFILL_SPLITS.get(bname)
        whole = bname in ("prefill_unsplit",) or self.split is not None
        base = get_config("prefill_ub_fp8" if whole else bname)
        self.cfg = base.with_(T=base.full_T, ub=None) if whole else base
        if self.fp8_mfma and self.cfg.w != "fp8":
            raise ValueError(f"{name}: the fp8 MFMA path needs fp8 weights")
        log(f"[bench] generating {name}")
        self.inp = make_inputs(self.cfg)
        self.packed = self.cfg.w != "f32" and not row_major
        c = self.cfg
        self.layer = moe.DeviceLayer(self.inp.router, self.inp.w13, self.inp.w2, c.k,
                                     c.n_shared, self.inp.s13, self.inp.s2, packed=self.packed)
        self.x = self.inp.x.cuda()
        self.valid = None if self.inp.valid is None else self.inp.valid.cuda()
        self.out = torch.empty_like(self.x)
        self.n_valid = self.inp.n_valid
        if self.split is None:
            self.parts = None
            # the switch is read when the plan is made: a workspace sized with
            # it on holds the two-term token planes
            with self._switches():
                self.ws = self.layer.workspace(c.T)
            if self.signaled:
                self.sig = self.layer.block_signals(c.T)
                self.consumer = torch.cuda.Stream()
        else:
            a, b = (midpoint_split(c.T) if self.split == "midpoint"
                    else boundary_split(list(base.requests)))
            self.parts = []
            for lo, n in ((0, a), (a, b)):
                ws = torch.empty_like(self.layer.workspace(n))
                self.parts.append((self.x[lo:lo + n], self.out[lo:lo + n], ws,
                                   torch.cuda.Stream()))
            self.rows = (a, b)
        ids, _, _ = self.layer.route(self.x, self.valid)
        torch.cuda.synchronize()
        self.work = algorithmic_work(c, ids.cpu().numpy(), self.n_valid)

    @contextlib.contextmanager
    def _switches(self):
        """The library's process-wide path switches this workload runs with,
        on for the duration of one call and off again after it."""
        import expert_layer_moe_amd as moe
        if self.one_launch:
            moe.moe_set_one_launch(True)
        if self.fp8_mfma:
            moe.moe_set_fp8_mfma(True)
        try:
            yield
        finally:
            if self.one_launch:
                moe.moe_set_one_launch(False)
            if self.fp8_mfma:
                moe.moe_set_fp8_mfma(RUN_FP8_MFMA[0])

    def step(self):
        import torch
        if self.parts is None:
            if self.signaled:
                self.layer.forward_signaled(self.x, self.valid, self.out, self.ws, self.sig,
                                            consumer_stream=self.consumer)
            else:
                with self._switches():
                    self.layer.forward(self.x, self.valid, self.out, self.ws)
            return
        cur = torch.cuda.current_stream()
        ev = torch.cuda.Event()
        ev.record(cur)
        for xx, oo, ww, s in self.parts:
            s.wait_event(ev)
            with torch.cuda.stream(s):
                self.layer.forward(xx, None, oo, ww, stream=s)
        for _, _, _, s in self.parts:
            cur.wait_stream(s)

    def free(self):
        import torch
        del self.layer, self.x, self.out, self.parts, self.inp
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def dominant_kernel(wl):
    """Which gate/up kernel carries the work (weight-streaming or tiled GEMM),
    from one untimed step with both bracketed."""
    import torch
    import expert_layer_moe_amd as moe
    moe.moe_profile_enable(["gate_up", "gate_up_gemm"])
    wl.step()
    torch.cuda.synchronize()
    moe.moe_profile_enable(None)
    probe = moe.moe_profile_read()
    return "gate_up_gemm" if probe["gate_up_gemm"][0] > probe["gate_up"][0] else "gate_up"


def roofline(wl, dom, avg_s):
    """The dominant kernel against its roofline: its arithmetic intensity
    against the 312.5 flop/B bf16 ridge decides HBM or MFMA."""
    w = wl.work
    ai = w["gate_up_flops"] / w["gate_up_bytes"]
    if ai > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
        # a GEMM on the fp8 MFMA is priced against the fp8 peak (its
        # algorithmic flops, not the two terms' issued ones)
        peak = PEAK_FP8_TFLOPS if wl.fp8_mfma else PEAK_BF16_TFLOPS
        ach = w["gate_up_flops"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    else:
        ach = w["gate_up_bytes"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4)}
    roof["kernel"] = dom
    roof["kernel_avg_us"] = round(avg_s * 1e6, 2)
    # counters are stored per workload shape: a split or unsplit variant of
    # the prefill batch has none of its own
    roof["traffic"] = traffic_for(dom, wl.name) if wl.name == wl.cfg.name else None
    return roof


def step_fractions(wl, ms):
    s = ms / 1e3
    w = wl.work
    return {"algorithmic_GB": round(w["step_bytes"] / 1e9, 4),
            "algorithmic_GFLOP": round(w["step_flops"] / 1e9, 2),
            "hbm_frac": round(w["step_bytes"] / s / 1e9 / PEAK_HBM_GBPS, 4),
            "mfma_frac": round(w["step_flops"] / s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "touched_experts": w["touched_experts"]}


def config_of(wl):
    c = wl.cfg
    cfg = {"workload": wl.name, "T": c.T, "valid_rows": wl.n_valid, "H": c.H, "E": c.E,
           "topk": c.k, "I": c.I, "n_shared": c.n_shared, "weights": c.w,
           "weight_layout": "frag16" if wl.packed else "row_major",
           "two_streams": wl.parts is not None}
    if wl.signaled:
        cfg["block_signals"] = True
    if wl.one_launch:
        cfg["one_launch_gate_up_down"] = True
    if c.w == "fp8":
        cfg["fp8_gate_up_gemm"] = "fp8_mfma_two_term" if wl.fp8_mfma else "bf16_mfma"
    if wl.parts is not None:
        cfg["calls_rows"] = list(wl.rows)
    return cfg


def stage_breakdown(wl, steps):
    """Per-stage average microseconds, every stage bracketed by events (a
    separate pass: the events perturb the timeline)."""
    import torch
    import expert_layer_moe_amd as moe
    moe.moe_profile_enable("all")
    for _ in range(steps):
        wl.step()
    torch.cuda.synchronize()
    moe.moe_profile_enable(None)
    st = moe.moe_profile_read()
    return {k: round(v[0] / max(v[1], 1) * 1e3, 2) for k, v in st.items() if v[1]}


def measure_nested(name, steps, warmup):
    """Compact record of one non-headline workload."""
    import torch
    import expert_layer_moe_amd as moe
    wl = Workload(name)
    for _ in range(warmup):
        wl.step()
    ms = time_steps(wl.step, steps)
    rec = {"ms_per_step": round(ms, 5), "tokens_per_s": round(wl.n_valid / (ms / 1e3), 1),
           "steps": steps, "warmup": warmup, "dtype": compute_dtype(wl.cfg, wl.fp8_mfma),
           "config": config_of(wl)}
    rec["step"] = step_fractions(wl, ms)
    if wl.one_launch:
        # gate/up and down share one kernel: no gate/up kernel of its own
        rec["stages_us"] = stage_breakdown(wl, steps)
    elif wl.parts is None and wl.cfg.act != "f32":
        dom = dominant_kernel(wl)
        moe.moe_profile_enable([dom])
        for _ in range(steps):
            wl.step()
        torch.cuda.synchronize()
        moe.moe_profile_enable(None)
        d_ms, d_n = moe.moe_profile_read()[dom]
        rec["roofline"] = roofline(wl, dom, d_ms / max(d_n, 1) / 1e3)
        rec["stages_us"] = stage_breakdown(wl, steps)
    wl.free()
    log(f"[bench] {name}: {rec['ms_per_step']} ms/step")
    return rec


def run_headline(args, name):
    """The workload of the top-level figures: K timed steps (the dominant
    kernel's launch bracketed by events in every fourth), then a breakdown
    pass, an event-free pass and a HIP-graph pass."""
    import torch
    import expert_layer_moe_amd as moe

    wl = Workload(name, row_major=args.row_major)
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    dom = (dominant_kernel(wl)
           if wl.parts is None and wl.cfg.act != "f32" and not wl.one_launch else None)

    # timed region: K steps; on the launch stream, a HIP event pair brackets
    # the dominant kernel's launch (and nothing else) in every EVERY-th step,
    # which samples its average duration while perturbing the timeline less
    # than a pair around every launch
    every = 4 if args.steps >= 8 else 1
    t0, t1 = _events()
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        if dom:
            moe.moe_profile_enable([dom] if i % every == 0 else None)
        wl.step()
    t1.record()
    torch.cuda.synchronize()
    moe.moe_profile_enable(None)
    ms_total = t0.elapsed_time(t1)
    dom_rec = moe.moe_profile_read()
    ms_step = ms_total / args.steps

    res = {
        "metric": METRIC, "value": round(wl.n_valid / (ms_step / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": compute_dtype(wl.cfg, wl.fp8_mfma or args.fp8_mfma), "data": "synthetic",
        "config": config_of(wl),
    }
    if args.gemm_min_rows is not None:
        res["config"]["gemm_thresholds"] = [args.gemm_min_rows, args.gemm_min_tiles]
    if wl.cfg.w == "fp8":
        res["config"]["fp8_gate_up_gemm"] = ("fp8_mfma_two_term" if args.fp8_mfma or wl.fp8_mfma
                                             else "bf16_mfma")
    if dom:
        g_ms, g_n = dom_rec[dom]
        roof = roofline(wl, dom, g_ms / max(g_n, 1) / 1e3)
        roof["launches_timed"] = int(g_n)
        res["roofline"] = roof
        res["stages_us"] = stage_breakdown(wl, args.steps)
    ms_clean = time_steps(wl.step, args.steps)
    res["step"] = step_fractions(wl, ms_step)
    res["step"]["ms_per_step_without_events"] = round(ms_clean, 5)
    res["event_overhead_pct"] = round(100.0 * (ms_step - ms_clean) / ms_clean, 2)

    # HIP-graph pass: the step (both streams for a split batch) captured once
    # and replayed K times; moe_forward only enqueues kernels, so it captures
    res["graph_replay"] = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            wl.step()
        g.replay()
        ms_g = time_steps(g.replay, args.steps)
        res["graph_replay"] = {"ms_per_step": round(ms_g, 5),
                               "tokens_per_s": round(wl.n_valid / (ms_g / 1e3), 1)}
        del g
    res["source_sha"] = source_sha(dom or "gate_up")
    res["cpu_baseline"] = None
    if args.cpu_baseline and wl.parts is None:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(wl.inp)
    wl.free()
    return res


def run(args):
    import torch
    import expert_layer_moe_amd as moe

    moe.load_library()
    if args.gemm_min_rows is not None:
        moe.moe_set_path_thresholds(args.gemm_min_rows, args.gemm_min_tiles)
    if args.fp8_mfma:
        RUN_FP8_MFMA[0] = True
        moe.moe_set_fp8_mfma(True)
    if args.copy_calibrate:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return
    if args.config == "all":
        res = run_headline(args, HEADLINE)
        nested = {}
        for name in NESTED:
            prefill = name.startswith("prefill")
            nested[name] = measure_nested(name, steps=10 if prefill else 20, warmup=3)
        res["workloads"] = nested
    else:
        res = run_headline(args, args.config)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all",
                    help="all (the headline workload, then every other one nested), "
                         "or one workload name")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--copy-calibrate", action="store_true")
    ap.add_argument("--gemm-min-rows", type=int, default=None,
                    help="segments above this many rows may take the tiled GEMM kernels")
    ap.add_argument("--gemm-min-tiles", type=int, default=-1,
                    help="... once their 128-row tiles number this many (-1: fill the chip)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay pass")
    ap.add_argument("--fp8-mfma", action="store_true",
                    help="fp8 weights on the tiled gate/up GEMM: fp8 MFMA on two-term token "
                         "codes instead of bf16 MFMA on dequantised weights")
    ap.add_argument("--row-major", action="store_true",
                    help="time the expert weights in the row-major layout they are handed over in")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the layer on one GPU (asked for --gpus {args.gpus}): "
              "each GPU of a TP-MoE group runs this same per-GPU share, and the "
              "cross-GPU reduce_scatter is outside the measured path",
              file=sys.stderr)
        sys.exit(2)
    valid = ["all", HEADLINE] + NESTED
    if args.config not in valid:
        ap.error(f"--config must be one of {valid}")
    run(args)


if __name__ == "__main__":
    main()
