"""GPU tests of moe_forward_signaled: the down kernels' per-(expert, 64-row
block) completion counters and the combine that consumes them on a second
stream ("[SGLang] Single Batch Overlap for MoE models", combine-signal
section).  The output must be moe_forward's bit for bit wherever moe_forward
also sends its y rows through memory (the signaled call runs the same kernels
in the same summation order), and the oracle's within tolerance elsewhere;
the counters must end at exactly H for every block that holds rows and 0
for the others.  Needs an MI355X."""
import contextlib

import numpy as np
import pytest
import torch

from workloads import get_config, make_inputs
from workloads.gen import random_small

from .parity import compare, device_layer, gemm_path, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_layer_moe_amd as moe
    moe.load_library()
    yield


def _expected_signals(layer, ids, valid_rows, T):
    """H for each 64-row block of each segment that holds rows, else 0: the
    segment sizes are the expert histogram of the routed ids (and every
    valid row for the shared expert)."""
    nb64 = (T + 63) // 64
    exp = np.zeros((layer.E + layer.n_shared, nb64), dtype=np.int64)
    ids = ids.cpu().numpy()
    cnt = np.bincount(ids[ids >= 0].ravel(), minlength=layer.E)
    if layer.n_shared:
        cnt = np.append(cnt, int((ids[:, 0] >= 0).sum()))
    for e, c in enumerate(cnt):
        exp[e, :(int(c) + 63) // 64] = layer.H
    return exp


def _run_signaled(layer, xd, vd, consumer=True):
    """One signaled call, the combine on its own stream (or on the caller's),
    and the routing of the same rows."""
    cs = torch.cuda.Stream() if consumer else None
    out, sig = layer.forward_signaled(xd, vd, consumer_stream=cs)
    ids, _, _ = layer.route(xd, vd)
    torch.cuda.synchronize()
    return out, sig, ids


# layers where moe_forward writes the y rows to memory too (more than 1216
# assignments, or a tiled GEMM that may run): every down kernel that raises
# counters, both y formats of bf16 weights, fp8, the shared expert
BITWISE = [
    # all streaming, 24-bit y rows
    (dict(T=1300, H=256, E=8, k=2, I=128, valid_frac=0.8), "auto"),
    # tiled bf16 down (I = 128) beside streaming segments, shared expert
    (dict(T=1300, H=256, E=8, k=2, I=128, n_shared=1), "gemm"),
    # fp8: streaming down with bf16 y rows, then the tiled fp8 down (I = 256)
    (dict(T=700, H=512, E=6, k=2, I=256, w="fp8", valid_frac=0.7), "auto"),
    (dict(T=400, H=512, E=4, k=2, I=256, w="fp8"), "gemm"),
    # the general tiled down GEMM (I a multiple of 128 other than 128, 256)
    (dict(T=300, H=256, E=4, k=2, I=384), "gemm"),
    (dict(T=300, H=256, E=4, k=2, I=384, w="fp8"), "gemm"),
    (dict(T=260, H=384, E=5, k=2, I=640, n_shared=1), "gemm"),
    # H not a multiple of 256: the last streaming column group half used
    (dict(T=2100, H=8320, E=8, k=2, I=64, valid_frac=0.6), "auto"),
]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kw,path", BITWISE)
def test_signaled_forward_is_forward_bitwise(kw, path, packed):
    inp = random_small(seed=131, **kw)
    log(f"[case] signaled vs forward packed={packed} path={path}: {kw}")
    layer = device_layer(inp, packed=packed)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    with gemm_path() if path == "gemm" else contextlib.nullcontext():
        ref = layer.forward(xd, vd)
        torch.cuda.synchronize()
        out, sig, ids = _run_signaled(layer, xd, vd)
    assert torch.equal(out, ref), float((out.float() - ref.float()).abs().max())
    exp = _expected_signals(layer, ids, vd, xd.shape[0])
    assert np.array_equal(sig.cpu().numpy(), exp)


# decode-sized layers: moe_forward keeps y on chip (one launch for down +
# combine), the signaled call sends it through memory, so the comparison is
# with the oracle
SMALL = [
    dict(T=70, H=256, E=8, k=2, I=64),
    dict(T=90, H=256, E=6, k=2, I=128, w="fp8"),
    dict(T=100, H=512, E=16, k=4, I=96, n_shared=1, valid_frac=0.7),
]


@pytest.mark.parametrize("kw", SMALL)
def test_signaled_small_layers_match_oracle(kw):
    inp = random_small(seed=137, **kw)
    log(f"[case] signaled small layer: {kw}")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    out, sig, ids = _run_signaled(layer, xd, vd)
    gpu = run_gpu(inp, layer)
    gpu["out"] = out.float().cpu().double().numpy()
    compare(inp, gpu)
    assert np.array_equal(sig.cpu().numpy(), _expected_signals(layer, ids, vd, xd.shape[0]))


@pytest.mark.parametrize("block_m", [64, 256])
def test_signaled_block_m_is_forward_bitwise(block_m):
    """Larger segment padding in the sorted list moves the segment starts;
    the counters index blocks from each segment's start either way."""
    kw = dict(T=1300, H=256, E=8, k=2, I=128, n_shared=1, valid_frac=0.8)
    inp = random_small(seed=157, **kw)
    log(f"[case] signaled block_m={block_m}: {kw}")
    layer = device_layer(inp, packed=True, block_m=block_m)
    xd = inp.x.cuda()
    vd = inp.valid.cuda()
    with gemm_path():
        ref = layer.forward(xd, vd)
        torch.cuda.synchronize()
        out, sig, ids = _run_signaled(layer, xd, vd)
    assert torch.equal(out, ref)
    assert np.array_equal(sig.cpu().numpy(), _expected_signals(layer, ids, vd, xd.shape[0]))


def test_signaled_on_one_stream():
    """consumer_stream = stream: the waits find every block complete."""
    kw = dict(T=1300, H=256, E=8, k=2, I=128, n_shared=1)
    inp = random_small(seed=139, **kw)
    log(f"[case] signaled on one stream: {kw}")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    ref = layer.forward(xd)
    out, sig, ids = _run_signaled(layer, xd, None, consumer=False)
    assert torch.equal(out, ref)
    assert np.array_equal(sig.cpu().numpy(), _expected_signals(layer, ids, None, xd.shape[0]))


def test_rest_pass_takes_the_rows_a_wait_left():
    """A zero wait bound: every wait that does not find its blocks complete at
    once gives up, and the rest pass on the caller's stream combines those
    rows; the bits do not change."""
    import expert_layer_moe_amd as moe
    kw = dict(T=1300, H=256, E=8, k=2, I=128, valid_frac=0.9)
    inp = random_small(seed=149, **kw)
    log(f"[case] signaled with a zero wait bound: {kw}")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = inp.valid.cuda()
    with gemm_path():
        ref = layer.forward(xd, vd)
        moe.moe_set_signal_wait_us(0)
        try:
            outs = [_run_signaled(layer, xd, vd)[0] for _ in range(3)]
        finally:
            moe.moe_set_signal_wait_us(10000)
    for o in outs:
        assert torch.equal(o, ref)


@pytest.mark.parametrize("name", ["gather_padded_e48", "prefill_ub_fp8"])
def test_signaled_workloads_are_forward_bitwise(name):
    """The padded mixed-phase gather (streaming down) and the prefill
    micro-batch (tiled fp8 down) at full size, the combine on its own stream."""
    cfg = get_config(name)
    log(f"[case] signaled {name}: generating inputs")
    inp = make_inputs(cfg)
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    log(f"[case] signaled {name}: GPU runs")
    ref = layer.forward(xd, vd)
    torch.cuda.synchronize()
    for _ in range(2):
        out, sig, ids = _run_signaled(layer, xd, vd)
        assert torch.equal(out, ref)
    assert np.array_equal(sig.cpu().numpy(), _expected_signals(layer, ids, vd, xd.shape[0]))


def test_signaled_forward_replays_in_a_hip_graph():
    """The signaled call forks the consumer stream off the caller's and joins
    it back with events, so it captures into one graph; every replay matches
    the eager call bit for bit."""
    kw = dict(T=1300, H=256, E=8, k=2, I=128, w="fp8", n_shared=1)
    inp = random_small(seed=151, **kw)
    log(f"[case] signaled graph capture: {kw}")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    cs = torch.cuda.Stream()
    out = torch.empty_like(xd)
    sig = layer.block_signals(xd.shape[0])
    ws = layer.workspace(xd.shape[0])
    ref, _ = layer.forward_signaled(xd, None, workspace=ws, block_signal=sig, consumer_stream=cs)
    ref = ref.clone()
    sig_ref = sig.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward_signaled(xd, None, out=out, workspace=ws, block_signal=sig,
                               consumer_stream=cs)
    for i in range(3):
        out.fill_(float("nan"))
        sig.fill_(-1)
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        assert torch.equal(sig, sig_ref), f"replay {i}"
        assert torch.isfinite(junk)
