"""GPU tests of the one-launch gate/up + down (moe_set_one_launch): the
streaming kernels' units taken in ticket order by one launch, the down units
waiting on per-item counts of finished gate/up units ("Step3 Inference
Optimization on AMD Instinct MI308X", optimisation list: the MoE one-stage
kernel).  The same unit code in the same order gives the two-launch path's
bits wherever that path also writes y rows (more than 1216 assignments),
moe_forward_signaled's bits on decode-sized calls (which send y through
memory too), and the oracle's values within tolerance.  Needs an MI355X."""
import contextlib

import numpy as np
import pytest
import torch

from workloads import get_config, make_inputs
from workloads.gen import random_small

from .parity import compare, device_layer, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_layer_moe_amd as moe
    moe.load_library()
    yield


@contextlib.contextmanager
def one_launch(enable=True):
    import expert_layer_moe_amd as moe
    moe.moe_set_one_launch(enable)
    try:
        yield
    finally:
        moe.moe_set_one_launch(False)


# every segment streams, more than 1216 assignments: the two-launch path
# writes 24-bit y rows too
BITWISE = [
    dict(T=1300, H=512, E=8, k=2, I=128, valid_frac=0.8),
    dict(T=700, H=1024, E=6, k=2, I=256, n_shared=1),
    dict(T=2000, H=512, E=64, k=4, I=384, valid_frac=0.6),
]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kw", BITWISE)
def test_one_launch_is_two_launches_bitwise(kw, packed):
    inp = random_small(seed=171, **kw)
    log(f"[case] one launch vs two packed={packed}: {kw}")
    layer = device_layer(inp, packed=packed)
    ref = run_gpu(inp, layer)
    with one_launch():
        gpu = run_gpu(inp, layer)
    assert np.array_equal(gpu["out"], ref["out"])
    compare(inp, gpu)


SMALL = [
    dict(T=64, H=512, E=16, k=3, I=128),
    dict(T=100, H=512, E=16, k=4, I=128, n_shared=1, valid_frac=0.7),
    dict(T=1, H=1024, E=4, k=1, I=128),
    dict(T=40, H=512, E=64, k=8, I=256, n_shared=1),
]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kw", SMALL)
def test_one_launch_small_layers(kw, packed):
    """Decode-sized calls: the oracle's values, and the signaled call's bits
    (both send the y rows through memory)."""
    inp = random_small(seed=173, **kw)
    log(f"[case] one launch small packed={packed}: {kw}")
    layer = device_layer(inp, packed=packed)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    sig_out, _ = layer.forward_signaled(xd, vd)
    with one_launch():
        gpu = run_gpu(inp, layer)
    assert np.array_equal(gpu["out"], sig_out.float().cpu().double().numpy())
    compare(inp, gpu)


@pytest.mark.parametrize("name", ["decode_e48", "decode_e256_shared"])
def test_one_launch_decode_workloads(name):
    cfg = get_config(name)
    log(f"[case] one launch {name}: generating inputs")
    inp = make_inputs(cfg)
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    sig_out, _ = layer.forward_signaled(xd, None)
    log(f"[case] one launch {name}: GPU runs")
    with one_launch():
        gpu = run_gpu(inp, layer)
        again = layer.forward(xd)           # counters and flags reset by every call
    torch.cuda.synchronize()
    assert np.array_equal(gpu["out"], sig_out.float().cpu().double().numpy())
    assert torch.equal(again, sig_out)
    log(f"[case] one launch {name}: oracle")
    compare(inp, gpu)


def test_one_launch_rest_pass_takes_the_units_a_wait_left():
    """A zero wait bound: down units whose item is not finished when they
    look give up and the rest pass runs them; the bits do not change."""
    import expert_layer_moe_amd as moe
    kw = dict(T=1300, H=512, E=8, k=2, I=128, valid_frac=0.8)
    inp = random_small(seed=179, **kw)
    log(f"[case] one launch with a zero wait bound: {kw}")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = inp.valid.cuda()
    ref = layer.forward(xd, vd)
    with one_launch():
        moe.moe_set_signal_wait_us(0)
        try:
            outs = [layer.forward(xd, vd).clone() for _ in range(3)]
        finally:
            moe.moe_set_signal_wait_us(10000)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_one_launch_replays_in_a_hip_graph():
    inp = random_small(seed=181, T=256, H=512, E=16, k=3, I=128, valid_frac=0.9)
    log("[case] one launch graph capture")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = inp.valid.cuda()
    with one_launch():
        ref = layer.forward(xd, vd)
        out = torch.empty_like(ref)
        ws = layer.workspace(xd.shape[0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(xd, vd, out=out, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        assert torch.isfinite(junk)


def _random_shape(seed):
    """A seeded shape the one launch takes (bf16, H % 512 == 0, I % 128 == 0)."""
    r = np.random.default_rng(2000 + seed)
    E = int(r.choice([1, 3, 8, 13, 48, 64, 200]))
    return dict(T=int(r.choice([1, 5, 33, 100, 257, 700, 1500])), H=int(r.choice([512, 1024, 1536])),
                E=E, k=int(r.integers(1, min(8, E) + 1)), I=int(r.choice([128, 256, 384])),
                n_shared=int(r.integers(2)), valid_frac=float(r.choice([1.0, 0.75, 0.3])))


@pytest.mark.parametrize("seed", range(8))
def test_one_launch_random_shapes(seed):
    """Seeded random shapes: the oracle's values, the same bits on a second
    call, and the signaled call's bits (y through memory on both)."""
    kw = _random_shape(seed)
    inp = random_small(seed=190 + seed, **kw)
    log(f"[case] one launch random seed={seed}: {kw}")
    layer = device_layer(inp, packed=bool(seed % 2))
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    sig_out, _ = layer.forward_signaled(xd, vd)
    with one_launch():
        gpu = run_gpu(inp, layer)
        again = layer.forward(xd, vd)
    torch.cuda.synchronize()
    assert np.array_equal(gpu["out"], again.float().cpu().double().numpy())
    compare(inp, gpu)
    if not _may_tile(kw):
        # every segment streams in both calls: the same units, the same bits
        assert torch.equal(again, sig_out)


def _may_tile(kw):
    """Whether the tiled GEMM may take segments of this call (the library's
    rule: some segment above 128 rows, and enough 128-row tiles to fill the
    chip at I / 128 blocks each)."""
    T, kk, I = kw["T"], kw["k"] + kw["n_shared"], kw["I"]
    min_tiles = (256 + I // 128 - 1) // (I // 128)
    bound = T * kk // 128 + T * kk // 129 + 1
    return T > 128 and bound >= min_tiles


def test_one_launch_in_the_fixed_scratch():
    """moe_forward_noalloc takes the one launch too (its counters live in the
    scratch like every other workspace part): the bits of moe_forward under
    the same switch, on two calls in a row, the second smaller."""
    import expert_layer_moe_amd as moe
    inp = random_small(seed=199, T=300, H=512, E=16, k=3, I=128, n_shared=1, valid_frac=0.8)
    log("[case] one launch in the fixed scratch")
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = inp.valid.cuda()
    with one_launch():
        for rows in (300, 97):
            x, v = xd[:rows].contiguous(), vd[:rows].contiguous()
            ref = layer.forward(x, v)
            got = torch.full_like(x, float("nan"))
            moe.moe_forward_noalloc(layer.desc(rows), x, v, layer.router, layer.w13, layer.w2,
                                    layer.topk, got)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), rows
