"""moe_forward_noalloc (the entry point that runs in the library's fixed
device scratch instead of a caller's workspace) against moe_forward, through
the C ABI: same bits, on consecutive calls whose second input is smaller
(the scratch keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import get_config, make_inputs
from workloads.gen import random_small

from .parity import compare, device_layer, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_layer_moe_amd as moe
    moe.load_library()
    yield


def _noalloc(layer, x, valid):
    import expert_layer_moe_amd as moe
    out = torch.full_like(x, float("nan"))
    moe.moe_forward_noalloc(layer.desc(x.shape[0]), x, valid, layer.router, layer.w13,
                            layer.w2, layer.topk, out)
    return out


def _check_pair(layer, x, valid):
    """moe_forward_noalloc and moe_forward on the same rows: equal bits."""
    got = _noalloc(layer, x, valid)
    ref = layer.forward(x, valid)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), float((got.float() - ref.float()).abs().nan_to_num(1e9).max())
    return got


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_decode_layer_two_calls(packed):
    """The 48-expert decode share (256 rows), then its first 64 rows."""
    cfg = get_config("decode_e48")
    inp = make_inputs(cfg)
    layer = device_layer(inp, packed=packed)
    x = inp.x.cuda()
    log(f"[case] noalloc decode_e48 packed={packed}: 256 rows, then 64")
    out = _check_pair(layer, x, None)
    gpu = dict(out=out.float().cpu().double().numpy())
    ids, w, lg = layer.route(x, None, logits=True)
    gpu.update(ids=ids.cpu().numpy(), w=w.cpu().double().numpy(),
               logits=lg.cpu().double().numpy())
    compare(inp, gpu)
    _check_pair(layer, x[:64].contiguous(), None)


@pytest.mark.parametrize("kw", [
    dict(T=300, H=512, E=16, k=4, I=128, n_shared=1, valid_frac=0.7),
    dict(T=260, H=384, E=8, k=2, I=256, w="fp8", n_shared=1),
    dict(T=90, H=256, E=6, k=2, I=64, act="f32", w="f32"),
])
def test_noalloc_small_layers_two_calls(kw):
    """A layer with padding rows (or fp8 weights, or fp32), then a smaller
    batch of the same layer."""
    inp = random_small(seed=81, **kw)
    packed = kw.get("w") != "f32"
    layer = device_layer(inp, packed=packed)
    x = inp.x.cuda()
    valid = None if inp.valid is None else inp.valid.cuda()
    log(f"[case] noalloc {kw}: {x.shape[0]} rows, then {x.shape[0] // 3}")
    _check_pair(layer, x, valid)
    n = x.shape[0] // 3
    _check_pair(layer, x[:n].contiguous(), None if valid is None else valid[:n].contiguous())


def test_noalloc_rejects_layers_above_the_scratch():
    import expert_layer_moe_amd as moe
    inp = random_small(T=8, H=256, E=8, k=2, I=128, seed=83)
    layer = device_layer(inp)
    d = layer.desc(200000)
    assert moe.moe_workspace_size(d, 2) > moe.SCRATCH_BYTES
    x = torch.zeros((200000, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(d, x, None, layer.router, layer.w13, layer.w2, 2,
                                torch.empty_like(x))
    assert e.value.status == -3
