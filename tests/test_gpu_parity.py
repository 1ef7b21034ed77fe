"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Needs an MI355X."""
import contextlib

import numpy as np
import pytest
import torch

import oracle
from workloads import get_config, make_inputs
from workloads.gen import random_small

from .parity import (TOL, compare, device_layer, fp8_mfma, gemm_path, log, one_stage,
                     run_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_layer_moe_amd as moe
    moe.load_library()
    yield


# ------------------------------------------------------------------ routing --
def _exact_inputs(T, H, E, k, seed, dup=True, zero_router=False, valid_frac=1.0):
    """x in {-2..2}, router in {-8..8} * 2^-6: every partial sum of a logit is
    a multiple of 2^-6 below 2^11, hence exact in fp32 in any order."""
    inp = random_small(T=T, H=H, E=E, k=k, I=32, seed=seed, valid_frac=valid_frac)
    g = torch.Generator().manual_seed(seed)
    inp.x = torch.randint(-2, 3, (T, H), generator=g).to(torch.bfloat16)
    R = torch.randint(-8, 9, (E, H), generator=g).float() * 2.0 ** -6
    if dup:
        R[E - 1] = R[1]          # exact ties between expert 1 and E-1
        R[E // 2] = R[0]
    if zero_router:
        R.zero_()
    inp.router = R.to(torch.bfloat16)
    return inp


@pytest.mark.parametrize("T,H,E,k,vf,zero", [
    (100, 256, 40, 5, 0.8, False),
    (37, 7168, 48, 3, 1.0, False),
    (70, 1024, 256, 8, 0.9, False),
    (16, 256, 8, 2, 1.0, True),
])
def test_route_exact_arithmetic_bitwise(T, H, E, k, vf, zero):
    inp = _exact_inputs(T, H, E, k, seed=T + E, zero_router=zero, valid_frac=vf)
    layer = device_layer(inp)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    ids, w, lg = layer.route(xd, vd, logits=True)
    torch.cuda.synchronize()
    x64, R64 = oracle.to_f64(inp.x), oracle.to_f64(inp.router)
    valid = None if inp.valid is None else inp.valid.numpy().astype(bool)
    ids_o, w_o, l_o = oracle.route(x64, valid, R64, k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    v = np.ones(T, bool) if valid is None else valid
    assert np.array_equal(lg.cpu().double().numpy()[v], l_o[v])
    assert np.abs(w.cpu().double().numpy() - w_o).max() <= 1e-6
    if zero:
        assert (ids.cpu().numpy() == np.arange(k)).all()


@pytest.mark.parametrize("name", ["decode_e48", "decode_e256_shared", "gather_padded_e48",
                                  "prefill_ub_fp8"])
def test_route_selection_on_gpu_logits_is_bitwise(name):
    """The oracle's selection run on the GPU's own fp32 logits (moe_route's
    debug output) gives the GPU's ids and slot order bit for bit on every
    valid row, and its weights are the softmax of those logits within 2e-6;
    padding rows get ids -1 and weights 0."""
    cfg = get_config(name)
    log(f"[case] route on own logits: {name}")
    inp = make_inputs(cfg)
    layer = device_layer(inp)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    ids, w, lg = layer.route(xd, vd, logits=True)
    torch.cuda.synchronize()
    ids, w, l32 = ids.cpu().numpy(), w.cpu().double().numpy(), lg.cpu().numpy()
    valid = np.ones(cfg.T, bool) if inp.valid is None else inp.valid.numpy().astype(bool)
    assert (ids[~valid] == -1).all() and (w[~valid] == 0).all()
    worst = 0.0
    for t in np.nonzero(valid)[0]:
        sel = oracle.select_topk(l32[t], cfg.k)
        assert ids[t].tolist() == sel, f"row {t}: gpu {ids[t].tolist()} vs {sel}"
        ref = oracle.topk_weights(l32[t, sel].astype(np.float64))
        worst = max(worst, float(np.abs(w[t] - ref).max()))
    log(f"[parity] {name}: ids bitwise on {int(valid.sum())} rows, max |dw| {worst:.2e}")
    assert worst <= 2e-6


# -------------------------------------------------------------------- align --
def _random_ids(T, E, k, seed, pad_frac=0.1):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[rng.random(T) < pad_frac] = -1
    return ids


CANARY = -7


def _gpu_align(ids, E, bm, ns=0, workspace=False, stream=None):
    """moe_align through the C ABI into canary-filled buffers (each longer
    than its documented capacity); workspace=True passes one, which sends
    batches of more than 8192 assignments to the span-parallel kernels."""
    import expert_layer_moe_amd as moe
    T, k = ids.shape
    cap = T * (k + ns) + (E + ns) * (bm - 1)
    d = moe.make_desc(T, 128, E, 128, ns)
    idd = torch.from_numpy(ids).cuda()
    s = torch.full((cap + 64,), CANARY, dtype=torch.int32, device="cuda")
    be = torch.full(((cap + bm - 1) // bm + 16,), CANARY, dtype=torch.int32, device="cuda")
    off = torch.full((E + ns + 1 + 8,), CANARY, dtype=torch.int32, device="cuda")
    n = torch.full((1,), CANARY, dtype=torch.int32, device="cuda")
    ws = moe.alloc_workspace(d, k) if workspace else None
    moe.moe_align(d, idd, k, bm, s, be, off, n, ws, stream)
    return s, be, off, n


def _oracle_align(ids, E, bm, ns):
    """oracle.align, with the shared expert (ns = 1) entered as one more
    expert E on every row whose first id is valid, and its entries given in
    the ABI's encoding (token t of the shared segment as t * k)."""
    T, k = ids.shape
    if ns == 0:
        return oracle.align(ids, E, bm)
    ext = np.concatenate([ids, np.where(ids[:, :1] >= 0, E, -1)], axis=1).astype(np.int32)
    s, be, off, n = oracle.align(ext, E + 1, bm)
    t, j = s // (k + 1), s % (k + 1)
    s = np.where(s >= 0, t * k + np.where(j < k, j, 0), -1).astype(np.int32)
    return s, be, off, n


ALIGN_CASES = [
    (1, 4, 1, 32, 0), (37, 9, 3, 1, 0), (256, 48, 3, 32, 0), (128, 256, 8, 16, 0),
    (1000, 64, 6, 64, 0), (333, 200, 7, 256, 0), (100, 9, 3, 4, 1),
    # more than 8192 assignments: the span-parallel path when given a workspace
    (8192, 256, 8, 16, 0), (8192, 256, 8, 32, 0), (16384, 256, 8, 16, 0),
    (8192, 48, 3, 128, 0), (4096, 48, 3, 32, 1), (3000, 20, 2, 16, 1), (2049, 7, 4, 1, 0),
]


@pytest.mark.parametrize("workspace", [False, True])
@pytest.mark.parametrize("T,E,k,bm,ns", ALIGN_CASES)
def test_align_bitwise(T, E, k, bm, ns, workspace):
    """sorted_ids, block_expert, expert_offsets and n_post_padded equal the
    oracle's bit for bit, on the one-block and the span-parallel paths; no
    entry past what the call documents as written is touched."""
    ids = _random_ids(T, E, k, seed=T * 7 + E)
    log(f"[case] align T={T} E={E} k={k} bm={bm} ns={ns} workspace={workspace}")
    s, be, off, n = _gpu_align(ids, E, bm, ns, workspace)
    torch.cuda.synchronize()
    s_o, be_o, off_o, n_o = _oracle_align(ids, E, bm, ns)
    s, be, off = s.cpu().numpy(), be.cpu().numpy(), off.cpu().numpy()
    n_g = int(n.item())
    assert n_g == n_o
    assert np.array_equal(s[:n_g], s_o)
    assert np.array_equal(be[:n_g // bm], be_o)
    assert np.array_equal(off[:E + ns + 1], off_o)
    assert (s[n_g:] == CANARY).all(), "sorted_ids written past n_post_padded"
    assert (be[n_g // bm:] == CANARY).all(), "block_expert written past its blocks"
    assert (off[E + ns + 1:] == CANARY).all(), "expert_offsets written past E + n_shared + 1"


def test_align_deterministic_across_repeats_and_streams():
    ids = _random_ids(4096, 256, 8, seed=5)
    ref = [t.cpu() for t in _gpu_align(ids, 256, 32, workspace=True)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(10):
        with torch.cuda.stream(s1):
            a = _gpu_align(ids, 256, 32, workspace=True, stream=s1)
        with torch.cuda.stream(s2):
            b = _gpu_align(ids, 256, 32, stream=s2)
        torch.cuda.synchronize()
        for x, y, r in zip(a, b, ref):
            assert torch.equal(x.cpu(), r) and torch.equal(y.cpu(), r)


# ------------------------------------------------------- small full layers --
SMALL = [
    dict(T=70, H=256, E=8, k=2, I=64),
    dict(T=100, H=512, E=16, k=4, I=96, n_shared=1, valid_frac=0.7),
    dict(T=90, H=256, E=6, k=2, I=128, w="fp8"),
    dict(T=50, H=384, E=10, k=3, I=256, n_shared=1, w="fp8", valid_frac=0.6),
    dict(T=33, H=128, E=5, k=2, I=32, act="f32", w="f32"),
    dict(T=40, H=256, E=256, k=8, I=32),
    dict(T=1, H=128, E=4, k=1, I=32),
    dict(T=20, H=128, E=4, k=4, I=64),
    dict(T=300, H=1024, E=32, k=4, I=160, valid_frac=0.5),
    # larger segments (with path "gemm" many of them take the tiled GEMMs)
    dict(T=300, H=256, E=4, k=2, I=128),
    dict(T=400, H=512, E=4, k=2, I=256, w="fp8"),
    dict(T=1100, H=256, E=16, k=2, I=64, valid_frac=0.7),   # + router GEMM
    dict(T=200, H=384, E=8, k=2, I=128, n_shared=1),        # shared expert tiled
    # more than 8192 assignments: the span-parallel align
    dict(T=1200, H=256, E=64, k=8, I=128, n_shared=1, valid_frac=0.8),
    # router of up to 128 experts on large batches: E not a multiple of 4
    # (scalar partial stores), E across two waves, odd K windows per chunk
    dict(T=1500, H=256, E=13, k=3, I=64, valid_frac=0.6),
    dict(T=1030, H=384, E=100, k=5, I=128, n_shared=1),
    # the general tiled down GEMM (I a multiple of 128 other than 128 and 256),
    # bf16 and fp8, both layouts
    dict(T=300, H=256, E=4, k=2, I=384),
    dict(T=260, H=384, E=5, k=2, I=640, n_shared=1),
    dict(T=300, H=256, E=4, k=2, I=384, w="fp8"),
    # a large batch (one combine block per row) with H past 8192 columns and
    # not a multiple of 256 (the down kernel's last column group half used)
    dict(T=2100, H=8320, E=8, k=2, I=64, valid_frac=0.6),
]


def _gemm_capable(kw):
    return kw.get("act", "bf16") == "bf16" and kw["I"] % 128 == 0 and kw["H"] % 128 == 0


def _small_cases():
    """(layer, packed, path) combinations that apply: fp32 weights have no
    packed layout; the GEMM paths need a shape the tiled kernels take; the fp8
    MFMA setting only concerns fp8 weights."""
    out = []
    for i, kw in enumerate(SMALL):
        for packed in (False, True):
            if packed and kw.get("w") == "f32":
                continue
            for path in ("auto", "gemm", "gemm-fp8mfma"):
                if path != "auto" and not _gemm_capable(kw):
                    continue
                if path == "gemm-fp8mfma" and kw.get("w") != "fp8":
                    continue
                out.append((i, packed, path))
    return out


@pytest.mark.parametrize("i,packed,path", _small_cases())
def test_small_layers_match_oracle(i, packed, path):
    """path "gemm": segments above 16 rows take the tiled GEMM kernels (the
    others stream), so both expert paths meet in one call; "gemm-fp8mfma":
    the same with the fp8 MFMA on two-term token codes instead of fp8
    weights dequantised for bf16 MFMA."""
    kw = SMALL[i]
    log(f"[case] small layer {i} packed={packed} path={path}: {kw}")
    inp = random_small(seed=100 + i, **kw)
    with fp8_mfma(path == "gemm-fp8mfma"):
        layer = device_layer(inp, packed=packed)
        if path == "auto":
            gpu = run_gpu(inp, layer)
        else:
            with gemm_path():
                gpu = run_gpu(inp, layer)
    compare(inp, gpu)


def _pack_reference(w: torch.Tensor) -> torch.Tensor:
    """The documented fragment layout of a [rows, K] matrix, by reshaping:
    (t, m, s, g, i) -> (t, s, g, m, i)."""
    R, K = w.shape
    return w.reshape(R // 16, 16, K // 32, 4, 8).permute(0, 2, 3, 1, 4).reshape(R, K)


@pytest.mark.parametrize("w", ["bf16", "fp8"])
def test_pack_weights_layout_bitwise(w):
    import expert_layer_moe_amd as moe
    inp = random_small(T=8, H=256, E=3, k=2, I=128, n_shared=1, w=w, seed=7)
    ne, I, H = 4, 128, 256
    d = moe.make_desc(8, H, 3, I, 1, moe.MOE_BF16,
                      moe.MOE_BF16 if w == "bf16" else moe.MOE_FP8_E4M3)
    w13, w2 = inp.w13.cuda(), inp.w2.cuda()
    p13, p2 = moe.moe_pack_weights(d, w13, w2)
    torch.cuda.synchronize()
    as_int = (lambda t: t.view(torch.int16)) if w == "bf16" else (lambda t: t)
    ref13 = _pack_reference(as_int(inp.w13).reshape(ne * 2 * I, H)).reshape(ne, 2 * I, H)
    ref2 = _pack_reference(as_int(inp.w2).reshape(ne * H, I)).reshape(ne, H, I)
    assert torch.equal(as_int(p13.cpu()), ref13)
    assert torch.equal(as_int(p2.cpu()), ref2)


_PACKED_CASES = [
    dict(T=300, H=1024, E=32, k=4, I=160, valid_frac=0.5),
    dict(T=400, H=512, E=4, k=2, I=256, w="fp8"),
    dict(T=200, H=384, E=8, k=2, I=128, n_shared=1),
    dict(T=300, H=256, E=4, k=2, I=384),
    dict(T=260, H=384, E=5, k=2, I=640, n_shared=1),
    dict(T=300, H=256, E=4, k=2, I=384, w="fp8"),
]


@pytest.mark.parametrize("kw,path", [(kw, p) for kw in _PACKED_CASES for p in ("auto", "gemm")
                                     if p == "auto" or _gemm_capable(kw)])
def test_packed_weights_give_identical_output(kw, path):
    """Only the weight addresses change with the layout: same bits out (the
    GEMM path where the tiled kernels take the shape)."""
    inp = random_small(seed=11, **kw)
    with gemm_path() if path == "gemm" else contextlib.nullcontext():
        a = run_gpu(inp, device_layer(inp, packed=False))
        b = run_gpu(inp, device_layer(inp, packed=True))
    assert np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("path", ["auto", "gemm", "gemm-fp8mfma"])
@pytest.mark.parametrize("packed", [False, True])
def test_fp8_zero_and_tiny_block_scales(packed, path):
    """W2 blocks whose first or second 128-wide K block has a zero scale, or a
    second-block scale 1e-25 of the first: the block scales multiply fp32
    partial sums in the kernels, and these cases take their edge paths."""
    inp = random_small(T=400, H=512, E=4, k=2, I=256, w="fp8", seed=41)
    s2 = inp.s2.clone()
    E1, NB, _ = s2.shape
    for e in range(E1):
        for nb in range(NB):
            c = (e + nb) % 4
            if c == 0:
                s2[e, nb, 1] = 0.0
            elif c == 1:
                s2[e, nb, 0] = 0.0
            elif c == 2:
                s2[e, nb, 1] = s2[e, nb, 0] * 1e-25
    inp.s2 = s2
    s13 = inp.s13.clone()
    s13[0, :, 1] = 0.0                       # a zero K block in every gate/up row block
    s13[1, 0, :] = 0.0                       # a gate row block with all scales zero
    s13[2, :, 2] = s13[2, :, 0] * 1e-25      # a K block far below the others
    s13[3, 1, 0] = -s13[3, 1, 0]             # a negative scale
    inp.s13 = s13
    log(f"[case] fp8 zero/tiny scales packed={packed} path={path}")
    with fp8_mfma(path == "gemm-fp8mfma"):
        layer = device_layer(inp, packed=packed)
        with gemm_path() if path != "auto" else contextlib.nullcontext():
            gpu = run_gpu(inp, layer)
    compare(inp, gpu)


@pytest.mark.parametrize("w", ["bf16", "fp8"])
def test_largest_gemm_k(w):
    """H = 16384, the largest K the tiled GEMMs take: their fp8 scale rows fill
    the LDS arrays exactly (128 K blocks) and the 32-bit offsets are at their
    largest; both expert paths, packed weights.  The outputs grow with H
    (|out| up to ~8.5 here, where rounding to bf16 alone can be off by half a
    spacing, 2^-5 = 3.1e-2, against |out| <= ~4.4 in the workloads the
    absolute bars were set on), so for this shape only the max-abs bar scales
    with the reference's largest |out| / 4.4; nL1 keeps its bar."""
    kw = dict(T=300, H=16384, E=4, k=2, I=128, w=w, n_shared=1)
    log(f"[case] largest GEMM K: {kw}")
    inp = random_small(seed=61, **kw)
    ref = oracle.moe_forward(inp, return_routing=True)
    max_abs, nl1 = TOL[w]
    tol = (max_abs * max(1.0, float(np.abs(ref[0]).max()) / 4.4), nl1)
    layer = device_layer(inp, packed=True)
    compare(inp, run_gpu(inp, layer), ref=ref, tol=tol)
    with gemm_path():
        compare(inp, run_gpu(inp, layer), ref=ref, tol=tol)
    if w == "fp8":
        with fp8_mfma(True):
            layer = device_layer(inp, packed=True)
            with gemm_path():
                compare(inp, run_gpu(inp, layer), ref=ref, tol=tol)


@pytest.mark.parametrize("kw,path", [
    (dict(T=300, H=256, E=8, k=2, I=128, n_shared=1, valid_frac=0.8), "auto"),
    (dict(T=300, H=256, E=8, k=2, I=128, n_shared=1, valid_frac=0.8), "gemm"),
    (dict(T=400, H=512, E=4, k=2, I=256, w="fp8"), "gemm"),
    (dict(T=33, H=128, E=5, k=2, I=32, act="f32", w="f32"), "auto"),
])
def test_block_m_gives_identical_output(kw, path):
    """Every accepted block_m (the segments' padding in the sorted row list)
    gives the same output bits, which also match the oracle."""
    inp = random_small(seed=71, **kw)
    packed = kw.get("w") != "f32"
    outs = []
    for bm in (0, 16, 32, 64, 128, 256):
        log(f"[case] block_m={bm} path={path}: {kw}")
        layer = device_layer(inp, packed=packed, block_m=bm)
        with gemm_path() if path == "gemm" else contextlib.nullcontext():
            outs.append(run_gpu(inp, layer))
    for o in outs[1:]:
        assert np.array_equal(o["out"], outs[0]["out"])
    compare(inp, outs[0])


def test_all_rows_padding_gives_zero_output():
    inp = random_small(T=40, H=256, E=8, k=2, I=64, seed=3)
    inp.valid = torch.zeros(40, dtype=torch.uint8)
    inp.x = torch.full_like(inp.x, float("nan"))
    gpu = run_gpu(inp)
    assert (gpu["out"] == 0).all() and (gpu["ids"] == -1).all()


# ------------------------------------------------------ full-size workloads --
# the benchmark runs the packed layout; decode_e48 is also checked row-major
@pytest.mark.parametrize("name,packed", [
    ("tiny", False), ("decode_e48", False), ("decode_e48", True),
    ("decode_e256_shared", True), ("gather_padded_e48", True), ("prefill_ub_fp8", True)])
def test_workload_matches_oracle(name, packed):
    cfg = get_config(name)
    log(f"[case] {name} packed={packed}: generating inputs")
    inp = make_inputs(cfg)
    log(f"[case] {name}: GPU run")
    gpu = run_gpu(inp, device_layer(inp, packed=packed))
    log(f"[case] {name}: oracle run")
    compare(inp, gpu)


def test_prefill_fp8_mfma_two_term_matches_oracle():
    """The prefill micro-batch with its tiled gate/up on the fp8 MFMA over the
    two-term e4m3 token codes (the moe_set_fp8_mfma option): the oracle's
    values within the fp8 bar, at the full size."""
    cfg = get_config("prefill_ub_fp8")
    log("[case] prefill_ub_fp8 fp8 MFMA two-term: generating inputs")
    inp = make_inputs(cfg)
    with fp8_mfma(True):
        layer = device_layer(inp, packed=True)
        log("[case] prefill_ub_fp8 fp8 MFMA two-term: GPU run")
        gpu = run_gpu(inp, layer)
    log("[case] prefill_ub_fp8 fp8 MFMA two-term: oracle run")
    compare(inp, gpu)


# The one-launch expert MLP (gate/up and down in one persistent launch, work
# items taken from per-XCD queues, down units waiting on per-item counts) is
# switched off and its kernel is not in the library: the first GPU run of its
# first case (T=300, row-major weights) went silent until it was killed after
# 180 s, and no cause has been found in its code.  The tests stay, skipped.
# (The one launch built later with a ticket counter, moe_set_one_launch, has
# its own tests in test_gpu_one_launch.py.)
ONE_STAGE_OFF = ("one-launch expert MLP switched off: its first GPU run hung and the "
                 "cause is not found")

ONE_STAGE_SMALL = [
    dict(T=300, H=512, E=16, k=4, I=128, n_shared=1, valid_frac=0.7),
    dict(T=64, H=512, E=8, k=2, I=256, w="fp8"),
    dict(T=1, H=1024, E=4, k=1, I=128),
    dict(T=200, H=512, E=3, k=2, I=384, w="fp8", n_shared=1),   # segments of several items
    dict(T=40, H=512, E=64, k=8, I=128, n_shared=1),            # fewer items than XCD queues
]


@pytest.mark.skip(reason=ONE_STAGE_OFF)
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kw", ONE_STAGE_SMALL)
def test_one_stage_matches_two_launches(kw, packed):
    """Gate/up and down in one launch (per-XCD work queues, h handed over
    through one XCD's L2) give the two-launch path's bits, and the oracle's
    values."""
    inp = random_small(seed=91, **kw)
    log(f"[case] one stage packed={packed}: {kw}")
    ref = run_gpu(inp, device_layer(inp, packed=packed))
    with one_stage(True):
        gpu = run_gpu(inp, device_layer(inp, packed=packed))
    assert np.array_equal(gpu["out"], ref["out"])
    compare(inp, gpu)


@pytest.mark.skip(reason=ONE_STAGE_OFF)
@pytest.mark.parametrize("name", ["decode_e48", "decode_e256_shared"])
def test_one_stage_decode_workloads(name):
    cfg = get_config(name)
    log(f"[case] one stage {name}")
    inp = make_inputs(cfg)
    ref = run_gpu(inp, device_layer(inp, packed=True))
    with one_stage(True):
        layer = device_layer(inp, packed=True)
        gpu = run_gpu(inp, layer)
        again = run_gpu(inp, layer)         # the sync words are reset by every call
    assert np.array_equal(gpu["out"], ref["out"])
    assert np.array_equal(again["out"], ref["out"])
    compare(inp, gpu)


@pytest.mark.skip(reason=ONE_STAGE_OFF)
def test_one_stage_replays_in_a_hip_graph():
    inp = random_small(seed=93, T=256, H=512, E=16, k=3, I=128, valid_frac=0.9)
    with one_stage(True):
        layer = device_layer(inp, packed=True)
        xd = inp.x.cuda()
        vd = inp.valid.cuda()
        ref = layer.forward(xd, vd)
        out = torch.empty_like(ref)
        ws = layer.workspace(xd.shape[0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(xd, vd, out=out, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        assert torch.isfinite(junk)


def test_gather_nan_padding_rows_are_never_read():
    cfg = get_config("gather_padded_e48")
    inp = make_inputs(cfg)
    layer = device_layer(inp)
    a = run_gpu(inp, layer)
    x_nan = inp.x.clone()
    x_nan[inp.valid == 0] = float("nan")
    b = run_gpu(inp, layer, x=x_nan)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["ids"], b["ids"])


@pytest.mark.parametrize("kw", [
    dict(T=1500, H=256, E=13, k=3, I=64, valid_frac=0.3),            # tiled router
    dict(T=1030, H=384, E=100, k=5, I=128, n_shared=1, valid_frac=0.5),
    dict(T=1200, H=256, E=64, k=8, I=128, w="fp8", valid_frac=0.2),   # bf16 y rows
    dict(T=1100, H=256, E=200, k=4, I=64, valid_frac=0.4),           # the 256-expert router GEMM
    dict(T=300, H=256, E=8, k=2, I=64, valid_frac=0.5),              # small batch router
])
def test_padding_output_rows_are_zeroed_whatever_out_held(kw):
    """Every output row of a padding token is written with zeros (out filled
    with NaN beforehand), for each router and combine variant."""
    inp = random_small(seed=77, **kw)
    log(f"[case] padding rows zeroed in a NaN-filled out: {kw}")
    layer = device_layer(inp, packed=True)
    xd, vd = inp.x.cuda(), inp.valid.cuda()
    out = torch.full_like(xd, float("nan"))
    layer.forward(xd, vd, out=out)
    torch.cuda.synchronize()
    o = out.float().cpu()
    pad = inp.valid == 0
    assert pad.any() and (o[pad] == 0).all()
    assert torch.isfinite(o).all()
    ref = run_gpu(inp, layer)["out"]
    assert np.array_equal(o.double().numpy(), ref)


@pytest.mark.parametrize("kw", [
    dict(T=152, H=512, E=64, k=8, I=128),                      # 1216 assignments: one launch
    dict(T=153, H=512, E=64, k=8, I=128),                      # 1224: down, then combine
    dict(T=135, H=384, E=100, k=8, I=64, n_shared=1, valid_frac=0.9),   # 1215 with the shared slot
    dict(T=152, H=256, E=64, k=8, I=128, w="fp8", valid_frac=0.7),
])
@pytest.mark.parametrize("packed", [False, True])
def test_down_and_combine_in_one_launch_at_its_row_limit(kw, packed):
    """Small batches where every segment streams run the down projection and
    the combine in one launch while their assignments fit its 1216 LDS rows,
    and in two launches past that; both match the oracle."""
    inp = random_small(seed=1216 + kw["T"], **kw)
    log(f"[case] down + combine row limit, packed={packed}: {kw}")
    compare(inp, run_gpu(inp, device_layer(inp, packed=packed)))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("ns", [0, 1])
def test_all_streaming_nan_padding_rows_are_never_read(packed, ns):
    """A layer whose segments all stream (its gate/up reads the token rows
    straight from x through the sorted list, padding slots of the list
    pointing at row 0) with row 0 and every other padding row NaN: the same
    output bits as with finite padding rows, zero rows for padding tokens,
    and the oracle's result."""
    inp = random_small(T=200, H=512, E=8, k=2, I=128, n_shared=ns, valid_frac=0.6,
                       seed=321 + ns)
    inp.valid[0] = 0
    log(f"[case] all-streaming layer with NaN padding rows, packed={packed} ns={ns}")
    layer = device_layer(inp, packed=packed)
    a = run_gpu(inp, layer)
    x_nan = inp.x.clone()
    x_nan[inp.valid == 0] = float("nan")
    b = run_gpu(inp, layer, x=x_nan)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["ids"], b["ids"])
    assert np.isfinite(b["out"]).all()
    assert (b["out"][inp.valid.numpy() == 0] == 0).all()
    compare(inp, a)


def test_prefill_two_streams_match_unsplit_batch():
    """ub0 and ub1 (midpoint split) on two HIP streams give exactly the rows of
    the unsplit 16384-row batch; ub1 also matches the oracle."""
    cfg = get_config("prefill_ub_fp8")
    full = make_inputs(cfg.with_(T=16384, ub=None))
    layer = device_layer(full, packed=True)
    xd = full.x.cuda()
    ref = layer.forward(xd)
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    ws0, ws1 = layer.workspace(8192), torch.empty_like(layer.workspace(8192))
    torch.cuda.synchronize()
    outs = []
    for s, ws, lo in ((s0, ws0, 0), (s1, ws1, 8192)):
        with torch.cuda.stream(s):
            outs.append(layer.forward(xd[lo:lo + 8192], workspace=ws, stream=s))
    torch.cuda.synchronize()
    both = torch.cat(outs)
    assert torch.equal(both, ref), float((both.float() - ref.float()).abs().max())
    ub1 = make_inputs(cfg.with_(ub=1))
    gpu = dict(out=outs[1].float().cpu().double().numpy())
    ids, w, lg = layer.route(ub1.x.cuda(), None, logits=True)
    gpu.update(ids=ids.cpu().numpy(), w=w.cpu().double().numpy(),
               logits=lg.cpu().double().numpy())
    compare(ub1, gpu)


# ---------------------------------------------------------- graph capture --
@pytest.mark.parametrize("kw,path", [
    (dict(T=256, H=512, E=16, k=3, I=128, valid_frac=0.9), "auto"),
    (dict(T=300, H=256, E=4, k=2, I=128, w="fp8", n_shared=1), "gemm"),
])
def test_forward_replays_in_a_hip_graph(kw, path):
    """moe_forward only enqueues kernels (no allocation, memset or sync), so it
    captures into a HIP graph; every replay, with eager work and
    synchronisations between replays, matches the eager call bit for bit."""
    inp = random_small(seed=21, **kw)
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    vd = None if inp.valid is None else inp.valid.cuda()
    with gemm_path() if path == "gemm" else contextlib.nullcontext():
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


def test_two_stream_pair_replays_in_a_hip_graph():
    """The ub0/ub1 pair on two HIP streams (forked and joined with events)
    captures into one graph; replays match the eager pair bit for bit."""
    inp = random_small(T=512, H=256, E=8, k=2, I=128, w="fp8", seed=23)
    layer = device_layer(inp, packed=True)
    xd = inp.x.cuda()
    halves = (xd[:256], xd[256:])
    wss = (layer.workspace(256), torch.empty_like(layer.workspace(256)))
    outs = [torch.empty_like(h) for h in halves]
    streams = (torch.cuda.Stream(), torch.cuda.Stream())

    def pair():
        cur = torch.cuda.current_stream()
        ev = torch.cuda.Event()
        ev.record(cur)
        for s, xx, oo, ww in zip(streams, halves, outs, wss):
            s.wait_event(ev)
            with torch.cuda.stream(s):
                layer.forward(xx, None, oo, ww, stream=s)
        for s in streams:
            cur.wait_stream(s)

    pair()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert torch.equal(torch.cat(ref), layer.forward(xd))   # = the unsplit batch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pair()
    for i in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(outs, ref)), f"replay {i}"


# ------------------------------------------------------------ random shapes --
def _random_shape(seed):
    """A seeded layer shape within what the ABI accepts for bf16 activations."""
    r = np.random.default_rng(1000 + seed)
    w = ["bf16", "fp8"][r.integers(2)]
    H = int(r.choice([128, 256, 384, 512, 768]))
    I = int(r.choice([128, 256, 384]) if w == "fp8" else r.choice([32, 64, 96, 128, 160, 256]))
    E = int(r.choice([1, 2, 3, 5, 8, 13, 16, 33, 64, 128]))
    k = int(r.integers(1, min(8, E) + 1))
    T = int(r.choice([1, 2, 7, 16, 31, 64, 100, 257, 513, 700]))
    ns = int(r.integers(2))
    vf = float(r.choice([1.0, 1.0, 0.75, 0.3]))
    return dict(T=T, H=H, E=E, k=k, I=I, n_shared=ns, w=w, valid_frac=vf)


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes_match_oracle(seed):
    """Seeded random shapes (ragged T, E from 1 to 128, k up to 8, shared
    expert, fp8, padding rows), packed weights, both expert paths."""
    kw = _random_shape(seed)
    log(f"[case] random shape {seed}: {kw}")
    inp = random_small(seed=500 + seed, **kw)
    layer = device_layer(inp, packed=True)
    gpu = run_gpu(inp, layer)
    compare(inp, gpu)
    if _gemm_capable(kw):
        with gemm_path():
            compare(inp, run_gpu(inp, layer))


@pytest.mark.parametrize("w,I", [("bf16", 1024), ("fp8", 2048)])
def test_streaming_units_beyond_the_capped_grid(w, I):
    """Every segment on the streaming kernels with more gate/up work units
    (128 items of 64 rows x 64 column groups = 8192) than their grid holds
    (4096 blocks): blocks loop over the units."""
    import expert_layer_moe_amd as moe
    kw = dict(T=2048, H=256, E=32, k=4, I=I, w=w)
    log(f"[case] streaming units beyond the grid: {kw}")
    inp = random_small(seed=900 + I, **kw)
    layer = device_layer(inp, packed=True)
    moe.moe_set_path_thresholds(2**31 - 1, -1)   # no segment takes the GEMM
    try:
        gpu = run_gpu(inp, layer)
    finally:
        moe.moe_set_path_thresholds()
    compare(inp, gpu)
