"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's formulas: each checks it against a
hand-worked example, a closed form, an exact (rational) computation, brute
force, an invariant, or a special case that reduces to a library routine.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import (CONFIGS, LayerConfig, LayerInputs, boundary_split,
                       get_config, midpoint_split, valid_mask)
from workloads.gen import random_small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _inputs_from_arrays(x, R, w13, w2, k, valid=None, n_shared=0):
    T, H = x.shape
    E = R.shape[0]
    I = w13.shape[1] // 2
    cfg = LayerConfig(name="hand", T=T, H=H, E=E, k=k, I=I, n_shared=n_shared,
                      act="f32", w="f32")
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    v = None if valid is None else torch.as_tensor(np.asarray(valid, dtype=np.uint8))
    return LayerInputs(cfg=cfg, x=t(x), valid=v, router=t(R), w13=t(w13), w2=t(w2))


# ------------------------------------------------------------ fp8 format --
def test_fp8_table_matches_torch_cast_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    mine = oracle.e4m3fn_decode(codes.numpy())
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


def test_fp8_golden_codes_and_block_scales():
    g = _load("fp8_e4m3fn_codes.json")
    for c, v in g["codes"].items():
        got = oracle.e4m3fn_decode(np.array([int(c, 16)]))[0]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), c
    for c in g["nan_codes"]:
        assert np.isnan(oracle.e4m3fn_decode(np.array([int(c, 16)]))[0])
    ex = g["block_scaled_example"]
    q = np.zeros((256, 256), dtype=np.uint8)
    for r, c, code, _ in ex["probes"]:
        q[r, c] = int(code, 16)
    W = oracle.dequant_block_scaled(q, np.array(ex["scales"], dtype=np.float32))
    for r, c, _, v in ex["probes"]:
        assert W[r, c] == v


# ---------------------------------------------------------- hand example --
def _golden_layer():
    g = _load("tiny_layer_example.json")
    L = math.log(3.0)
    x = np.array(g["x"], dtype=np.float64)
    R = np.array(g["router_in_units_of_L"], dtype=np.float64) * L
    gate = np.array(g["w13_in_units_of_L_for_gate"]["gate_rows"], dtype=np.float64) * L
    up = np.array(g["w13_in_units_of_L_for_gate"]["up_rows"], dtype=np.float64)
    w13 = np.concatenate([gate, up], axis=1)
    w2 = np.array(g["w2"], dtype=np.float64)
    return g, L, _inputs_from_arrays(x, R, w13, w2, g["k"])


def test_hand_worked_layer_example():
    g, L, inp = _golden_layer()
    out, r = oracle.moe_forward(inp, return_routing=True)
    assert r["ids"].tolist() == g["expected_ids"]
    assert np.allclose(r["w"], g["expected_weights"], rtol=0, atol=1e-15)
    exp = np.array(g["expected_out_in_units_of_L"]) * L
    assert np.allclose(out, exp, rtol=0, atol=1e-14)


def test_hand_worked_align_example():
    g, L, inp = _golden_layer()
    _, r = oracle.moe_forward(inp, return_routing=True)
    s, be, off, n = oracle.align(r["ids"], g["E"], g["block_m"])
    assert s.tolist() == g["expected_sorted_ids"]
    assert be.tolist() == g["expected_block_expert"]
    assert off.tolist() == g["expected_expert_offsets"]
    assert n == g["expected_n_post_padded"]


# -------------------------------------------------------------- routing --
def test_logits_exact_rational():
    """fp64 logits of bf16 inputs agree with exact rational dot products."""
    inp = random_small(T=3, H=512, E=5, k=2, I=128, seed=7)
    x = oracle.to_f64(inp.x)
    R = oracle.to_f64(inp.router)
    l = oracle.router_logits(x, R)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], R[e]))
            assert abs(Fraction(float(l[t, e])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


def test_logits_one_hot_rows_pick_router_columns():
    rng = np.random.default_rng(3)
    R = rng.standard_normal((6, 9))
    x = np.eye(9)[[2, 7, 0]]
    l = oracle.router_logits(x, R)
    assert np.array_equal(l, R[:, [2, 7, 0]].T)


def _brute_topk(l, k):
    """Unique k-subset whose members all beat all non-members under the
    order (logit desc, id asc); then sorted in that order."""
    E = len(l)
    beats = lambda a, b: (l[a] > l[b]) or (l[a] == l[b] and a < b)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [u for u in range(E) if u not in S]
        if all(beats(s, u) for s in S for u in rest):
            found.append(S)
    assert len(found) == 1
    S = list(found[0])
    # order by pairwise "beats" (a total order)
    return sorted(S, key=lambda a: sum(beats(b, a) for b in S))


@pytest.mark.parametrize("seed", range(40))
def test_select_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 8))
    k = int(rng.integers(1, E + 1))
    l = rng.integers(-3, 4, size=E).astype(np.float32)   # many exact ties
    assert oracle.select_topk(l, k) == _brute_topk(l.tolist(), k)


def test_zero_router_gives_lowest_ids_uniform_weights():
    x = np.random.default_rng(0).standard_normal((4, 16))
    ids, w, _ = oracle.route(x, None, np.zeros((7, 16)), 3)
    assert (ids == np.array([0, 1, 2])).all()
    assert np.allclose(w, 1 / 3, rtol=0, atol=1e-16)


def test_duplicate_router_rows_tie_to_lower_id():
    rng = np.random.default_rng(1)
    R = rng.standard_normal((5, 8))
    R[3] = R[1]
    x = np.zeros((1, 8))
    x[0] = R[1] * 10     # makes experts 1 and 3 the clear winners, tied
    ids, w, _ = oracle.route(x, None, R, 2)
    assert ids[0].tolist() == [1, 3]
    assert w[0, 0] == w[0, 1] == 0.5


def test_topk_weight_closed_forms():
    assert oracle.topk_weights([0.7]).tolist() == [1.0]
    l0, l1 = 1.3, -0.4
    w = oracle.topk_weights([l0, l1])
    assert abs(w[0] - 1 / (1 + math.exp(l1 - l0))) < 1e-15
    assert np.allclose(oracle.topk_weights([2.5] * 4), 0.25, rtol=0, atol=1e-16)


def test_routing_invariants_random():
    inp = random_small(T=50, H=256, E=16, k=4, I=128, seed=11, valid_frac=0.7)
    out, r = oracle.moe_forward(inp, return_routing=True)
    valid = inp.valid.numpy().astype(bool)
    ids, w, l = r["ids"], r["w"], r["logits"]
    for t in range(50):
        if not valid[t]:
            assert (ids[t] == -1).all() and (w[t] == 0).all() and (out[t] == 0).all()
            continue
        assert len(set(ids[t].tolist())) == 4
        assert abs(w[t].sum() - 1) <= 4 * 2 ** -52
        assert (np.diff(w[t]) <= 0).all()
        sel = l[t, ids[t]].astype(np.float32)
        rest = np.delete(l[t], ids[t]).astype(np.float32)
        assert sel.min() >= rest.max()


def test_weights_equal_full_softmax_renormalised():
    """softmax over the k selected logits == full softmax, keep k, renormalise
    (torch.softmax as the library routine)."""
    rng = np.random.default_rng(5)
    l = rng.standard_normal(12)
    p = torch.softmax(torch.tensor(l), dim=0).numpy()
    sel = oracle.select_topk(l.astype(np.float32), 5)
    ref = p[sel] / p[sel].sum()
    assert np.allclose(oracle.topk_weights(l[sel]), ref, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- align --
@pytest.mark.parametrize("seed,bm", [(0, 1), (1, 2), (2, 16), (3, 32), (4, 64), (5, 7)])
def test_align_matches_comparison_sort(seed, bm):
    rng = np.random.default_rng(seed)
    T, E, k = 37, 9, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[rng.random(T) < 0.2] = -1
    s, be, off, n = oracle.align(ids, E, bm)
    pairs = sorted((int(ids[t, j]), t, j) for t in range(T) for j in range(k) if ids[t, j] >= 0)
    # rebuild the padded layout from the comparison sort
    exp = []
    for e in range(E):
        seg = [t * k + j for (ee, t, j) in pairs if ee == e]
        if seg:
            pad = (-len(seg)) % bm
            exp += seg + [-1] * pad
    assert s.tolist() == exp and n == len(exp)
    # invariants
    assert off[0] == 0 and off[-1] == n and (np.diff(off) % bm == 0).all()
    assert len(be) * bm == n
    flat = s[s >= 0]
    assert sorted(flat.tolist()) == sorted(t * k + j for t in range(T) for j in range(k) if ids[t, j] >= 0)
    for b, e in enumerate(be):
        blk = s[b * bm:(b + 1) * bm]
        assert all(ids[a // k, a % k] == e for a in blk if a >= 0)
        # sentinels only at the tail of a segment
        real = blk >= 0
        assert not (~real[:-1] & real[1:]).any()


# -------------------------------------------------------------- experts --
def test_silu_closed_forms():
    L = math.log(3.0)
    v = oracle.silu(np.array([0.0, L, -L, 40.0, -800.0]))
    assert v[0] == 0.0
    assert abs(v[1] - 0.75 * L) < 1e-15 and abs(v[2] + 0.25 * L) < 1e-15
    assert abs(v[3] - 40.0) < 1e-12 and v[4] == 0.0


def test_single_expert_top1_is_dense_swiglu():
    """E = 1, k = 1: routing, weights and combine reduce to a dense SwiGLU
    FFN, here computed with torch.nn.functional.silu and torch matmuls."""
    inp = random_small(T=9, H=128, E=1, k=1, I=256, seed=21)
    out = oracle.moe_forward(inp)
    x = inp.x.double()
    W13 = inp.w13[0].double()
    W2 = inp.w2[0].double()
    g = x @ W13[:256].T
    u = x @ W13[256:].T
    ref = (torch.nn.functional.silu(g) * u) @ W2.T
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_identical_experts_make_routing_irrelevant():
    inp = random_small(T=12, H=128, E=6, k=3, I=128, seed=23)
    inp.w13[:] = inp.w13[2]
    inp.w2[:] = inp.w2[2]
    out = oracle.moe_forward(inp)
    one = inp.w13[:1].clone(), inp.w2[:1].clone()
    inp1 = random_small(T=12, H=128, E=1, k=1, I=128, seed=23)
    inp1.x = inp.x
    inp1.w13, inp1.w2 = one
    assert np.allclose(out, oracle.moe_forward(inp1), rtol=1e-12, atol=1e-14)


def test_k_equals_E_is_dense_softmax_mixture():
    inp = random_small(T=7, H=128, E=4, k=4, I=128, seed=29)
    out = oracle.moe_forward(inp)
    x = inp.x.double()
    p = torch.softmax(x @ inp.router.double().T, dim=1)
    ref = torch.zeros_like(x)
    for e in range(4):
        W13 = inp.w13[e].double()
        y = (torch.nn.functional.silu(x @ W13[:128].T) * (x @ W13[128:].T)) @ inp.w2[e].double().T
        ref += p[:, e:e + 1] * y
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_shared_expert_adds_with_weight_one():
    inp = random_small(T=10, H=128, E=5, k=2, I=128, n_shared=1, seed=31)
    out = oracle.moe_forward(inp)
    inp0 = random_small(T=10, H=128, E=5, k=2, I=128, seed=31)
    inp0.x, inp0.router = inp.x, inp.router
    inp0.w13, inp0.w2 = inp.w13[:5], inp.w2[:5]
    routed = oracle.moe_forward(inp0)
    x = inp.x.double()
    W13 = inp.w13[5].double()
    sh = (torch.nn.functional.silu(x @ W13[:128].T) * (x @ W13[128:].T)) @ inp.w2[5].double().T
    assert np.allclose(out, routed + sh.numpy(), rtol=1e-12, atol=1e-14)


def test_tp_slices_sum_to_unsliced_output():
    """Slicing I across TP ranks (gate rows, matching up rows, matching W2
    columns) gives partial outputs that sum to the whole layer."""
    inp = random_small(T=16, H=128, E=4, k=2, I=512, seed=37)
    full = oracle.moe_forward(inp)
    I, tp = 512, 4
    acc = np.zeros_like(full)
    for s in range(tp):
        c = slice(s * I // tp, (s + 1) * I // tp)
        cu = slice(I + s * I // tp, I + (s + 1) * I // tp)
        part = random_small(T=16, H=128, E=4, k=2, I=I // tp, seed=37)
        part.x, part.router = inp.x, inp.router
        part.w13 = torch.cat([inp.w13[:, c], inp.w13[:, cu]], dim=1)
        part.w2 = inp.w2[:, :, c].contiguous()
        acc += oracle.moe_forward(part)
    assert np.allclose(acc, full, rtol=1e-12, atol=1e-13)


def test_padding_rows_never_read():
    inp = random_small(T=24, H=128, E=6, k=2, I=128, seed=41, valid_frac=0.6)
    out = oracle.moe_forward(inp)
    bad = inp.valid == 0
    assert bad.any()
    x2 = inp.x.clone()
    x2[bad] = float("nan")
    inp.x = x2
    out2 = oracle.moe_forward(inp)
    assert np.array_equal(out, out2)
    assert (out2[bad.numpy()] == 0).all()


def test_fp8_layer_matches_dequantised_bf16_free_layer():
    """fp8 codes + block scales give the same layer as the fp64 weights q*s
    fed as plain float weights."""
    inp = random_small(T=8, H=256, E=3, k=2, I=128, w="fp8", seed=43)
    out = oracle.moe_forward(inp)
    deq = random_small(T=8, H=256, E=3, k=2, I=128, w="f32", seed=43)
    deq.x, deq.router = inp.x, inp.router
    q13 = inp.w13.view(torch.float8_e4m3fn).double()
    q2 = inp.w2.view(torch.float8_e4m3fn).double()
    s13 = inp.s13.double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    s2 = inp.s2.double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    deq.w13, deq.w2 = q13 * s13, q2 * s2
    assert np.allclose(out, oracle.moe_forward(deq), rtol=1e-13, atol=1e-15)


# ----------------------------------------------------- split and masks --
def test_page_numbers_padding_and_splits():
    g = _load("page_numbers.json")
    cfg = get_config("gather_padded_e48")
    m = valid_mask(cfg)
    p = g["padding_waste"]
    assert len(m) == p["ranks"] * p["rows_per_rank"] == cfg.T
    assert sum(m) == 1136
    waste = 1 - sum(m) / len(m)
    assert waste == 0.861328125 and round(100 * waste) == p["waste_percent_printed"]
    s = g["microbatch_split"]
    assert midpoint_split(sum(s["requests"])) == tuple(s["midpoint"])
    b = boundary_split(s["requests"])
    assert b == tuple(s["boundary"])
    assert round(b[1] / b[0], 2) == s["boundary_ratio_printed"]
    es = g["expert_selection"]
    c2 = get_config("decode_e48")
    assert (c2.E, c2.k) == (es["E"], es["k"])


def test_midpoint_split_reproduces_unsplit_result():
    """The layer is row-independent: two micro-batches cut at the token
    midpoint give the unsplit result (routing bitwise)."""
    inp = random_small(T=40, H=128, E=8, k=3, I=128, seed=47)
    full, r = oracle.moe_forward(inp, return_routing=True)
    a, b = midpoint_split(40)
    parts = []
    for lo, hi in ((0, a), (a, a + b)):
        sub = random_small(T=hi - lo, H=128, E=8, k=3, I=128, seed=47)
        sub.x, sub.router, sub.w13, sub.w2 = inp.x[lo:hi], inp.router, inp.w13, inp.w2
        o, rr = oracle.moe_forward(sub, return_routing=True)
        assert np.array_equal(rr["ids"], r["ids"][lo:hi])
        parts.append(o)
    assert np.allclose(np.concatenate(parts), full, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------- near-tie helpers --
def test_admissible_sets():
    l = np.array([3.0, 1.0, 1.0 + 1e-9, -2.0, 0.99])
    sets = oracle.admissible_sets(l, 2, 1e-6)
    assert sets == [(0, 1), (0, 2)]
    assert oracle.admissible_sets(l, 2, 0.0) == [(0, 2)]
    sets = oracle.admissible_sets(l, 2, 0.05)
    assert sets == [(0, 1), (0, 2), (0, 4)]


def _brute_admissible(l, k, delta):
    """Every k-subset S with min over S >= max over the rest - delta, by
    enumerating all k-subsets (the definition, no shortcut)."""
    E = len(l)
    res = []
    for S in itertools.combinations(range(E), k):
        rest = [l[u] for u in range(E) if u not in S]
        if not rest or min(l[s] for s in S) >= max(rest) - delta:
            res.append(tuple(S))
    return res


@pytest.mark.parametrize("seed", range(30))
def test_admissible_sets_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(2, 9))
    k = int(rng.integers(1, E + 1))
    # coarse values: many exact and near ties
    l = rng.integers(-3, 4, size=E) + rng.choice([0.0, 1e-7, -1e-7, 0.5], size=E)
    delta = float(rng.choice([0.0, 1e-6, 0.3, 0.6]))
    assert oracle.admissible_sets(l, k, delta) == _brute_admissible(l.tolist(), k, delta)


def test_tie_threshold_hand_worked():
    g = _load("near_tie_example.json")["threshold"]
    d = oracle.tie_threshold(np.array(g["x"], dtype=np.float64), np.array(g["R"], dtype=np.float64))
    assert d.tolist() == [v * 2.0 ** -20 for v in g["expected_delta_in_units_of_2^-20"]]


def test_near_tie_rows_constructed_gaps():
    g = _load("near_tie_example.json")["near_tie_rows"]
    rows = oracle.near_tie_rows(np.array(g["logits"]), g["k"], np.array(g["delta"]),
                                np.array(g["valid"], dtype=bool))
    assert rows.tolist() == g["expected_rows"]


def _alt_layer():
    g = _load("near_tie_example.json")["alternate_set_layer"]
    L = math.log(3.0)
    w13 = np.concatenate([np.array(g["gate_rows_in_units_of_L"]) * L, np.array(g["up_rows"])],
                         axis=1)
    inp = _inputs_from_arrays(np.array(g["x"], dtype=np.float64),
                              np.array(g["router_in_units_of_L"]) * L, w13, np.array(g["w2"]),
                              g["k"], n_shared=g["n_shared"])
    return g, L, inp


def test_alternate_set_row_hand_worked():
    """A row with an exact tie for its last slot: the oracle's own routing,
    its admissible sets, and the layer output of that row under the other
    admissible set (the shared expert still added with weight 1)."""
    g, L, inp = _alt_layer()
    out, r = oracle.moe_forward(inp, return_routing=True)
    assert r["ids"].tolist() == g["expected_ids"]
    assert np.allclose(out, np.array(g["expected_out_in_units_of_L"]) * L, rtol=0, atol=1e-14)
    t = g["alternate_row"]
    delta = oracle.tie_threshold(r["x64"], r["R64"])
    adm = oracle.admissible_sets(r["logits"][t], g["k"], delta[t])
    assert adm == [tuple(s) for s in g["expected_admissible_sets_row1"]]
    assert oracle.near_tie_rows(r["logits"], g["k"], delta).tolist() == [0, 1]
    alt = oracle.forward_rows_with_sets(inp, r["x64"], r["logits"], [t], [g["alternate_set"]])
    assert np.allclose(alt[0], np.array(g["expected_alternate_out_in_units_of_L"]) * L,
                       rtol=0, atol=1e-14)
    own = oracle.forward_rows_with_sets(inp, r["x64"], r["logits"], [0, 1], r["ids"].tolist())
    assert np.allclose(own, out, rtol=0, atol=1e-14)


@pytest.mark.parametrize("n_shared,w", [(0, "bf16"), (1, "bf16"), (1, "fp8")])
def test_forward_rows_with_own_sets_reproduce_the_layer(n_shared, w):
    """Routing each valid row to the oracle's own expert set reproduces the
    layer's rows (fp64, so only the matmul grouping differs)."""
    inp = random_small(T=30, H=256, E=12, k=3, I=128, n_shared=n_shared, w=w, seed=53,
                       valid_frac=0.7)
    out, r = oracle.moe_forward(inp, return_routing=True)
    rows = np.nonzero(inp.valid.numpy())[0].tolist()
    sets = [r["ids"][t].tolist() for t in rows]
    got = oracle.forward_rows_with_sets(inp, r["x64"], r["logits"], rows, sets)
    assert np.allclose(got, out[rows], rtol=1e-12, atol=1e-15)
