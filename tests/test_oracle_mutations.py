"""Each plausible mistake planted in the oracle (on the CPU) must make at
least one pin of test_oracle.py fail.  This guards the pins' strength."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as mo
import tests.test_oracle as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(mo, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _swapped_ffn(X, W13, W2):
    I = W13.shape[0] // 2
    return (mo.silu(X @ W13[I:].T) * (X @ W13[:I].T)) @ W2.T


def _sigmoid_only(z):
    with np.errstate(over="ignore"):   # exp(-z) -> inf gives sigma = 0, as it should
        return 1.0 / (1.0 + np.exp(-z))


def _ties_high(l32_row, k):
    E = l32_row.shape[0]
    return sorted(range(E), key=lambda e: (-float(l32_row[e]), -e))[:k]


def _no_renorm(l_sel):
    l = np.asarray(l_sel, dtype=np.float64)
    u = np.exp(l - l.max())
    return u / (u.sum() + 1.0)


def _unstable_align(ids, E, block_m):
    s, be, off, n = _ORIG_ALIGN(ids, E, block_m)
    s = s.copy()
    for e in range(E):
        seg = s[off[e]:off[e + 1]]
        real = seg[seg >= 0][::-1]
        seg[:real.size] = real
    return s, be, off, n


_ORIG_ALIGN = mo.align
_ORIG_TABLE = mo._E4M3


def _bad_bias_decode(codes):
    t = _ORIG_TABLE.copy()
    t = t * 0.5
    return t[np.asarray(codes, dtype=np.uint8)]


def _transposed_scales(codes, scales, block=128):
    q = mo.e4m3fn_decode(codes)
    s = np.asarray(scales, dtype=np.float64).T
    return q * np.repeat(np.repeat(s, block, axis=0), block, axis=1)


def _delta_wrong_exponent(x64, R64):
    rn = np.sqrt((R64 * R64).sum(axis=1)).max()
    return (2.0 ** -10) * np.sqrt((x64 * x64).sum(axis=1)) * rn


def _delta_l1_rows(x64, R64):
    rn = np.sqrt((R64 * R64).sum(axis=1)).max()
    return (2.0 ** -20) * np.abs(x64).sum(axis=1) * rn


def _delta_min_router_norm(x64, R64):
    rn = np.sqrt((R64 * R64).sum(axis=1)).min()
    return (2.0 ** -20) * np.sqrt((x64 * x64).sum(axis=1)) * rn


def _ties_top_k_only(logits64, k, delta, valid=None):
    T, E = logits64.shape
    out = []
    for t in range(T):
        if valid is not None and not valid[t]:
            continue
        srt = np.sort(logits64[t])[::-1][:k]          # misses the (k+1)-th
        if np.any(np.diff(-srt) < delta[t]):
            out.append(t)
    return np.asarray(out, dtype=np.int64)


def _ties_ignore_valid(logits64, k, delta, valid=None):
    return _ORIG_NEAR(logits64, k, delta, None)


def _sets_without_shared(inp, x64, logits64, rows, sets):
    cfg = inp.cfg
    res = np.zeros((len(rows), cfg.H))
    for i, (t, s) in enumerate(zip(rows, sets)):
        s = list(s)
        for e, c in zip(s, mo.topk_weights(logits64[t, s])):
            W13, W2 = mo.expert_weights_f64(inp, e)
            res[i] += c * mo.expert_ffn(x64[t:t + 1], W13, W2)[0]
    return res


def _sets_wrong_row(inp, x64, logits64, rows, sets):
    # the i-th listed row's output computed from x row i instead of row rows[i]
    return _ORIG_SETS(inp, x64, logits64, list(range(len(rows))), sets)


_ORIG_NEAR = mo.near_tie_rows
_ORIG_SETS = mo.forward_rows_with_sets

MUTANTS = [
    ("expert_ffn", _swapped_ffn, [pins.test_hand_worked_layer_example]),
    ("silu", _sigmoid_only, [pins.test_silu_closed_forms]),
    ("select_topk", _ties_high, [pins.test_duplicate_router_rows_tie_to_lower_id]),
    ("topk_weights", _no_renorm, [pins.test_topk_weight_closed_forms]),
    ("align", _unstable_align, [lambda: pins.test_align_matches_comparison_sort(2, 16)]),
    ("e4m3fn_decode", _bad_bias_decode, [pins.test_fp8_table_matches_torch_cast_all_codes]),
    ("dequant_block_scaled", _transposed_scales, [pins.test_fp8_golden_codes_and_block_scales]),
    ("tie_threshold", _delta_wrong_exponent, [pins.test_tie_threshold_hand_worked]),
    ("tie_threshold", _delta_l1_rows, [pins.test_tie_threshold_hand_worked]),
    ("tie_threshold", _delta_min_router_norm, [pins.test_tie_threshold_hand_worked]),
    ("near_tie_rows", _ties_top_k_only, [pins.test_near_tie_rows_constructed_gaps]),
    ("near_tie_rows", _ties_ignore_valid, [pins.test_near_tie_rows_constructed_gaps]),
    ("forward_rows_with_sets", _sets_without_shared, [pins.test_alternate_set_row_hand_worked]),
    ("forward_rows_with_sets", _sets_wrong_row, [pins.test_alternate_set_row_hand_worked]),
]


@pytest.mark.parametrize("name,fn,checks", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, checks):
    _patch(monkeypatch, name, fn)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


def test_forgotten_shared_expert_is_caught(monkeypatch):
    orig = mo.moe_forward

    def no_shared(inp, return_routing=False):
        cfg = inp.cfg
        if cfg.n_shared:
            inp = type(inp)(cfg=cfg.with_(n_shared=0), x=inp.x, valid=inp.valid,
                            router=inp.router, w13=inp.w13[:cfg.E], w2=inp.w2[:cfg.E])
        return orig(inp, return_routing)

    _patch(monkeypatch, "moe_forward", no_shared)
    with pytest.raises(AssertionError):
        pins.test_shared_expert_adds_with_weight_one()
