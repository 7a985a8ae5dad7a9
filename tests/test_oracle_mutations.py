"""Plant plausible mistakes in the oracle (CPU only) and check that a pin catches each.

Each mutant replaces one oracle function with a subtly wrong copy; the pins in
test_oracle_layer / test_oracle_align must then fail.
"""
import numpy as np
import pytest

import oracle
from oracle import moe_oracle as mo
import test_oracle_align as ta
import test_oracle_layer as tl


def _up_swapped(x_rows, w13_e):
    x_rows = np.asarray(x_rows, np.float64)
    I = w13_e.shape[0] // 2
    return mo.silu(x_rows @ w13_e[I:].T) * (x_rows @ w13_e[:I].T)


def _up_wrong_silu(x_rows, w13_e):
    x_rows = np.asarray(x_rows, np.float64)
    I = w13_e.shape[0] // 2
    g = x_rows @ w13_e[:I].T
    return g / (1.0 + np.exp(g)) * (x_rows @ w13_e[I:].T)


def _down_transposed(act, w2_e):
    w = np.asarray(w2_e, np.float64)
    return np.asarray(act, np.float64) @ w.reshape(w.shape[1], w.shape[0])


def _combine_drops_last(slot_out, top_k, acc_dtype=np.float64):
    y = np.asarray(slot_out)
    T = y.shape[0] // top_k
    acc = np.zeros((T, y.shape[1]), acc_dtype)
    for j in range(max(top_k - 1, 1)):
        acc = acc + y[j::top_k]
    return acc


LAYER_MUTANTS = {
    "gate_up_swapped": ("expert_up", _up_swapped),
    "silu_sign": ("expert_up", _up_wrong_silu),
    "w2_transposed_layout": ("expert_down", _down_transposed),
    "combine_drops_slot": ("combine", _combine_drops_last),
}

LAYER_PINS = [tl.test_closed_form_worked_example,
              lambda: tl.test_dense_reduction_top1_weight1(5),
              tl.test_top_k_equals_E_mean_of_experts,
              tl.test_weighted_sum_of_dense_mlps]


def _some_pin_fails(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", list(LAYER_MUTANTS))
def test_layer_mutant_is_caught(name, monkeypatch):
    attr, fn = LAYER_MUTANTS[name]
    monkeypatch.setattr(mo, attr, fn)
    assert _some_pin_fails(LAYER_PINS), f"no pin caught mutant {name}"


def _gather_token_mod(x, topk_ids, topk_weights, experts, num_experts=None, **kw):
    # wrong gather: token = slot % k instead of slot // k
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    x = np.asarray(x, np.float64)
    idx = [(t * k + j) % T for t in range(T) for j in range(k)]
    return _ORIG_LAYER(x[np.array(idx[::k])], topk_ids, topk_weights, experts, num_experts, **kw)


_ORIG_LAYER = mo.moe_layer


def test_wrong_gather_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "moe_layer", _gather_token_mod)
    assert _some_pin_fails([tl.test_permutation_equivariance, tl.test_closed_form_worked_example])


def _align_unstable(topk_ids, num_experts, block_m):
    a = _ORIG_ALIGN(topk_ids, num_experts, block_m)
    # reverse each expert's segment (a non-stable order)
    for e in range(num_experts):
        lo, n = a.offsets[e], a.counts[e]
        seg = a.sorted_slots[lo:lo + n][::-1].copy()
        a.sorted_slots[lo:lo + n] = seg
        a.slot_row[seg] = np.arange(lo, lo + n)
    return a


def _align_no_padding(topk_ids, num_experts, block_m):
    a = _ORIG_ALIGN(topk_ids, num_experts, 1)
    return a


_ORIG_ALIGN = mo.align


@pytest.mark.parametrize("mutant", [_align_unstable, _align_no_padding])
def test_align_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "align", mutant)
    import json
    cases = json.load(open(ta.GOLDEN))["cases"]
    pins = [lambda c=c: ta.test_align_worked_examples(c) for c in cases]
    pins += [lambda: ta.test_align_matches_brute_force(*next(iter(ta.adversarial_routings())))]
    assert _some_pin_fails(pins)


# ---- routing -----------------------------------------------------------------------------
import test_oracle_route as tr  # noqa: E402

_ORIG_ROUTE = mo.route


def _route_ties_high(logits, top_k, renormalize):
    # ties broken toward the higher id
    lg = np.asarray(logits, np.float64)
    ids, w = _ORIG_ROUTE(lg[:, ::-1], top_k, renormalize)
    return (lg.shape[1] - 1 - ids).astype(np.int32), w


def _route_ascending(logits, top_k, renormalize):
    ids, w = _ORIG_ROUTE(-np.asarray(logits, np.float64), top_k, renormalize)
    lg = np.asarray(logits, np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def _route_never_renormalises(logits, top_k, renormalize):
    return _ORIG_ROUTE(logits, top_k, False)


def _route_always_renormalises(logits, top_k, renormalize):
    return _ORIG_ROUTE(logits, top_k, True)


ROUTE_PINS = [tr.test_worked_example_ties_no_renorm, tr.test_worked_example_renormalised_subset,
              tr.test_renormalised_pair_is_a_logistic, tr.test_selection_matches_brute_force,
              tr.test_weights_are_the_softmax_probabilities]


@pytest.mark.parametrize("mutant", [_route_ties_high, _route_ascending, _route_never_renormalises,
                                    _route_always_renormalises])
def test_route_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "route", mutant)
    assert _some_pin_fails(ROUTE_PINS)


# ---------------------------------------------------------------------------------------------
# MXFP4 up projection
# ---------------------------------------------------------------------------------------------
from oracle import mx_oracle as mx  # noqa: E402
import test_oracle_mx as tm  # noqa: E402


def _unpack_swapped(packed):
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b >> 4
    out[..., 1::2] = b & 0xF
    return out


def _decode_block16(packed, scales, block=32):
    vals = mx.e2m1_value(mx.unpack_e2m1(packed))
    sc = mx.e8m0_value(scales)
    idx = np.minimum(np.arange(vals.shape[-1]) // 16, sc.shape[-1] - 1)
    return vals * sc[..., idx]


def _swiglu_no_plus_one(gate, linear, alpha, limit):
    g = np.minimum(np.asarray(gate, np.float64), limit)
    lin = np.clip(np.asarray(linear, np.float64), -limit, limit)
    return g / (1.0 + np.exp(-alpha * g)) * lin


def _swiglu_gate_clamped_both_sides(gate, linear, alpha, limit):
    g = np.clip(np.asarray(gate, np.float64), -limit, limit)
    lin = np.clip(np.asarray(linear, np.float64), -limit, limit)
    return g / (1.0 + np.exp(-alpha * g)) * (lin + 1.0)


def _up_pairs_swapped(x_rows, w_packed_e, w_scales_e, bias_e, x_scale, alpha, limit):
    w = mx.mx_decode(w_packed_e, w_scales_e)
    h = (np.asarray(x_rows, np.float64) @ w.T) * float(x_scale) + np.asarray(bias_e, np.float64)
    return mx.gptoss_swiglu(h[:, 1::2], h[:, 0::2], alpha, limit)


def _up_bias_unscaled_order(x_rows, w_packed_e, w_scales_e, bias_e, x_scale, alpha, limit):
    w = mx.mx_decode(w_packed_e, w_scales_e)
    h = ((np.asarray(x_rows, np.float64) @ w.T) + np.asarray(bias_e, np.float64)) * float(x_scale)
    return mx.gptoss_swiglu(h[:, 0::2], h[:, 1::2], alpha, limit)


MX_MUTANTS = {
    "nibble_order": ("unpack_e2m1", _unpack_swapped),
    "scale_block_16": ("mx_decode", _decode_block16),
    "no_plus_one": ("gptoss_swiglu", _swiglu_no_plus_one),
    "gate_clamped_below": ("gptoss_swiglu", _swiglu_gate_clamped_both_sides),
    "gate_linear_swapped": ("expert_up_mxfp4", _up_pairs_swapped),
    "bias_scaled": ("expert_up_mxfp4", _up_bias_unscaled_order),
}

MX_PINS = [tm.test_mx_decode_worked_example, tm.test_decode_of_generator_quantiser_is_nearest_value,
           tm.test_swiglu_closed_forms, tm.test_swiglu_without_limit_is_silu_times_linear_plus_one,
           tm.test_top1_against_dense_torch, tm.test_invariants]


@pytest.mark.parametrize("name", list(MX_MUTANTS))
def test_mx_mutant_is_caught(name, monkeypatch):
    attr, fn = MX_MUTANTS[name]
    monkeypatch.setattr(mx, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _some_pin_fails(MX_PINS), f"no pin caught mutant {name}"
