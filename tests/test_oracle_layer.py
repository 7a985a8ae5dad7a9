"""Pins for the oracle's layer: out[t] = sum_j w[t,j] W2[e] (SiLU(W13g[e] x_t) * W13u[e] x_t).

References that are not the oracle: a closed-form worked example, a dense
SwiGLU MLP written with torch CPU ops (torch.nn.functional.linear / silu), the
mean of all experts' MLPs, permutation equivariance, linearity in the routing
weights, and torch's float8 cast for the fp8 activation quantisation.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from moe_inputs import get_config, make_case


def dense_swiglu_mlp(x, w13_e, w2_e):
    """Textbook SwiGLU MLP (gate first, then up): W2 (silu(Wg x) * (Wu x))."""
    x = torch.as_tensor(np.asarray(x, np.float64))
    w13 = torch.as_tensor(np.asarray(w13_e, np.float64))
    wg, wu = w13.chunk(2, dim=0)
    h = F.silu(F.linear(x, wg)) * F.linear(x, wu)
    return F.linear(h, torch.as_tensor(np.asarray(w2_e, np.float64))).numpy()


def rand_problem(rng, T, H, I, E, k, distinct=True):
    x = rng.standard_normal((T, H))
    w13 = 0.3 * rng.standard_normal((E, 2 * I, H))
    w2 = 0.3 * rng.standard_normal((E, H, I))
    if distinct:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    else:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k))
    return x, ids, w, w13, w2


def test_closed_form_worked_example():
    """H=2, I=1, E=2, top_k=2; every value written out by hand."""
    silu = lambda v: v / (1 + math.exp(-v))   # noqa: E731
    x = np.array([[1.0, 2.0], [-1.0, 4.0]])
    w13 = np.array([[[1.0, 0.0], [1.0, 0.5]],       # expert 0: gate row, up row
                    [[-1.0, 0.0], [0.0, 0.25]]])    # expert 1
    w2 = np.array([[[1.0], [3.0]],
                   [[2.0], [-4.0]]])
    ids = np.array([[0, 1], [1, 0]], np.int32)
    w = np.array([[0.25, 0.75], [0.6, 0.4]])
    # token 0: e0 g=1, u=2 ; e1 g=-1, u=0.5
    # token 1: e1 g=1, u=1 ; e0 g=-1, u=1
    a00, a01 = 2 * silu(1), 0.5 * silu(-1)
    a11, a10 = 1 * silu(1), 1 * silu(-1)
    expect = np.array([
        [0.25 * a00 * 1 + 0.75 * a01 * 2, 0.25 * a00 * 3 + 0.75 * a01 * -4],
        [0.6 * a11 * 2 + 0.4 * a10 * 1, 0.6 * a11 * -4 + 0.4 * a10 * 3],
    ])
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    np.testing.assert_allclose(out, expect, rtol=1e-15, atol=0)


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    v = oracle.silu(-800.0)
    assert v == 0.0 and np.signbit(v) and not np.isnan(v)
    g = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(oracle.silu(g), F.silu(torch.as_tensor(g)).numpy(), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("E", [1, 5])
def test_dense_reduction_top1_weight1(E):
    """Every token routed to one expert with weight 1 equals the dense MLP of that expert."""
    rng = np.random.default_rng(1)
    T, H, I = 13, 24, 40
    x, _, _, w13, w2 = rand_problem(rng, T, H, I, E, 1)
    ids = rng.integers(0, E, (T, 1)).astype(np.int32)
    w = np.ones((T, 1))
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    for t in range(T):
        ref = dense_swiglu_mlp(x[t:t + 1], w13[ids[t, 0]], w2[ids[t, 0]])[0]
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-12)


def test_top_k_equals_E_mean_of_experts():
    rng = np.random.default_rng(2)
    T, H, I, E = 9, 16, 32, 4
    x, _, _, w13, w2 = rand_problem(rng, T, H, I, E, E)
    ids = np.stack([rng.permutation(E) for _ in range(T)]).astype(np.int32)
    w = np.full((T, E), 1.0 / E)
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    ref = np.mean([dense_swiglu_mlp(x, w13[e], w2[e]) for e in range(E)], axis=0)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_weighted_sum_of_dense_mlps():
    """General routing (duplicates allowed) equals the explicit sum over j of w * MLP_e(x)."""
    rng = np.random.default_rng(3)
    T, H, I, E, k = 11, 20, 36, 6, 3
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k, distinct=False)
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    ref = np.zeros_like(out)
    for t in range(T):
        for j in range(k):
            ref[t] += w[t, j] * dense_swiglu_mlp(x[t:t + 1], w13[ids[t, j]], w2[ids[t, j]])[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_permutation_equivariance():
    rng = np.random.default_rng(4)
    T, H, I, E, k = 23, 16, 24, 5, 2
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k)
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    p = rng.permutation(T)
    out_p = oracle.moe_layer(x[p], ids[p], w[p], (w13, w2))
    np.testing.assert_allclose(out_p, out[p], rtol=1e-13, atol=1e-13)


def test_linearity_in_routing_weights():
    rng = np.random.default_rng(5)
    T, H, I, E, k = 10, 16, 24, 4, 2
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k)
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    assert np.array_equal(oracle.moe_layer(x, ids, 2 * w, (w13, w2)), 2 * out)
    assert np.all(oracle.moe_layer(x, ids, 0 * w, (w13, w2)) == 0)


def test_identical_experts():
    rng = np.random.default_rng(6)
    T, H, I, E, k = 8, 12, 20, 3, 2
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k)
    w13[:] = w13[0]
    w2[:] = w2[0]
    out = oracle.moe_layer(x, ids, w, (w13, w2))
    ref = w.sum(axis=1, keepdims=True) * dense_swiglu_mlp(x, w13[0], w2[0])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_invalid_ids_contribute_nothing():
    rng = np.random.default_rng(8)
    T, H, I, E, k = 6, 8, 16, 3, 2
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k)
    bad = ids.copy()
    bad[:, 1] = 7
    out = oracle.moe_layer(x, bad, w, (w13, w2))
    ref = oracle.moe_layer(x, ids[:, :1], w[:, :1], (w13, w2))
    np.testing.assert_allclose(out, ref, rtol=1e-15, atol=0)


def test_token_subset_matches_full():
    rng = np.random.default_rng(9)
    T, H, I, E, k = 30, 16, 24, 5, 3
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k)
    full = oracle.moe_layer(x, ids, w, (w13, w2))
    sub = [29, 3, 17]
    np.testing.assert_allclose(oracle.moe_layer(x, ids, w, (w13, w2), tokens=sub), full[sub],
                               rtol=1e-13, atol=1e-13)


def test_combine_order_and_rounding():
    """Ascending-j fp32 accumulation on values where the order changes the result."""
    y = np.array([[1e8], [1.0], [-1e8], [1.0]], np.float32)      # one token, k=4
    assert oracle.combine(y, 4, np.float32)[0, 0] == np.float32(1.0)   # ((1e8+1)-1e8)+1 in fp32
    assert oracle.combine(y, 4, np.float64)[0, 0] == 2.0
    y2 = np.array([[3.0], [5.0], [7.0], [11.0]])
    assert oracle.combine(y2, 2, np.float64).ravel().tolist() == [8.0, 18.0]


def test_fp8_layer_vs_torch_quantisation_chain():
    """fp8 layer against a chain built from torch ops: dequantised weights, X and
    the activation quantised per 128-group with torch's float8_e4m3fn cast."""
    cfg = get_config("dsv3_fp8_e4m3", T=6, H=256, I=256, E=3, top_k=2)
    case = make_case(cfg, "cpu", seed=1)
    x = case.x_host()
    w13c, w2c, s13, s2 = case.weights_host()
    out = oracle.moe_layer(x, case.ids_host, case.w_host, (w13c, w2c, s13, s2), fp8=True)

    def tq(v, G=128):
        v = torch.as_tensor(np.asarray(v, np.float32))
        R, C = v.shape
        g = v.reshape(R, C // G, G)
        amax = g.abs().amax(dim=2)
        s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
        q = (g / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * s.double()[:, :, None]).reshape(R, C)

    W13 = (case.w13.to(torch.float64).reshape(3, 4, 128, 2, 128)
           * case.w13_scales.double()[:, :, None, :, None]).reshape(3, 512, 256)
    W2 = (case.w2.to(torch.float64).reshape(3, 2, 128, 2, 128)
          * case.w2_scales.double()[:, :, None, :, None]).reshape(3, 256, 256)
    xd = tq(x)
    ref = torch.zeros((6, 256), dtype=torch.float64)
    for t in range(6):
        for j in range(2):
            e = int(case.ids_host[t, j])
            wg, wu = W13[e].chunk(2, dim=0)
            a = F.silu(F.linear(xd[t:t + 1], wg)) * F.linear(xd[t:t + 1], wu)
            a = tq(a.numpy())
            ref[t] += float(case.w_host[t, j]) * F.linear(a, W2[e])[0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fp8", [False, True])
def test_expert_threads_bit_identical(fp8):
    """Evaluating the experts on several threads changes nothing: each expert's arithmetic
    and the combine order are the same."""
    rng = np.random.default_rng(31)
    T, H, I, E, k = 37, 256, 128, 9, 3
    x, ids, w, w13, w2 = rand_problem(rng, T, H, I, E, k, distinct=False)
    ids[5, 1] = E                       # an excluded id
    if fp8:
        c13 = rng.integers(0, 126, (E, 2 * I, H)).astype(np.uint8)
        c2 = rng.integers(0, 126, (E, H, I)).astype(np.uint8)
        s13 = rng.uniform(1e-3, 1e-2, (E, 2 * I // 128, H // 128))
        s2 = rng.uniform(1e-3, 1e-2, (E, H // 128, I // 128))
        experts = (c13, c2, s13, s2)
    else:
        experts = (w13, w2)
    one, slots1 = oracle.moe_layer(x, ids, w, experts, E, fp8=fp8, return_slots=True)
    many, slots8 = oracle.moe_layer(x, ids, w, experts, E, fp8=fp8, return_slots=True, workers=8)
    assert np.array_equal(one, many) and np.array_equal(slots1, slots8)
