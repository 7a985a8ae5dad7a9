"""Pins for the oracle's MXFP4 up projection with the GPT-OSS SwiGLU (oracle.mx_oracle).

What ties it to something other than itself:
  * the e2m1 values against the literal list of the format's 16 values, the e8m0 decode
    against torch's float8_e8m0fnu cast;
  * the packed decode against a hand-worked example (nibble order, one scale per 32 values);
  * decode(mx_quantize(w)) against brute force: the input generator's quantiser (a separate
    implementation) must give, for every element, the representable value nearest to w / 2^e
    (ties to the even code), with e the OCP rule's shared exponent;
  * the SwiGLU against closed forms (saturated gate and linear part, zeros, the lower side of
    the gate left unclamped) and, with limit = inf and alpha = 1, against torch's SiLU;
  * the whole projection against a dense per-token torch computation for top-1 routing, and
    against invariants (permutation of tokens, excluded ids, a zero x gives swiglu(bias)).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import mx_quantize


def test_e2m1_values():
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert oracle.e2m1_value(np.arange(8)).tolist() == pos
    assert oracle.e2m1_value(np.arange(8, 16)).tolist() == [-v for v in pos]


def test_e8m0_values_against_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(oracle.e8m0_value(codes), ref)
    assert np.isnan(oracle.e8m0_value([255])[0])
    assert oracle.e8m0_value([127, 128, 126]).tolist() == [1.0, 2.0, 0.5]


def test_mx_decode_worked_example():
    # one row of K = 64: block 0 scale 2^0, block 1 scale 2^2.
    # byte 0 = 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    # byte 1 = 0x9F: element 2 = code 15 (-6), element 3 = code 9 (-0.5)
    # byte 16 = 0x07: element 32 = code 7 (6) * 4 = 24, element 33 = 0
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0], packed[0, 1], packed[0, 16] = 0x21, 0x9F, 0x07
    out = oracle.mx_decode(packed, np.array([[127, 129]], np.uint8))
    want = np.zeros((1, 64))
    want[0, :4] = [0.5, 1.0, -6.0, -0.5]
    want[0, 32] = 24.0
    assert np.array_equal(out, want)


def _nearest_e2m1(a):
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.minimum(np.abs(a), 6.0)
    d = np.abs(a[..., None] - mags)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    # ties: the even code (of the two candidates at most one is even)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    any_ = cand.min(axis=-1)
    idx = np.where((d == best).sum(axis=-1) > 1, even, any_)
    return mags[idx]


def test_decode_of_generator_quantiser_is_nearest_value():
    g = torch.Generator().manual_seed(4)
    w = torch.randn(64, 256, generator=g) * torch.exp(torch.randn(64, 1, generator=g))
    w[3, :32] = 0.0                                   # an all-zero block
    w[5, 40] = 1e-3                                   # tiny next to larger values
    w[7, :32] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4)   # exact ties
    p, s = mx_quantize(w)
    dec = oracle.mx_decode(p.numpy(), s.numpy())
    wn = w.double().numpy()
    blocks = wn.reshape(64, 8, 32)
    amax = np.abs(blocks).max(axis=2)
    ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    scale = np.exp2(ex)
    q = blocks / scale[:, :, None]
    want = (np.sign(q) * _nearest_e2m1(q) * scale[:, :, None]).reshape(64, 256)
    assert np.array_equal(dec, want)
    assert np.array_equal(s.numpy(), (ex + 127).astype(np.uint8))
    assert (dec[3, :32] == 0).all()
    # the worked ties: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4, 7->6 (saturated)
    assert dec[7, :8].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]


def test_swiglu_closed_forms():
    a, lim = 1.15, 1.4
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))   # noqa: E731
    # gate and linear both above the limit: limit * sigma(alpha * limit) * (limit + 1)
    v = oracle.gptoss_swiglu([5.0], [9.0], a, lim)[0]
    assert v == pytest.approx(lim * sig(a * lim) * (lim + 1), rel=1e-15)
    # linear below -limit: factor (1 - limit); the gate is not clamped from below
    v = oracle.gptoss_swiglu([-2.0], [-3.0], a, lim)[0]
    assert v == pytest.approx(-2.0 * sig(-2.0 * a) * (1 - lim), rel=1e-15)
    # zero gate or linear = -1 give zero
    assert oracle.gptoss_swiglu([0.0], [0.7], a, lim)[0] == 0.0
    assert oracle.gptoss_swiglu([0.9], [-1.0], a, lim)[0] == 0.0


def test_swiglu_without_limit_is_silu_times_linear_plus_one():
    g = torch.linspace(-8, 8, 101, dtype=torch.float64)
    lin = torch.linspace(3, -3, 101, dtype=torch.float64)
    ref = torch.nn.functional.silu(g) * (lin + 1)
    got = oracle.gptoss_swiglu(g.numpy(), lin.numpy(), 1.0, float("inf"))
    assert np.allclose(got, ref.numpy(), rtol=1e-14, atol=1e-15)


def _small_case(T=24, H=128, I=64, E=3, k=1, seed=0):
    rng = np.random.default_rng(seed)
    w = torch.from_numpy(rng.standard_normal((E, 2 * I, H)).astype(np.float32) * 0.1)
    packed, scales = zip(*[mx_quantize(w[e]) for e in range(E)])
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
    xc = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    bias = rng.standard_normal((E, 2 * I))
    return (xc, ids, np.stack([p.numpy() for p in packed]), np.stack([s.numpy() for s in scales]),
            bias)


def test_top1_against_dense_torch():
    """Top-1, per token: h = x_scale * W13[e] x + b; act_i = swiglu(h[2i], h[2i+1]).  The dense
    reference uses torch's own e4m3 decode of X and torch matmul/sigmoid in float64."""
    xc, ids, wp, ws, bias = _small_case()
    xs, alpha, lim = 0.8, 1.1, 1.4
    got = oracle.moe_up_mxfp4(xc, xs, ids, wp, ws, bias, alpha, lim)
    x = torch.from_numpy(xc).view(torch.float8_e4m3fn).to(torch.float64)
    for t in range(xc.shape[0]):
        e = int(ids[t, 0])
        w = torch.from_numpy(oracle.mx_decode(wp[e], ws[e]))
        h = xs * (w @ x[t]) + torch.from_numpy(bias[e])
        g = torch.clamp(h[0::2], max=lim)
        lin = torch.clamp(h[1::2], min=-lim, max=lim)
        ref = g * torch.sigmoid(alpha * g) * (lin + 1)
        assert np.allclose(got[t], ref.numpy(), rtol=1e-12, atol=1e-12), t


def test_invariants():
    xc, ids, wp, ws, bias = _small_case(T=20, k=2, E=4, seed=3)
    args = (0.9, ids, wp, ws, bias, 1.05, 1.45)
    base = oracle.moe_up_mxfp4(xc, *args)
    # permuting tokens permutes slot rows
    perm = np.random.default_rng(1).permutation(20)
    got = oracle.moe_up_mxfp4(xc[perm], 0.9, ids[perm], wp, ws, bias, 1.05, 1.45)
    slot_perm = (perm[:, None] * 2 + np.arange(2)).reshape(-1)
    assert np.array_equal(got, base[slot_perm])
    # an excluded id gives a NaN row and leaves the others alone
    ids2 = ids.copy()
    ids2[4, 1] = 4
    got = oracle.moe_up_mxfp4(xc, 0.9, ids2, wp, ws, bias, 1.05, 1.45)
    assert np.isnan(got[9]).all()
    keep = np.ones(40, bool)
    keep[9] = False
    assert np.array_equal(got[keep], base[keep])
    # x = 0: every slot row is swiglu(bias of its expert)
    got = oracle.moe_up_mxfp4(np.zeros_like(xc), 0.9, ids, wp, ws, bias, 1.05, 1.45)
    for s in range(40):
        e = ids.reshape(-1)[s]
        ref = oracle.gptoss_swiglu(bias[e, 0::2], bias[e, 1::2], 1.05, 1.45)
        assert np.array_equal(got[s], ref)
    # slot subsets
    sub = oracle.moe_up_mxfp4(xc, *args, slots=[3, 17])
    assert np.array_equal(sub[[3, 17]], base[[3, 17]])
    assert np.isnan(sub[0]).all()


def test_output_code_is_the_e4m3_rounding_of_act_over_scale():
    act = np.array([0.0, 1.0, -2.5, 1e6, 3.9 * 0.7])
    codes = oracle.quantize_out_e4m3(act, 3.9)
    assert np.array_equal(codes, oracle.e4m3_encode(act / 3.9))
    assert oracle.e4m3_decode(codes)[3] == 448.0
