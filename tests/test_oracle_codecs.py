"""Pins for the oracle's number codecs: e4m3 encode/decode, group quantisation, bf16 rounding.

Independent references: torch's float8_e4m3fn and bfloat16 casts (a separate
implementation of the same formats), literal values fixed by the OCP FP8 E4M3
format definition, and the rounding error bound of a 3-bit mantissa.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x):
    t = torch.from_numpy(np.asarray(x, np.float64)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256)
    mine = oracle.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert nan.tolist() == np.isnan(mine).tolist()
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),
    (0x77, 240.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x80, -0.0),
])
def test_e4m3_literal_codes(code, value):
    v = oracle.e4m3_decode([code])[0]
    assert v == value and np.signbit(v) == np.signbit(value)
    assert oracle.e4m3_encode([value])[0] == code


def test_e4m3_roundtrip_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),            # halfway 1.0 | 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),            # halfway 1.125 | 1.25 -> even mantissa (1.25)
    (-1.0625, 0xB8),
    (2.0 ** -10, 0x00),        # halfway 0 | 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),    # halfway 2^-9 | 2^-8 -> code 2
    (15 * 2.0 ** -10, 0x08),   # halfway 7*2^-9 | 2^-6 -> 2^-6 (code 8, even)
    (464.0, 0x7E),             # would round to 480, which is NaN in e4m3fn: saturate
    (1e6, 0x7E), (-1e6, 0xFE), (np.inf, 0x7E),
    (1e-12, 0x00), (-1e-12, 0x80), (-0.0, 0x80),
    (1.06251, 0x39),           # just above the tie
])
def test_e4m3_encode_ties_and_saturation(x, code):
    assert oracle.e4m3_encode([x])[0] == code


def test_e4m3_encode_vs_torch_random():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(50000) * 10.0 ** rng.uniform(-4, 3, 50000),
        rng.uniform(-500, 500, 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),
        oracle.e4m3_decode(np.arange(126)) * (1 + 2.0 ** -30),
    ])
    x = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(oracle.e4m3_encode(x), torch_encode(x))


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-20, 20, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_round(x), ref)


@pytest.mark.parametrize("x,y", [
    (1 + 2.0 ** -8, 1.0),                  # halfway 1 | 1+2^-7 -> even
    (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),    # halfway 1+2^-7 | 1+2^-6 -> even
    (1 + 2.0 ** -8 + 2.0 ** -20, 1 + 2.0 ** -7),
    (-3.0, -3.0),
])
def test_bf16_round_literal(x, y):
    assert oracle.bf16_round(np.float32(x)) == np.float32(y)


def test_quantize_groups_properties():
    rng = np.random.default_rng(11)
    R, C, G = 37, 512, 128
    x = (rng.standard_normal((R, C)) * 10.0 ** rng.uniform(-3, 3, (R, 1))).astype(np.float32)
    x[5, 128:256] = 0.0                       # an all-zero group
    codes, s = oracle.quantize_groups_e4m3(x, G)
    assert codes.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (R, C // G)
    amax = np.abs(x.reshape(R, C // G, G)).max(axis=2)
    nz = amax > 0
    # scale = amax / 448 in fp32, 1 for an all-zero group
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    assert s[5, 1] == 1.0 and np.all(codes[5, 128:256] == 0)
    deq = oracle.dequantize_groups(codes, s, G)
    # the largest element of each group maps to +-448 (code 0x7E / 0xFE)
    for r in range(R):
        for g in range(C // G):
            if nz[r, g]:
                i = np.argmax(np.abs(x[r, g * G:(g + 1) * G]))
                assert codes[r, g * G + i] & 0x7F == 0x7E
    # rounding error: <= 2^-4 relative in the normal range, <= 2^-10 * s below it
    q = np.abs(x.astype(np.float64)) / np.repeat(s, G, axis=1)
    err = np.abs(deq - x)
    normal = q >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * np.repeat(s, G, axis=1)[~normal] * (1 + 1e-6))
    # the codes agree with torch's cast of the same fp32 quotient
    quot = (x.reshape(R, C // G, G) / s[:, :, None]).astype(np.float32).reshape(R, C)
    assert np.array_equal(codes, torch_encode(quot.astype(np.float64)))


def test_dequantize_blocks_layout():
    # one distinct scale per 128x128 block; codes of 1.0 everywhere
    codes = np.full((256, 384), 0x38, np.uint8)
    s = np.arange(1, 7, dtype=np.float32).reshape(2, 3)
    w = oracle.dequantize_blocks(codes, s, 128)
    assert w[0, 0] == 1 and w[0, 200] == 2 and w[0, 383] == 3
    assert w[255, 0] == 4 and w[130, 129] == 5 and w[255, 383] == 6
