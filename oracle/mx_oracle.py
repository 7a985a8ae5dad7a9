"""Plain CPU definition of the MXFP4 up projection with the GPT-OSS SwiGLU.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, smoke() and the
benchmark's cpu_baseline leg use it; the product path never does.

Source (page title as published): "MOE Bmm1 Fused Gather", the example's own
variant of the first expert GEMM:
  [mma]      mma_partition: the expert weights are e2m1 ("fp4") values with
             block scales along K (the microscale block of the config is 32),
             multiplied by the e4m3 gathered activations, fp32 accumulation;
  [bias]     apply_bias_and_scale / epilogue_partition: the accumulator is
             multiplied by x_scale * w_scale (the activation's and the weight's
             per-tensor scales; the weights carry none beyond their microscales
             here) and the expert's bias row is added;
  [swiglu]   _swiglu_step1 / _swiglu_step2: the 2I accumulator columns come in
             (gate, linear) pairs -- even column gate, odd column linear; the
             gate is capped at `limit` from above, the linear part is clamped to
             [-limit, limit]; act = gate / (1 + exp(-alpha * gate)) computed
             as shown, and the output is act * linear + act, i.e.
             act * (linear + 1);
  [fp8-out]  pack_fp8_out_fragment / epilogue_partition: the output is
             multiplied by 1 / out_scale and converted to e4m3 with
             round-to-nearest-even and saturation to the largest finite value;
  [rows]     load_activations: slot r of an expert-sorted slice reads token
             row gather_indx = slot // top_k.
  [case]     prepare_case: x e4m3, w e2m1 with microscales along K, fp32 bias
             [E, 2I], alpha in [1, 1.2), limit in [1.3, 1.5), x_scale in
             [0.5, 1.5), out scale in [3.5, 4.5).

The formats themselves follow the OCP Microscaling (MX) specification, which
the page names through its "mxfp4" and "e8m0"-scaled inputs:
  * e2m1: bits s.ee.m, exponent bias 1; exponent 0 holds the subnormals
    m * 0.5; no infinity or NaN; largest magnitude 6;
  * e8m0: an unsigned biased exponent, value 2^(c - 127); code 255 is NaN;
  * two e2m1 elements per byte, the element with the lower K index in the
    low nibble (the layout of torch's float4_e2m1fn_x2).

Reading where the page leaves a choice open: the weights are stored as
W13[E, 2I, H/2] bytes (row n = accumulator column n, K contiguous) with scales
[E, 2I, H/32]; the page's [E, H, 2I] holds the same numbers transposed.
Everything is float64 here; the fp8 output code is the e4m3 rounding of the
float64 act / out_scale.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from .moe_oracle import e4m3_decode, e4m3_encode

MX_BLOCK = 32


def e2m1_value(codes) -> np.ndarray:
    """Value of each 4-bit e2m1 code (0..15) as float64, from the bit layout s.ee.m."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    ex = (c >> 1) & 0x3
    man = (c & 1).astype(np.float64)
    normal = (1.0 + man / 2.0) * np.exp2(ex.astype(np.float64) - 1.0)
    sub = man * 0.5
    return sign * np.where(ex == 0, sub, normal)


def e8m0_value(codes) -> np.ndarray:
    """Value of each e8m0 scale code: 2^(c - 127); 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def unpack_e2m1(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2i is the low nibble of byte i."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def mx_decode(packed, scales, block: int = MX_BLOCK) -> np.ndarray:
    """Dequantise MXFP4 rows: value[r, k] = e2m1(code[r, k]) * e8m0(scale[r, k // block])."""
    vals = e2m1_value(unpack_e2m1(packed))
    sc = e8m0_value(scales)
    K = vals.shape[-1]
    if sc.shape[-1] * block != K:
        raise ValueError(f"{sc.shape[-1]} scales per row do not cover K = {K}")
    return vals * np.repeat(sc, block, axis=-1)


def gptoss_swiglu(gate, linear, alpha: float, limit: float) -> np.ndarray:
    """[swiglu]: gate capped at limit, linear clamped to [-limit, limit],
    out = gate / (1 + exp(-alpha * gate)) * (linear + 1)."""
    g = np.minimum(np.asarray(gate, dtype=np.float64), limit)
    lin = np.clip(np.asarray(linear, dtype=np.float64), -limit, limit)
    act = g / (1.0 + np.exp(-alpha * g))
    return act * (lin + 1.0)


def expert_up_mxfp4(x_rows, w_packed_e, w_scales_e, bias_e, x_scale: float, alpha: float,
                    limit: float) -> np.ndarray:
    """One expert: x_rows [n, H] (float64 values of the e4m3 codes) -> act [n, I].

    h = x_scale * (W13[e] . x) + bias[e]  ([mma], [bias]); columns (2i, 2i+1) are
    (gate_i, linear_i) ([swiglu]).
    """
    w = mx_decode(w_packed_e, w_scales_e)                      # [2I, H]
    h = (np.asarray(x_rows, dtype=np.float64) @ w.T) * float(x_scale) + np.asarray(bias_e, np.float64)
    return gptoss_swiglu(h[:, 0::2], h[:, 1::2], alpha, limit)


def moe_up_mxfp4(x_codes, x_scale: float, topk_ids, w_packed, w_scales, bias, alpha: float,
                 limit: float, num_experts: Optional[int] = None,
                 slots: Optional[Sequence[int]] = None) -> np.ndarray:
    """act[s] for every flat slot s = t*top_k + j whose id is a local expert, float64 [N, I]
    (rows of excluded slots are NaN).  `slots` limits the work to those slots (the returned
    array still has N rows; the others stay NaN).

    w_packed [E, 2I, H/2] uint8, w_scales [E, 2I, H/32] uint8 (or a callable e -> (packed,
    scales)), bias [E, 2I] float.
    """
    xc = np.asarray(x_codes)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    N = T * k
    if callable(w_packed):
        get = w_packed
        E = int(num_experts)
    else:
        E = int(np.asarray(w_packed).shape[0]) if num_experts is None else int(num_experts)

        def get(e):
            return w_packed[e], w_scales[e]
    flat = ids.reshape(-1)
    todo = np.arange(N) if slots is None else np.asarray(sorted(set(int(s) for s in slots)))
    I2 = None
    out = None
    for e in range(E):
        sel = todo[flat[todo] == e]
        if sel.size == 0:
            continue
        wp, ws = get(e)
        rows = e4m3_decode(xc[sel // k])                      # [rows]: token = slot // top_k
        act = expert_up_mxfp4(rows, wp, ws, np.asarray(bias)[e], x_scale, alpha, limit)
        if out is None:
            I2 = act.shape[1]
            out = np.full((N, I2), np.nan)
        out[sel] = act
    if out is None:
        H2 = np.asarray(get(0)[0]).shape[0] if E > 0 else 0
        out = np.full((N, H2 // 2), np.nan)
    return out


def quantize_out_e4m3(act, out_scale: float) -> np.ndarray:
    """[fp8-out]: e4m3 code of act / out_scale (round to nearest even, saturating)."""
    return e4m3_encode(np.asarray(act, dtype=np.float64) / float(out_scale))
