"""CPU oracle for the routed grouped-GEMM top-k MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``routed_grouped_gemm_topk_amd``) never imports it,
and this package imports nothing from the product path: the two share no code.

Every function here is a plain, slow, obviously correct restatement of what the
layer computes, in float64 (integer work in Python ints / int64).  Pins that
tie it to something other than itself live in ``tests/test_oracle_*.py``.
Parity pins: alignment (brute-force sort + worked example), layer (dense
SwiGLU MLP reduction, mean-of-experts, permutation equivariance, linearity,
closed-form worked example), e4m3 codec (all 256 codes, ties, saturation,
torch's float8_e4m3fn), group quantisation (error bound, amax code), bf16
rounding (torch's bfloat16 cast), combine order (crafted cancellation), routing
(worked examples with ties, brute force over expert subsets, the closed form of a
renormalised pair), MXFP4 up projection (e2m1 value list, torch's e8m0 decode, a
hand-worked packed row, brute-force nearest values of an independent quantiser,
SwiGLU closed forms and torch's SiLU, a dense torch top-1 computation).  No
function here is "parity unpinned".
"""
from .moe_oracle import (  # noqa: F401
    Alignment,
    align,
    bf16_round,
    combine,
    dequantize_blocks,
    dequantize_groups,
    e4m3_decode,
    e4m3_encode,
    expert_down,
    expert_histogram,
    expert_up,
    max_padded_slots,
    max_tiles,
    moe_layer,
    quantize_groups_e4m3,
    route,
    silu,
)
from .mx_oracle import (  # noqa: F401
    e2m1_value,
    e8m0_value,
    expert_up_mxfp4,
    gptoss_swiglu,
    moe_up_mxfp4,
    mx_decode,
    quantize_out_e4m3,
    unpack_e2m1,
)
