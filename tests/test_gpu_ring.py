"""Short K at 256-row m-blocks through moe_forward against the oracle.

The 256-row bf16 GEMMs give the m-block rows a ring of two stages and the weight rows one of
three, filled ahead of the k-loop and refilled in parts; with fewer k-slices than stages the
copies past the last slice repeat it.  These cases run 1 to 5 k-slices of 64 in the up GEMM
(K = H) and in the down GEMM (K = I; the separate rings need H a multiple of 256), with
experts whose rows end in partly filled m-blocks."""
import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case

pytestmark = pytest.mark.gpu

# (H, I): up k-slices = H / 64, down k-slices = I / 64
SHAPES = [(64, 256), (128, 512), (192, 256), (256, 64), (256, 128), (256, 192), (512, 320)]


@pytest.mark.parametrize("H,I", SHAPES)
def test_short_k_256_row_blocks(device, H, I):
    T, E, k = 700, 4, 2
    rng = np.random.default_rng([7, H, I])
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[: T // 2, 0] = 1                                  # one expert with three m-blocks
    cfg = get_config("mixtral_prefill_bf16", T=T, H=H, I=I, E=E, top_k=k)
    print(f"short-K ring: T={T} H={H} I={I} E={E} k={k} block_m=256", flush=True)
    case = make_case(cfg, device, seed=H * 1000 + I)
    case.ids_host = ids
    case.topk_ids = torch.from_numpy(ids).to(device)
    p = moe.make_problem(T, H, I, E, k, "bf16", "bf16", 256)
    assert moe.moe_pick_block_m(p) == 256
    out = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(case.x_host(), ids, case.w_host, case.expert_host, E)
    got = out.to(torch.float32).cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    print(f"  rel err {err:.3e} (tol 2e-2)", flush=True)
    assert err <= 2e-2
