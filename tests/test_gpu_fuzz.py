"""Seeded random problems through moe_forward against the oracle: shapes, expert counts, top-k,
block sizes and dtypes drawn at random within the documented limits (sizes the oracle finishes
quickly), routing with duplicates and excluded ids.  The cases are fixed by the seed, so a
failure names a reproducible case; they cross dispatch paths the workload tests do not (odd
multiples of 64, 128-wide ragged n-blocks at every block size, many experts with few slots)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}
N_CASES = 64


def draw(i):
    rng = np.random.default_rng([2024, i])
    w_dtype = ["f32", "bf16", "bf16", "e4m3"][int(rng.integers(0, 4))]
    mult = 128 if w_dtype == "e4m3" else 64
    H = mult * int(rng.integers(1, 6))
    I = mult * int(rng.integers(1, 6))
    E = int(rng.choice([1, 2, 3, 8, 17, 64]))
    k = int(rng.integers(1, min(E, 6) + 1))
    T = int(rng.integers(1, 300))
    bms = [0, 16, 32, 64, 128] + ([256] if w_dtype == "bf16" else [])
    bm = int(rng.choice(bms))
    ids = rng.integers(0, E, (T, k))
    if rng.random() < 0.5:                                # some excluded ids
        ids = np.where(rng.random((T, k)) < 0.1, E + rng.integers(0, 3, (T, k)), ids)
    if rng.random() < 0.3:                                # skew onto one expert
        ids[:, 0] = 0
    base = {"f32": "tiny_fp32", "bf16": "mixtral_prefill_bf16", "e4m3": "dsv3_fp8_e4m3"}[w_dtype]
    return base, dict(T=T, H=H, I=I, E=E, top_k=k), bm, ids.astype(np.int32)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(device, i):
    base, kw, bm, ids = draw(i)
    cfg = get_config(base, **kw)
    print(f"fuzz {i}: {base} {kw} block_m={bm}", flush=True)
    sys.stdout.flush()
    case = make_case(cfg, device, seed=100 + i)
    case.ids_host = ids
    case.topk_ids = torch.from_numpy(ids).to(device)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, cfg.x_dtype, cfg.w_dtype, bm)
    assert moe.moe_validate(p) == moe.MOE_OK
    ws = moe.alloc_workspace(p, case.x.device)
    out = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2,
                      case.w13_scales, case.w2_scales, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == int(((ids < 0) | (ids >= cfg.E)).sum())
    ref = oracle.moe_layer(case.x_host(), ids, case.w_host, case.expert_host, cfg.E,
                           fp8=cfg.w_dtype == "e4m3")
    got = out.to(torch.float32).cpu().numpy()
    assert np.isfinite(got).all()
    denom = np.abs(ref).max()
    err = float(np.abs(got - ref).max() / (denom if denom > 0 else 1.0))
    tol = TOL[cfg.w_dtype]
    print(f"  block_m {moe.moe_pick_block_m(p)}: rel err {err:.3e} (tol {tol})", flush=True)
    assert err <= tol


N_MX = 16


@pytest.mark.parametrize("i", range(N_MX))
def test_random_mxfp4_problem(device, i):
    """The MXFP4 first expert GEMM on random shapes (H and I multiples of 64, K tails),
    expert counts, block sizes and routings with excluded ids; the code-level bar of
    test_gpu_mx."""
    from moe_inputs import make_mx_case
    from test_gpu_mx import check_codes, run_mx
    rng = np.random.default_rng([4048, i])
    H, I = 64 * int(rng.integers(1, 8)), 64 * int(rng.integers(1, 6))
    E = int(rng.choice([1, 2, 5, 16, 40]))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(1, 260))
    bm = int(rng.choice([0, 16, 32, 64, 128]))
    ids = rng.integers(0, E, (T, k))
    if rng.random() < 0.5:
        ids = np.where(rng.random((T, k)) < 0.15, E + rng.integers(0, 2, (T, k)), ids)
    cfg = get_config("gptoss_shard_mxfp4", T=T, H=H, I=I, E=E, top_k=k, route_experts=0,
                     prod_like=False)
    print(f"mx fuzz {i}: T={T} H={H} I={I} E={E} k={k} block_m={bm}", flush=True)
    case = make_mx_case(cfg, device, seed=200 + i, ids=ids.astype(np.int32))
    _, a, act = run_mx(case, bm)
    assert int(a["n_invalid"].item()) == int((ids >= E).sum())
    if (ids < E).any():
        check_codes(case, a, act)
