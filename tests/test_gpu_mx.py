"""GPU parity of moe_grouped_gemm_up_mxfp4 (MXFP4 weights x e4m3 rows, bias, GPT-OSS SwiGLU,
e4m3 output) against the float64 oracle, through the C ABI.

The output is an e4m3 code of act / out_scale.  The oracle's value v is exact (float64); the
GPU accumulates in fp32, so near a rounding midpoint the two may round differently.  The bar:
every GPU code is as close to v as the correctly rounded code up to 2e-3 |v| + 1e-6 (so only
near-ties may differ), and at most 1% of the codes differ from the oracle's.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_mx_case, make_routing

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_mx(case, bm=0):
    cfg = case.cfg
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, "e4m3", "mxfp4", bm)
    a = moe.align(p, case.topk_ids)
    rows = moe.moe_max_padded_slots(p)
    act = torch.full((rows, cfg.I), 0x7F, dtype=torch.uint8, device=case.x_codes.device)  # NaN fill
    moe.moe_grouped_gemm_up_mxfp4(p, case.x_codes, case.x_scale, case.w13, case.w13_scales,
                                  case.bias, case.alpha, case.limit, case.out_scale,
                                  a["sorted_slots"], a["offsets"], a["tiles"], a["num_tiles"], act)
    torch.cuda.synchronize()
    return p, a, act


def check_codes(case, a, act, slots=None):
    """Compare the GPU codes of the valid sorted rows (or of `slots`) with the oracle."""
    cfg = case.cfg
    ss = a["sorted_slots"].cpu().numpy()
    N = cfg.T * cfg.top_k
    rows = np.nonzero(ss < N)[0]
    if slots is not None:
        keep = np.isin(ss[rows], np.asarray(slots))
        rows = rows[keep]
    sl = ss[rows]
    ref = oracle.moe_up_mxfp4(case.x_codes_host(), float(case.x_scale.item()), case.ids_host,
                              case.expert_host, None, case.bias_host(), case.alpha, case.limit,
                              num_experts=cfg.E, slots=sl)
    v = ref[sl] / float(case.out_scale.item())
    assert np.isfinite(v).all()
    got = act.cpu().numpy()[rows]
    want = oracle.e4m3_encode(v)
    dg = oracle.e4m3_decode(got)
    dw = oracle.e4m3_decode(want)
    assert np.isfinite(dg).all(), "a NaN code (unwritten row?)"
    slack = 2e-3 * np.abs(v) + 1e-6
    far = np.abs(dg - v) > np.abs(dw - v) + slack
    frac = float((got != want).mean())
    say(f"  {got.size} codes, {int((got != want).sum())} differ ({100 * frac:.3f}%), "
        f"{int(far.sum())} beyond the near-tie slack")
    assert not far.any()
    assert frac <= 0.01
    return rows


def small_case(device, T=40, H=192, I=128, E=4, k=2, seed=0, **kw):
    cfg = get_config("gptoss_shard_mxfp4", T=T, H=H, I=I, E=E, top_k=k, route_experts=0,
                     prod_like=False)
    return make_mx_case(cfg, device, seed=seed, **kw)


@pytest.mark.parametrize("shape", [dict(T=40, H=192, I=128), dict(T=300, H=256, I=192),
                                   dict(T=1, H=64, I=64, E=2, k=1), dict(T=130, H=320, I=64)])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_mx_small(device, shape, bm):
    case = small_case(device, **shape)
    say(f"mx {shape} bm {bm} alpha {case.alpha:.4f} limit {case.limit:.4f}")
    p, a, act = run_mx(case, bm)
    rows = check_codes(case, a, act)
    # padding rows are not written
    ss = a["sorted_slots"].cpu().numpy()
    nt = int(a["num_tiles"].item())
    pad = np.nonzero(ss[: nt * bm] >= case.cfg.T * case.cfg.top_k)[0]
    assert (act.cpu().numpy()[pad] == 0x7F).all()
    assert rows.size == int((case.ids_host < case.cfg.E).sum())


def test_mx_page_weight_scale(device):
    """Weights ~ N(0, 1) as the page draws them: most gate and linear values saturate at the
    limit; the codes must still match."""
    case = small_case(device, T=64, H=256, I=128, weight_std=1.0)
    _, a, act = run_mx(case, 32)
    check_codes(case, a, act)


def test_mx_excluded_ids(device):
    cfg = get_config("gptoss_shard_mxfp4", T=50, H=128, I=128, E=4, top_k=2, route_experts=0,
                     prod_like=False)
    rng = np.random.default_rng(5)
    ids = np.where(rng.random((50, 2)) < 0.3, 4 + rng.integers(0, 4, (50, 2)), rng.integers(0, 4, (50, 2)))
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 8, ids[:, 1])
    case = make_mx_case(cfg, device, seed=2, ids=ids)
    _, a, act = run_mx(case, 16)
    assert int(a["n_invalid"].item()) == int((ids >= 4).sum())
    check_codes(case, a, act)


SHARD_POINTS = {0: None, 20: 400, 47: 300}     # sweep index -> sampled slots (None: all)


@pytest.mark.parametrize("idx", list(SHARD_POINTS))
def test_mx_shard_sweep_points(device, idx):
    from moe_inputs import SWEEP_CONFIGS, sweep_batch_sizes
    base = SWEEP_CONFIGS["gptoss_shard_mxfp4"]
    T = sweep_batch_sizes(base.route_experts, base.top_k)[idx]
    cfg = get_config("gptoss_shard_mxfp4", T=T)
    say(f"mx shard T={T}: generating")
    case = make_mx_case(cfg, device, seed=0)
    bm = moe.moe_block_m_for(T * cfg.top_k / base.route_experts, "e4m3", "mxfp4")
    _, a, act = run_mx(case, bm)
    n = SHARD_POINTS[idx]
    slots = None
    if n is not None:
        flat = case.ids_host.reshape(-1)
        local = np.nonzero(flat < cfg.E)[0]
        slots = np.random.default_rng(3).choice(local, n, replace=False)
    say(f"mx shard T={T} block_m {bm}: oracle")
    check_codes(case, a, act, slots)
