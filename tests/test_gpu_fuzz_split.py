"""Seeded random bf16 problems large enough in K for the GEMMs' K-split of the last round (K of
at least 1024, so a split part spans at least 8 slices), through moe_forward against the
oracle: 128- and 256-row blocks, H and I odd multiples of 64 or 128 (ragged n-blocks), excluded
ids and skew. Whether a case splits depends on its device-side tile count; the cases are fixed
by the seed and the last test checks that enough of them split both GEMMs."""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case

pytestmark = pytest.mark.gpu

N_CASES = 16


def draw(i):
    rng = np.random.default_rng([4049, i])
    H = 64 * int(rng.choice([16, 18, 24, 30, 32]))
    I = 64 * int(rng.choice([16, 18, 20, 28, 32]))
    E = int(rng.choice([2, 4, 8, 16]))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(64, 700))
    bm = int(rng.choice([128, 256]))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if rng.random() < 0.3:                                # some excluded ids
        ids = np.where(rng.random((T, k)) < 0.1, E + rng.integers(0, 3, (T, k)), ids)
    if rng.random() < 0.3:                                # skew onto one expert
        ids[:, 0] = 0
    return dict(T=T, H=H, I=I, E=E, top_k=k), bm, ids.astype(np.int32)


def splits(num_tiles, kw, bm, slots):
    """Parts (S) of the K-split of the up and the down GEMM for this tile count."""
    def one(n_out, bna, K):
        total = num_tiles * -(-n_out // bna)
        r = total % slots
        if r == 0:
            return 1
        S = min(slots // r, (K // 64) // 8, 16)
        return S if S >= 2 else 1
    bna_up = 128 if bm == 256 or kw["I"] % 256 else 256
    bna_dn = 256 if kw["H"] % 256 == 0 else 128
    return one(kw["I"], bna_up, kw["H"]), one(kw["H"], bna_dn, kw["I"])


_split_cases = []


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_split_problem(device, i):
    kw, bm, ids = draw(i)
    cfg = get_config("mixtral_prefill_bf16", **kw)
    slots = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    o = oracle.align(ids, cfg.E, bm)
    s_up, s_dn = splits(o.num_tiles, kw, bm, slots)
    print(f"fuzz-split {i}: {kw} block_m={bm}: {o.num_tiles} m-blocks, up in {s_up} parts, "
          f"down in {s_dn} parts", flush=True)
    sys.stdout.flush()
    case = make_case(cfg, device, seed=300 + i)
    case.ids_host = ids
    case.topk_ids = torch.from_numpy(ids).to(device)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, "bf16", "bf16", bm)
    assert moe.moe_validate(p) == moe.MOE_OK
    out = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(case.x_host(), ids, case.w_host, case.expert_host, cfg.E)
    got = out.to(torch.float32).cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= 2e-2
    _split_cases.append((s_up > 1, s_dn > 1))


def test_enough_cases_split(device):
    """At least four of the cases above split the up GEMM and four the down GEMM (the draw is
    seeded, so this holds for a given device unless its compute-unit count differs)."""
    if len(_split_cases) < N_CASES:
        pytest.skip("run together with test_random_split_problem")
    assert sum(u for u, _ in _split_cases) >= 4
    assert sum(d for _, d in _split_cases) >= 4
