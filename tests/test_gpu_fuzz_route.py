"""Seeded random router-producer problems through moe_route_align against the oracle: token
counts from 1 to 12000, 1 to 1024 experts, top-k up to min(E, 64), with and without
renormalisation, logits with ties (integer-valued) or spread over several orders of magnitude.
Sizes up to 8192 slots take the one-launch path (routing spread over the GPU, the last
workgroup to finish aligns), larger ones the routing launch then the alignment launches; the
cases below straddle that boundary.  Ids, the whole alignment and n_invalid must match the
oracle exactly; weights to fp32 rounding of the softmax."""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe

pytestmark = pytest.mark.gpu

N_CASES = 40
W_RTOL = 1e-5


def draw(i):
    rng = np.random.default_rng([4242, i])
    E = int(rng.choice([1, 2, 7, 8, 16, 63, 64, 65, 128, 256, 512, 1024]))
    k = int(rng.integers(1, min(E, 64) + 1)) if rng.random() < 0.3 else int(rng.integers(1, min(E, 8) + 1))
    n_max = 12000 if rng.random() < 0.7 else 40
    T = int(rng.integers(1, max(2, min(n_max, 16384 // k) + 1)))
    if rng.random() < 0.3:                   # near the one-launch limit of 8192 slots
        T = max(1, 8192 // k + int(rng.integers(-2, 3)))
    kind = int(rng.integers(0, 3))
    if kind == 0:
        lg = rng.standard_normal((T, E))
    elif kind == 1:
        lg = rng.integers(-3, 4, (T, E)).astype(np.float64)          # many ties
    else:
        lg = rng.standard_normal((T, E)) * 10.0 ** rng.uniform(-3, 1.5, (T, 1))
    return T, E, k, bool(rng.random() < 0.5), lg.astype(np.float32)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_route_align(device, i):
    T, E, k, renorm, lg = draw(i)
    print(f"route fuzz {i}: T={T} E={E} k={k} slots={T * k} renorm={renorm}", flush=True)
    sys.stdout.flush()
    p = moe.make_problem(T, 128, 128, E, k, "bf16")
    a = moe.route_align(p, torch.from_numpy(lg).to(device), renorm)
    torch.cuda.synchronize()
    o_ids, o_w = oracle.route(lg.astype(np.float64), k, renorm)
    assert np.array_equal(a["topk_ids"].cpu().numpy(), o_ids)
    assert np.allclose(a["topk_weights"].cpu().numpy(), o_w, rtol=W_RTOL, atol=1e-30)
    o = oracle.align(o_ids, E, moe.moe_pick_block_m(p))
    assert a["counts"].cpu().numpy().tolist() == o.counts.tolist()
    assert a["offsets"].cpu().numpy().tolist() == o.offsets.tolist()
    assert np.array_equal(a["sorted_slots"].cpu().numpy(), o.sorted_slots)
    assert np.array_equal(a["slot_row"].cpu().numpy(), o.slot_row)
    assert np.array_equal(a["tiles"].cpu().numpy().reshape(-1, 2), o.tiles)
    assert int(a["num_tiles"].item()) == o.num_tiles and int(a["n_invalid"].item()) == 0
