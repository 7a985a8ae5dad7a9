"""GPU parity of the down GEMM's K-split tail (bf16, 128- and 256-row m-blocks).

With a workspace, moe_grouped_gemm_down cuts the tiles of its last, partly filled round of
workgroups along K; the parts' fp32 partial tiles are added in ascending part order. Each
case below is sized so that the split really happens (checked from the oracle's tile count),
and its output is compared with the oracle (layer tolerance 2e-2), with the same call made
without workspace (no split: the two differ only by the fp32 summation order, then one bf16
rounding) and with a second run (bit-identical).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case

pytestmark = pytest.mark.gpu

CASES = {
    # every tile split (fewer tiles than compute units)
    "all_tiles_bm256": (dict(T=512, H=1024, I=2048, E=4, top_k=2), 256),
    # whole tiles first, then a short last round split in two
    "tail_bm256": (dict(T=4096, H=2048, I=1024, E=8, top_k=2), 256),
    # 128-wide ragged n-blocks (H = 2880) at 128-row m-blocks
    "ragged_bm128": (dict(T=640, H=2880, I=1024, E=4, top_k=2), 128),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(gpu - ref).max() / np.abs(ref).max())


def predicted_split(num_tiles, H, I, slots):
    """The split the kernels choose: r tiles of the last round cut into S parts."""
    nblk = -(-H // (256 if H % 256 == 0 else 128))
    total = num_tiles * nblk
    r = total % slots
    if r == 0:
        return 0, 1
    S = min(slots // r, (I // 64) // 8, 16)
    return (r, S) if S >= 2 else (0, 1)


@pytest.mark.parametrize("label", list(CASES))
def test_down_split_parity(device, label):
    kw, bm = CASES[label]
    cfg = get_config("mixtral_prefill_bf16", **kw)
    case = make_case(cfg, device, seed=5)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, "bf16", "bf16", bm)
    assert moe.moe_pick_block_m(p) == bm
    o = oracle.align(case.ids_host, cfg.E, bm)
    slots = torch.cuda.get_device_properties(0).multi_processor_count
    r, S = predicted_split(o.num_tiles, cfg.H, cfg.I, min(slots, 256))
    say(f"split {label} {p}: {o.num_tiles} m-blocks, {r} tiles split {S} ways")
    assert S >= 2, "the case must exercise the split"

    a = moe.align(p, case.topk_ids)
    rows = moe.moe_max_padded_slots(p)
    act = torch.full((rows, cfg.I), float("nan"), dtype=torch.bfloat16, device=device)
    moe.moe_grouped_gemm_up(p, case.x, None, case.w13, None, a["sorted_slots"], a["offsets"],
                            a["tiles"], a["num_tiles"], act, None)
    ws = moe.alloc_down_workspace(p, device)
    assert ws is not None

    def down(workspace):
        so = torch.full((cfg.T * cfg.top_k, cfg.H), float("nan"), dtype=torch.bfloat16, device=device)
        moe.moe_grouped_gemm_down(p, act, None, case.w2, None, case.topk_weights, a["sorted_slots"],
                                  a["offsets"], a["tiles"], a["num_tiles"], so, workspace)
        return so

    ws.fill_(0xFF)                      # NaN partials if the reduce read an unwritten one
    split1 = down(ws)
    split2 = down(ws)
    plain = down(None)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=device)
    moe.moe_combine(p, split1, a["slot_row"], out)
    fwd = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2)
    torch.cuda.synchronize()

    s1 = split1.float().cpu().numpy()
    assert np.isfinite(s1).all(), "a slot row was not written"
    assert torch.equal(split1, split2), "split result not deterministic"
    assert torch.equal(out, fwd), "moe_forward differs from the entry points"
    d = rel_err(s1, plain.float().cpu().numpy())
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, case.expert_host, cfg.E)
    err = rel_err(out.float().cpu().numpy(), ref)
    say(f"  split vs unsplit {d:.3e}; layer vs oracle {err:.3e}")
    assert d <= 1e-2
    assert err <= 2e-2
