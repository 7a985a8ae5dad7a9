"""GPU parity of the GEMMs' K-split tail (bf16, 128- and 256-row m-blocks).

With a workspace, moe_grouped_gemm_up and moe_grouped_gemm_down cut the tiles of their last,
partly filled round of workgroups along K; the parts' fp32 partial tiles are added in
ascending part order before the epilogue. Each case below is sized so that both GEMMs really
split (checked from the oracle's tile count), and the outputs are compared with the oracle
(layer tolerance 2e-2), with the same calls made without workspace (no split: they differ only
by the fp32 summation order, then one bf16 rounding), with a second run (bit-identical) and
with moe_forward (bit-identical).  Which tiles split, and into how many parts, depends on the
device's compute-unit count; the workspace shows the units the kernels wrote, which must be the
ones predicted from that count.
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
    # whole tiles first, then a short last round split
    "tail_bm256": (dict(T=4096, H=2048, I=1024, E=8, top_k=2), 256),
    # 128-wide ragged n-blocks (H = 2880) at 128-row m-blocks
    "ragged_bm128": (dict(T=640, H=2880, I=1024, E=4, top_k=2), 128),
    # and at 256-row m-blocks (down n-block 128, up 2 x 128)
    "ragged_bm256": (dict(T=384, H=2880, I=1024, E=4, top_k=2), 256),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(gpu - ref).max() / np.abs(ref).max())


def predicted_split(num_tiles, n_out, bna, K, slots):
    """The split the kernels choose: r tiles of the last round cut into S parts."""
    total = num_tiles * -(-n_out // bna)
    r = total % slots
    if r == 0:
        return 0, 1
    S = min(slots // r, (K // 64) // 8, 16)
    return (r, S) if S >= 2 else (0, 1)


@pytest.mark.parametrize("label", list(CASES))
def test_gemm_split_parity(device, label):
    kw, bm = CASES[label]
    cfg = get_config("mixtral_prefill_bf16", **kw)
    case = make_case(cfg, device, seed=5)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, "bf16", "bf16", bm)
    assert moe.moe_pick_block_m(p) == bm
    o = oracle.align(case.ids_host, cfg.E, bm)
    slots = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    bna_up = 128 if bm == 256 or cfg.I % 256 else 256
    bna_down = 256 if cfg.H % 256 == 0 else 128
    up = predicted_split(o.num_tiles, cfg.I, bna_up, cfg.H, slots)
    down = predicted_split(o.num_tiles, cfg.H, bna_down, cfg.I, slots)
    say(f"split {label} {p}: {o.num_tiles} m-blocks; up {up[0]} tiles in {up[1]} parts, "
        f"down {down[0]} tiles in {down[1]} parts")
    assert up[1] >= 2 and down[1] >= 2, "the case must exercise both splits"

    a = moe.align(p, case.topk_ids)
    rows = moe.moe_max_padded_slots(p)
    ws = moe.alloc_gemm_workspace(p, device)
    assert ws is not None
    ws.fill_(0xFF)                      # NaN partials if a reduce read an unwritten one

    def up_gemm(workspace):
        act = torch.full((rows, cfg.I), float("nan"), dtype=torch.bfloat16, device=device)
        moe.moe_grouped_gemm_up(p, case.x, None, case.w13, None, a["sorted_slots"], a["offsets"],
                                a["tiles"], a["num_tiles"], act, None, workspace)
        return act

    def down_gemm(act, workspace):
        so = torch.full((cfg.T * cfg.top_k, cfg.H), float("nan"), dtype=torch.bfloat16, device=device)
        moe.moe_grouped_gemm_down(p, act, None, case.w2, None, case.topk_weights, a["sorted_slots"],
                                  a["offsets"], a["tiles"], a["num_tiles"], so, workspace)
        return so

    def units_written(n_units, pw):
        # K-split unit u writes its fp32 partial tile at u * (block_m x pw) floats of the
        # workspace; its first row always holds a slot.  The workspace was filled with 0xFF
        # (NaN), so written units start with a finite value and the next one with NaN.
        f = ws.view(torch.float32)
        stride = bm * pw
        first = [float(f[u * stride].item()) for u in range(min(n_units + 1, f.numel() // stride))]
        return first

    act1 = up_gemm(ws)
    torch.cuda.synchronize()
    # the split the kernels chose follows the device's compute-unit count (predicted above)
    first = units_written(up[0] * up[1], 2 * bna_up)
    assert all(np.isfinite(first[: up[0] * up[1]])), "a predicted up K-split unit was not written"
    if len(first) > up[0] * up[1]:
        assert np.isnan(first[up[0] * up[1]]), "more up K-split units than predicted"
    act2 = up_gemm(ws)
    act_plain = up_gemm(None)
    ws.fill_(0xFF)
    so1 = down_gemm(act1, ws)
    torch.cuda.synchronize()
    first = units_written(down[0] * down[1], bna_down)
    assert all(np.isfinite(first[: down[0] * down[1]])), "a predicted down K-split unit was not written"
    if len(first) > down[0] * down[1]:
        assert np.isnan(first[down[0] * down[1]]), "more down K-split units than predicted"
    so2 = down_gemm(act1, ws)
    so_plain = down_gemm(act1, None)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=device)
    moe.moe_combine(p, so1, a["slot_row"], out)
    fwd = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2)
    torch.cuda.synchronize()

    used = int(o.offsets[-1])
    a1 = act1.float().cpu().numpy()[:used]
    assert np.isfinite(a1).all(), "an act row was not written"
    pad = o.sorted_slots[:used] >= cfg.T * cfg.top_k
    assert np.all(a1[pad] == 0), "padding rows of act not zero"
    s1 = so1.float().cpu().numpy()
    assert np.isfinite(s1).all(), "a slot row was not written"
    # rows past the last valid tile are never written (NaN here): compare the used rows
    assert torch.equal(act1[:used], act2[:used]) and torch.equal(so1, so2), \
        "split result not deterministic"
    assert torch.equal(out, fwd), "moe_forward differs from the entry points"
    d_up = rel_err(a1, act_plain.float().cpu().numpy()[:used])
    d_down = rel_err(s1, so_plain.float().cpu().numpy())
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, case.expert_host, cfg.E)
    err = rel_err(out.float().cpu().numpy(), ref)
    say(f"  split vs unsplit: up {d_up:.3e}, down {d_down:.3e}; layer vs oracle {err:.3e}")
    assert d_up <= 1e-2 and d_down <= 1e-2
    assert err <= 2e-2
