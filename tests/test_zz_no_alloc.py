"""moe_forward_scratch -- the entry point that allocates nothing -- against moe_forward.

moe_forward_scratch runs moe_forward's kernels with its intermediates in a library-owned
device array instead of a caller workspace.  Same launch sequence and workspace layout, so
the output must equal moe_forward's bit for bit (and the excluded-slot count must agree).
Calls run back to back, the second smaller than the first (the array keeps the previous
call's contents), on bf16 prefill with the GEMMs' K-split, bf16 decode-size blocks, fp8 and
fp32 problems; a problem whose workspace exceeds the array is refused on the host.
"""
import ctypes
import sys

import pytest
import torch

import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def case_of(device, base, seed, **kw):
    cfg = get_config(base, **kw)
    case = make_case(cfg, device, seed=seed)
    ids = case.ids_host.copy()
    ids[0, -1] = cfg.E                       # one excluded slot
    case.ids_host = ids
    case.topk_ids = torch.from_numpy(ids).to(device)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, cfg.x_dtype, cfg.w_dtype)
    return cfg, case, p


def run_both(device, cfg, case, p):
    assert moe.moe_workspace_bytes(p) <= moe.moe_scratch_max_bytes()
    ref = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2,
                      case.w13_scales, case.w2_scales)
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=case.x.dtype, device=device)
    n_inv = torch.full((1,), -1, dtype=torch.int32, device=device)
    moe.moe_forward_scratch(p, case.x, case.topk_ids, case.topk_weights, case.w13,
                            case.w13_scales, case.w2, case.w2_scales, out, n_inv)
    torch.cuda.synchronize()
    return ref, out, int(n_inv.item())


# (base workload, sizes): each pair runs larger first, then smaller
PAIRS = {
    "bf16_split_then_decode": [("mixtral_prefill_bf16", dict(T=512, H=1024, I=2048, E=4, top_k=2)),
                               ("dsv3_decode_bf16", dict(T=40, H=512, I=256, E=16, top_k=4))],
    "fp8_then_fp8": [("dsv3_fp8_e4m3", dict(T=300, H=1024, I=512, E=16, top_k=4)),
                     ("dsv3_fp8_e4m3", dict(T=24, H=256, I=256, E=8, top_k=2))],
    "bf16_256_then_f32": [("skewed_prefill_bf16", dict(T=2000, H=512, I=384, E=16, top_k=6)),
                          ("tiny_fp32", dict())],
}


@pytest.mark.parametrize("label", list(PAIRS))
def test_scratch_forward_matches_forward(device, label):
    for i, (base, kw) in enumerate(PAIRS[label]):
        cfg, case, p = case_of(device, base, seed=10 + i, **kw)
        say(f"no-alloc {label} call {i}: {p}, workspace {moe.moe_workspace_bytes(p)} bytes")
        ref, out, n_inv = run_both(device, cfg, case, p)
        assert n_inv == int((case.ids_host >= cfg.E).sum())
        assert torch.equal(out, ref), f"call {i}: moe_forward_scratch differs from moe_forward"
        assert not torch.isnan(out.float()).any()


def test_scratch_forward_repeat_and_shrink(device):
    """The same problem twice, then a smaller one: the array's old contents do not leak in."""
    cfg, case, p = case_of(device, "mixtral_prefill_bf16", seed=3, T=700, H=768, I=1024, E=8, top_k=2)
    ref, out1, _ = run_both(device, cfg, case, p)
    _, out2, _ = run_both(device, cfg, case, p)
    assert torch.equal(out1, ref) and torch.equal(out2, ref)
    cfg, case, p = case_of(device, "mixtral_prefill_bf16", seed=4, T=33, H=768, I=1024, E=8, top_k=2)
    ref, out3, _ = run_both(device, cfg, case, p)
    assert torch.equal(out3, ref)


def test_scratch_forward_refuses_too_large(device):
    """A problem whose intermediates exceed the array is refused on the host (nothing runs)."""
    cfg = get_config("mixtral_prefill_bf16")          # ~331 MB of intermediates
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, "bf16")
    assert moe.moe_workspace_bytes(p) > moe.moe_scratch_max_bytes() == 128 << 20
    ptr = torch.empty(256, dtype=torch.uint8, device=device).data_ptr()
    rc = moe.load().moe_forward_scratch(ctypes.byref(p), ptr, ptr, ptr, ptr, None, ptr, None, ptr,
                                        None, None)
    assert rc == moe.MOE_ERR_WORKSPACE
