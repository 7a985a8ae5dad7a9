"""moe_forward captured in a HIP graph: every replay equals the eager result bit for bit, with
eager work and synchronisations between the replays (the library records no memset, no
allocation and no host synchronisation, so the whole layer is capturable; the workspace is
cleared before each replay, so the K-split partial tiles must be rewritten by every replay)."""
import pytest
import torch

import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [("mixtral_prefill_bf16", dict(T=300, H=256, I=384)),
                                     # 256-row m-blocks whose GEMMs split their last round
                                     # along K (partials in the workspace, a second launch)
                                     ("mixtral_prefill_bf16", dict(T=512, H=1024, I=2048, E=4)),
                                     ("dsv3_fp8_e4m3", dict(T=200, H=512, I=256, E=16)),
                                     ("tiny_fp32", dict())])
def test_forward_graph_replays_match_eager(device, name, kw):
    cfg = get_config(name, **kw)
    case = make_case(cfg, device, seed=4)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, cfg.x_dtype, cfg.w_dtype)
    args = (case.x, case.topk_ids, case.topk_weights, case.w13, case.w2, case.w13_scales,
            case.w2_scales)
    ws_e = moe.alloc_workspace(p, case.x.device)
    eager = moe.forward(p, *args, workspace=ws_e)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    ws = moe.alloc_workspace(p, case.x.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.forward(p, *args, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(p, *args, out=out, workspace=ws)
    for rep in range(4):
        out.zero_()
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        # eager work on the same buffers between replays
        moe.forward(p, *args, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("T,E,k", [(64, 256, 8), (4096, 8, 2)])
def test_route_align_graph_replays_match_eager(device, T, E, k):
    """moe_route_align in one launch, captured: each replay reuses the completion counter taken
    at capture (set back to zero by the launch's last workgroup), with eager calls, which take
    other counters, between the replays."""
    import numpy as np
    rng = np.random.default_rng(8)
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(device)
    p = moe.make_problem(T, 128, 128, E, k, "bf16")
    eager = moe.route_align(p, lg, True)
    torch.cuda.synchronize()
    b = {n: torch.empty_like(v) for n, v in eager.items()}

    def call():
        moe.moe_route_align(p, lg, True, b["topk_ids"], b["topk_weights"], b["counts"],
                            b["offsets"], b["sorted_slots"], b["slot_row"], b["tiles"],
                            b["num_tiles"], b["n_invalid"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for v in b.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for n, v in eager.items():
            assert torch.equal(b[n], v), f"replay {rep}: {n}"
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        for n, v in eager.items():
            assert torch.equal(b[n], v), f"eager after replay {rep}: {n}"
