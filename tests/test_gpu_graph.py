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
