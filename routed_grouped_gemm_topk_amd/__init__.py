"""MI355X (gfx950) routed grouped-GEMM top-k MoE expert layer.

The computation lives in libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h).  This package is its Python binding: ``_lib`` mirrors the C
entry points one to one; the helpers below only allocate buffers with torch
and call them.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MOE_BF16,
    MOE_E4M3,
    MOE_ERR_ALIGN,
    MOE_ERR_DEVICE,
    MOE_ERR_DTYPE,
    MOE_ERR_LAUNCH,
    MOE_ERR_NULL,
    MOE_ERR_SHAPE,
    MOE_ERR_WORKSPACE,
    MOE_F32,
    MOE_MXFP4,
    MOE_OK,
    MoeError,
    Problem,
    load,
    make_problem,
    moe_align,
    moe_block_m_for,
    moe_combine,
    moe_gemm_workspace_bytes,
    moe_forward,
    moe_forward_scratch,
    moe_grouped_gemm_down,
    moe_grouped_gemm_up,
    moe_grouped_gemm_up_mxfp4,
    moe_max_padded_slots,
    moe_max_tiles,
    moe_pick_block_m,
    moe_quantize_rows_e4m3,
    moe_route,
    moe_route_align,
    moe_scratch_max_bytes,
    moe_validate,
    moe_workspace_bytes,
    status_str,
)


def alloc_align(p: Problem, device) -> dict:
    rows, mt = moe_max_padded_slots(p), moe_max_tiles(p)
    z = lambda n: torch.empty(n, dtype=torch.int32, device=device)  # noqa: E731
    return {"counts": z(p.E), "offsets": z(p.E + 1), "sorted_slots": z(rows),
            "slot_row": z(p.T * p.top_k), "tiles": z(2 * mt), "num_tiles": z(1),
            "n_invalid": z(1)}


def align(p: Problem, topk_ids: torch.Tensor, stream=None) -> dict:
    """Run moe_align into freshly allocated buffers; returns them by name."""
    a = alloc_align(p, topk_ids.device)
    moe_align(p, topk_ids, a["counts"], a["offsets"], a["sorted_slots"], a["slot_row"],
              a["tiles"], a["num_tiles"], a["n_invalid"], stream)
    return a


def route(p: Problem, logits: torch.Tensor, renormalize: bool, stream=None):
    """Run moe_route into fresh buffers; returns (topk_ids int32 [T,k], topk_weights fp32 [T,k])."""
    ids = torch.empty((p.T, p.top_k), dtype=torch.int32, device=logits.device)
    w = torch.empty((p.T, p.top_k), dtype=torch.float32, device=logits.device)
    moe_route(p, logits, renormalize, ids, w, stream)
    return ids, w


def route_align(p: Problem, logits: torch.Tensor, renormalize: bool, stream=None) -> dict:
    """Run moe_route_align into fresh buffers; returns align()'s buffers plus topk_ids and
    topk_weights."""
    a = alloc_align(p, logits.device)
    a["topk_ids"] = torch.empty((p.T, p.top_k), dtype=torch.int32, device=logits.device)
    a["topk_weights"] = torch.empty((p.T, p.top_k), dtype=torch.float32, device=logits.device)
    moe_route_align(p, logits, renormalize, a["topk_ids"], a["topk_weights"], a["counts"],
                    a["offsets"], a["sorted_slots"], a["slot_row"], a["tiles"], a["num_tiles"],
                    a["n_invalid"], stream)
    return a


def alloc_workspace(p: Problem, device) -> torch.Tensor:
    return torch.empty(moe_workspace_bytes(p), dtype=torch.uint8, device=device)


def alloc_gemm_workspace(p: Problem, device) -> Optional[torch.Tensor]:
    """The optional workspace of moe_grouped_gemm_up / _down (None when the problem's GEMMs
    use none)."""
    n = moe_gemm_workspace_bytes(p)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def forward(p: Problem, x, topk_ids, topk_weights, w13, w2, w13_scales=None, w2_scales=None,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """The whole layer through moe_forward.  Allocates `out` / `workspace` if not given."""
    if out is None:
        out = torch.empty((p.T, p.H), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(p, x.device)
    moe_forward(p, x, topk_ids, topk_weights, w13, w13_scales, w2, w2_scales, out, workspace,
                stream)
    return out
