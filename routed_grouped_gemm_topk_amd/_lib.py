"""ctypes binding of libmoe.so: argument marshalling only.

Every function mirrors one ``extern "C"`` entry point of include/moe.h under the
same name.  Tensors are torch tensors on the current HIP device; the binding
checks dtype, shape, device and contiguity, then passes raw pointers and the
current stream.  All arithmetic happens in the HIP kernels behind the C ABI.
If libmoe.so is missing, loading raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_DTYPE = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_LAUNCH = -5
MOE_ERR_DEVICE = -6
MOE_ERR_ALIGN = -7

MOE_F32, MOE_BF16, MOE_E4M3, MOE_MXFP4 = 0, 1, 2, 3
_DT_NAME = {"f32": MOE_F32, "bf16": MOE_BF16, "e4m3": MOE_E4M3, "mxfp4": MOE_MXFP4}
_TORCH_DT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_E4M3: torch.float8_e4m3fn}

EXPORTS = ["moe_status_str", "moe_validate", "moe_pick_block_m", "moe_block_m_for", "moe_max_padded_slots",
           "moe_max_tiles", "moe_workspace_bytes", "moe_route", "moe_route_align", "moe_align",
           "moe_quantize_rows_e4m3", "moe_grouped_gemm_up", "moe_grouped_gemm_up_mxfp4",
           "moe_grouped_gemm_down", "moe_gemm_workspace_bytes",
           "moe_combine", "moe_forward", "moe_scratch_max_bytes", "moe_forward_scratch"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class Problem(ctypes.Structure):
    """Mirror of ``moe_problem``."""
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]

    def __repr__(self):
        return ("Problem(T=%d, H=%d, I=%d, E=%d, top_k=%d, block_m=%d, dtype=%d, w_dtype=%d)"
                % (self.T, self.H, self.I, self.E, self.top_k, self.block_m, self.dtype, self.w_dtype))


def make_problem(T, H, I, E, top_k, dtype="bf16", w_dtype=None, block_m=0) -> Problem:
    dt = _DT_NAME[dtype] if isinstance(dtype, str) else int(dtype)
    wdt = dt if w_dtype is None else (_DT_NAME[w_dtype] if isinstance(w_dtype, str) else int(w_dtype))
    return Problem(int(T), int(H), int(I), int(E), int(top_k), int(block_m), dt, wdt)


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libmoe.so not found at {p}; build it with "
                          "`python -m routed_grouped_gemm_topk_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    sig = {
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_validate": (ctypes.c_int, [P]),
        "moe_pick_block_m": (i32, [P]),
        "moe_block_m_for": (i32, [ctypes.c_double, i32, i32]),
        "moe_max_padded_slots": (ctypes.c_int64, [P]),
        "moe_max_tiles": (ctypes.c_int64, [P]),
        "moe_workspace_bytes": (ctypes.c_int64, [P]),
        "moe_align": (ctypes.c_int, [P] + [vp] * 8 + [vp]),
        "moe_route": (ctypes.c_int, [P, vp, ctypes.c_int, vp, vp, vp]),
        "moe_route_align": (ctypes.c_int, [P, vp, ctypes.c_int] + [vp] * 9 + [vp]),
        "moe_quantize_rows_e4m3": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "moe_grouped_gemm_up": (ctypes.c_int, [P] + [vp] * 11 + [ctypes.c_size_t, vp]),
        "moe_grouped_gemm_up_mxfp4": (ctypes.c_int, [P] + [vp] * 5 + [ctypes.c_float] * 2
                                      + [vp] * 6 + [vp]),
        "moe_grouped_gemm_down": (ctypes.c_int, [P] + [vp] * 11 + [ctypes.c_size_t, vp]),
        "moe_gemm_workspace_bytes": (ctypes.c_int64, [P]),
        "moe_combine": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "moe_forward": (ctypes.c_int, [P] + [vp] * 9 + [ctypes.c_size_t, vp]),
        "moe_scratch_max_bytes": (ctypes.c_int64, []),
        "moe_forward_scratch": (ctypes.c_int, [P] + [vp] * 9 + [vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


# ---------------------------------------------------------------------------------------------
# host-only queries
# ---------------------------------------------------------------------------------------------
def status_str(status: int) -> str:
    return load().moe_status_str(int(status)).decode()


def moe_validate(p: Problem) -> int:
    return load().moe_validate(ctypes.byref(p))


def _checked(v: int, where: str) -> int:
    if v < 0:
        raise MoeError(int(v), where)
    return int(v)


def moe_pick_block_m(p: Problem) -> int:
    return _checked(load().moe_pick_block_m(ctypes.byref(p)), "moe_pick_block_m")


def moe_block_m_for(slots_per_expert: float, dtype="bf16", w_dtype=None) -> int:
    dt = _DT_NAME[dtype] if isinstance(dtype, str) else int(dtype)
    wdt = dt if w_dtype is None else (_DT_NAME[w_dtype] if isinstance(w_dtype, str) else int(w_dtype))
    return _checked(load().moe_block_m_for(float(slots_per_expert), dt, wdt), "moe_block_m_for")


def moe_max_padded_slots(p: Problem) -> int:
    return _checked(load().moe_max_padded_slots(ctypes.byref(p)), "moe_max_padded_slots")


def moe_max_tiles(p: Problem) -> int:
    return _checked(load().moe_max_tiles(ctypes.byref(p)), "moe_max_tiles")


def moe_workspace_bytes(p: Problem) -> int:
    return _checked(load().moe_workspace_bytes(ctypes.byref(p)), "moe_workspace_bytes")


def moe_gemm_workspace_bytes(p: Problem) -> int:
    return _checked(load().moe_gemm_workspace_bytes(ctypes.byref(p)), "moe_gemm_workspace_bytes")


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------
def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _act_dtype(p: Problem):
    return torch.uint8 if p.w_dtype == MOE_E4M3 else _TORCH_DT[p.dtype]


def _w_dtype(p: Problem):
    return (torch.float8_e4m3fn, torch.uint8) if p.w_dtype == MOE_E4M3 else _TORCH_DT[p.w_dtype]


# ---------------------------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------------------------
def moe_align(p: Problem, topk_ids, counts, offsets, sorted_slots, slot_row, tiles, num_tiles,
              n_invalid, stream=None) -> None:
    N = p.T * p.top_k
    rows = moe_max_padded_slots(p)
    mt = moe_max_tiles(p)
    i32 = torch.int32
    args = [_ptr(topk_ids, "topk_ids", i32, N), _ptr(counts, "counts", i32, p.E),
            _ptr(offsets, "offsets", i32, p.E + 1), _ptr(sorted_slots, "sorted_slots", i32, rows),
            _ptr(slot_row, "slot_row", i32, N), _ptr(tiles, "tiles", i32, 2 * mt),
            _ptr(num_tiles, "num_tiles", i32, 1), _ptr(n_invalid, "n_invalid", i32, 1)]
    _checked(load().moe_align(ctypes.byref(p), *args, _stream(stream)), "moe_align")


def moe_route(p: Problem, logits, renormalize: bool, topk_ids, topk_weights, stream=None) -> None:
    N = p.T * p.top_k
    args = [_ptr(logits, "logits", torch.float32, p.T * p.E), ctypes.c_int(1 if renormalize else 0),
            _ptr(topk_ids, "topk_ids", torch.int32, N), _ptr(topk_weights, "topk_weights", torch.float32, N)]
    _checked(load().moe_route(ctypes.byref(p), *args, _stream(stream)), "moe_route")


def moe_route_align(p: Problem, logits, renormalize: bool, topk_ids, topk_weights, counts, offsets,
                    sorted_slots, slot_row, tiles, num_tiles, n_invalid, stream=None) -> None:
    N = p.T * p.top_k
    rows = moe_max_padded_slots(p)
    mt = moe_max_tiles(p)
    i32 = torch.int32
    args = [_ptr(logits, "logits", torch.float32, p.T * p.E), ctypes.c_int(1 if renormalize else 0),
            _ptr(topk_ids, "topk_ids", i32, N), _ptr(topk_weights, "topk_weights", torch.float32, N),
            _ptr(counts, "counts", i32, p.E), _ptr(offsets, "offsets", i32, p.E + 1),
            _ptr(sorted_slots, "sorted_slots", i32, rows), _ptr(slot_row, "slot_row", i32, N),
            _ptr(tiles, "tiles", i32, 2 * mt), _ptr(num_tiles, "num_tiles", i32, 1),
            _ptr(n_invalid, "n_invalid", i32, 1)]
    _checked(load().moe_route_align(ctypes.byref(p), *args, _stream(stream)), "moe_route_align")


def moe_quantize_rows_e4m3(p: Problem, x, xq, scales, stream=None) -> None:
    args = [_ptr(x, "x", torch.bfloat16, p.T * p.H),
            _ptr(xq, "xq", (torch.uint8, torch.float8_e4m3fn), p.T * p.H),
            _ptr(scales, "scales", torch.float32, p.T * p.H // 128)]
    _checked(load().moe_quantize_rows_e4m3(ctypes.byref(p), *args, _stream(stream)),
             "moe_quantize_rows_e4m3")


def moe_grouped_gemm_up(p: Problem, x, x_scales, w13, w13_scales, sorted_slots, offsets, tiles,
                        num_tiles, act, act_scales, workspace=None, stream=None) -> None:
    rows = moe_max_padded_slots(p)
    fp8 = p.w_dtype == MOE_E4M3
    xdt = (torch.uint8, torch.float8_e4m3fn) if fp8 else _TORCH_DT[p.dtype]
    args = [_ptr(x, "x", xdt, p.T * p.H),
            _ptr(x_scales, "x_scales", torch.float32, p.T * p.H // 128),
            _ptr(w13, "w13", _w_dtype(p), p.E * 2 * p.I * p.H),
            _ptr(w13_scales, "w13_scales", torch.float32, p.E * (2 * p.I // 128) * (p.H // 128)),
            _ptr(sorted_slots, "sorted_slots", torch.int32, rows),
            _ptr(offsets, "offsets", torch.int32, p.E + 1),
            _ptr(tiles, "tiles", torch.int32, 2 * moe_max_tiles(p)),
            _ptr(num_tiles, "num_tiles", torch.int32, 1),
            _ptr(act, "act", (_act_dtype(p), torch.float8_e4m3fn) if fp8 else _act_dtype(p), rows * p.I),
            _ptr(act_scales, "act_scales", torch.float32, rows * p.I // 128),
            _ptr(workspace, "workspace", torch.uint8),
            0 if workspace is None else workspace.numel() * workspace.element_size()]
    _checked(load().moe_grouped_gemm_up(ctypes.byref(p), *args, _stream(stream)),
             "moe_grouped_gemm_up")


def moe_grouped_gemm_up_mxfp4(p: Problem, x, x_scale, w13, w13_scales, bias, alpha: float,
                              limit: float, out_scale, sorted_slots, offsets, tiles, num_tiles,
                              act, stream=None) -> None:
    rows = moe_max_padded_slots(p)
    u8 = (torch.uint8, torch.float8_e4m3fn)
    args = [_ptr(x, "x", u8, p.T * p.H),
            _ptr(x_scale, "x_scale", torch.float32, 1),
            _ptr(w13, "w13", torch.uint8, p.E * 2 * p.I * p.H // 2),
            _ptr(w13_scales, "w13_scales", torch.uint8, p.E * (p.H // 32) * 2 * p.I),
            _ptr(bias, "bias", torch.float32, p.E * 2 * p.I),
            ctypes.c_float(alpha), ctypes.c_float(limit),
            _ptr(out_scale, "out_scale", torch.float32, 1),
            _ptr(sorted_slots, "sorted_slots", torch.int32, rows),
            _ptr(offsets, "offsets", torch.int32, p.E + 1),
            _ptr(tiles, "tiles", torch.int32, 2 * moe_max_tiles(p)),
            _ptr(num_tiles, "num_tiles", torch.int32, 1),
            _ptr(act, "act", u8, rows * p.I)]
    _checked(load().moe_grouped_gemm_up_mxfp4(ctypes.byref(p), *args, _stream(stream)),
             "moe_grouped_gemm_up_mxfp4")


def moe_grouped_gemm_down(p: Problem, act, act_scales, w2, w2_scales, topk_weights, sorted_slots,
                          offsets, tiles, num_tiles, slot_out, workspace=None, stream=None) -> None:
    rows = moe_max_padded_slots(p)
    fp8 = p.w_dtype == MOE_E4M3
    args = [_ptr(act, "act", (_act_dtype(p), torch.float8_e4m3fn) if fp8 else _act_dtype(p), rows * p.I),
            _ptr(act_scales, "act_scales", torch.float32, rows * p.I // 128),
            _ptr(w2, "w2", _w_dtype(p), p.E * p.H * p.I),
            _ptr(w2_scales, "w2_scales", torch.float32, p.E * (p.H // 128) * (p.I // 128)),
            _ptr(topk_weights, "topk_weights", torch.float32, p.T * p.top_k),
            _ptr(sorted_slots, "sorted_slots", torch.int32, rows),
            _ptr(offsets, "offsets", torch.int32, p.E + 1),
            _ptr(tiles, "tiles", torch.int32, 2 * moe_max_tiles(p)),
            _ptr(num_tiles, "num_tiles", torch.int32, 1),
            _ptr(slot_out, "slot_out", _TORCH_DT[p.dtype], p.T * p.top_k * p.H),
            _ptr(workspace, "workspace", torch.uint8),
            0 if workspace is None else workspace.numel() * workspace.element_size()]
    _checked(load().moe_grouped_gemm_down(ctypes.byref(p), *args, _stream(stream)),
             "moe_grouped_gemm_down")


def moe_combine(p: Problem, slot_out, slot_row, out, stream=None) -> None:
    args = [_ptr(slot_out, "slot_out", _TORCH_DT[p.dtype], p.T * p.top_k * p.H),
            _ptr(slot_row, "slot_row", torch.int32, p.T * p.top_k),
            _ptr(out, "out", _TORCH_DT[p.dtype], p.T * p.H)]
    _checked(load().moe_combine(ctypes.byref(p), *args, _stream(stream)), "moe_combine")


def moe_forward(p: Problem, x, topk_ids, topk_weights, w13, w13_scales, w2, w2_scales, out,
                workspace, stream=None) -> None:
    ws_bytes = moe_workspace_bytes(p)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        raise MoeError(MOE_ERR_WORKSPACE, "moe_forward")
    args = [_ptr(x, "x", _TORCH_DT[p.dtype], p.T * p.H),
            _ptr(topk_ids, "topk_ids", torch.int32, p.T * p.top_k),
            _ptr(topk_weights, "topk_weights", torch.float32, p.T * p.top_k),
            _ptr(w13, "w13", _w_dtype(p), p.E * 2 * p.I * p.H),
            _ptr(w13_scales, "w13_scales", torch.float32, p.E * (2 * p.I // 128) * (p.H // 128)),
            _ptr(w2, "w2", _w_dtype(p), p.E * p.H * p.I),
            _ptr(w2_scales, "w2_scales", torch.float32, p.E * (p.H // 128) * (p.I // 128)),
            _ptr(out, "out", _TORCH_DT[p.dtype], p.T * p.H),
            _ptr(workspace, "workspace")]
    _checked(load().moe_forward(ctypes.byref(p), *args, ctypes.c_size_t(ws_bytes), _stream(stream)),
             "moe_forward")


def moe_scratch_max_bytes() -> int:
    return int(load().moe_scratch_max_bytes())


def moe_forward_scratch(p: Problem, x, topk_ids, topk_weights, w13, w13_scales, w2, w2_scales,
                        out, n_invalid=None, stream=None) -> None:
    args = [_ptr(x, "x", _TORCH_DT[p.dtype], p.T * p.H),
            _ptr(topk_ids, "topk_ids", torch.int32, p.T * p.top_k),
            _ptr(topk_weights, "topk_weights", torch.float32, p.T * p.top_k),
            _ptr(w13, "w13", _w_dtype(p), p.E * 2 * p.I * p.H),
            _ptr(w13_scales, "w13_scales", torch.float32, p.E * (2 * p.I // 128) * (p.H // 128)),
            _ptr(w2, "w2", _w_dtype(p), p.E * p.H * p.I),
            _ptr(w2_scales, "w2_scales", torch.float32, p.E * (p.H // 128) * (p.I // 128)),
            _ptr(out, "out", _TORCH_DT[p.dtype], p.T * p.H),
            _ptr(n_invalid, "n_invalid", torch.int32, 1)]
    _checked(load().moe_forward_scratch(ctypes.byref(p), *args, _stream(stream)),
             "moe_forward_scratch")
