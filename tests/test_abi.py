"""C-ABI tests that need no GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import oracle
import routed_grouped_gemm_topk_amd as moe
from routed_grouped_gemm_topk_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return moe.load()


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(-7, 1):
        assert moe.status_str(code).startswith("MOE_")
    assert "unknown" in moe.status_str(-99)


def bad(**kw):
    base = dict(T=16, H=128, I=256, E=8, top_k=2, dtype="bf16")
    base.update(kw)
    return moe.make_problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), moe.MOE_ERR_SHAPE), (dict(H=100), moe.MOE_ERR_SHAPE), (dict(I=160), moe.MOE_ERR_SHAPE),
    (dict(I=192, w_dtype="e4m3"), moe.MOE_ERR_SHAPE), (dict(H=64, w_dtype="e4m3"), moe.MOE_ERR_SHAPE),
    (dict(E=0), moe.MOE_ERR_SHAPE), (dict(E=1025, top_k=2), moe.MOE_ERR_SHAPE),
    (dict(top_k=0), moe.MOE_ERR_SHAPE), (dict(top_k=9), moe.MOE_ERR_SHAPE),
    (dict(block_m=48), moe.MOE_ERR_SHAPE), (dict(block_m=512), moe.MOE_ERR_SHAPE),
    (dict(block_m=256, dtype="f32"), moe.MOE_ERR_SHAPE), (dict(block_m=256, w_dtype="e4m3"), moe.MOE_ERR_SHAPE),
    (dict(dtype="f32", w_dtype="bf16"), moe.MOE_ERR_DTYPE), (dict(dtype="e4m3"), moe.MOE_ERR_DTYPE),
    (dict(dtype="f32", w_dtype="e4m3"), moe.MOE_ERR_DTYPE),
    (dict(H=2 ** 15 + 128), moe.MOE_ERR_SHAPE),                  # above the largest H
    (dict(H=2 ** 15, I=2 ** 15, dtype="f32"), moe.MOE_ERR_SHAPE),  # one expert slab >= 2^31 bytes
])
def test_validation_codes(kw, code):
    assert moe.moe_validate(bad(**kw)) == code
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_bytes(bad(**kw))


def test_multiples_of_64_are_valid_for_bf16_and_fp32():
    for dt in ("bf16", "f32"):
        assert moe.moe_validate(bad(H=192, I=2880, dtype=dt, w_dtype=dt)) == moe.MOE_OK
        assert moe.moe_validate(bad(H=64, I=64, dtype=dt, w_dtype=dt)) == moe.MOE_OK


def test_null_problem(lib):
    assert lib.moe_validate(None) == moe.MOE_ERR_NULL
    assert lib.moe_align(None, *([None] * 9)) == moe.MOE_ERR_NULL


def test_entry_points_reject_before_any_hip_call(lib):
    """Shape errors win over NULL pointers, NULL pointers over device checks, and a short
    workspace is reported before the device is touched (this host has no GPU)."""
    p = bad(H=100)
    P = ctypes.byref(p)
    assert lib.moe_align(P, *([None] * 9)) == moe.MOE_ERR_SHAPE
    assert lib.moe_grouped_gemm_up(P, *([None] * 11), 0, None) == moe.MOE_ERR_SHAPE
    assert lib.moe_grouped_gemm_down(P, *([None] * 11), 0, None) == moe.MOE_ERR_SHAPE
    assert lib.moe_combine(P, None, None, None, None) == moe.MOE_ERR_SHAPE
    assert lib.moe_forward(P, *([None] * 9), 0, None) == moe.MOE_ERR_SHAPE
    p = bad()
    P = ctypes.byref(p)
    assert lib.moe_align(P, *([None] * 9)) == moe.MOE_ERR_NULL
    assert lib.moe_grouped_gemm_up(P, *([None] * 11), 0, None) == moe.MOE_ERR_NULL
    assert lib.moe_grouped_gemm_down(P, *([None] * 11), 0, None) == moe.MOE_ERR_NULL
    assert lib.moe_combine(P, None, None, None, None) == moe.MOE_ERR_NULL
    assert lib.moe_quantize_rows_e4m3(P, 8, 8, 8, None) == moe.MOE_ERR_DTYPE   # bf16 weights
    fake = [ctypes.c_void_p(256)] * 9
    need = moe.moe_workspace_bytes(p)
    assert lib.moe_forward(P, *fake, need - 1, None) == moe.MOE_ERR_WORKSPACE
    pf = bad(w_dtype="e4m3")
    assert lib.moe_forward(ctypes.byref(pf), *fake[:4], None, fake[5], None, fake[7], fake[8],
                           10 ** 12, None) == moe.MOE_ERR_NULL


@pytest.mark.parametrize("T,H,I,E,k,dt,wdt,bm", [
    (16, 128, 256, 8, 2, "f32", "f32", 16), (4096, 4096, 14336, 8, 2, "bf16", "bf16", 256),
    (64, 7168, 2048, 256, 8, "bf16", "bf16", 16), (8192, 2048, 1408, 64, 6, "bf16", "bf16", 256),
    (2048, 4096, 1024, 8, 1, "bf16", "bf16", 256), (1024, 4096, 1024, 8, 1, "bf16", "bf16", 128),
    (4096, 4096, 1024, 8, 1, "f32", "f32", 128), (640, 2880, 2880, 16, 1, "bf16", "bf16", 64),
    (2048, 7168, 2048, 256, 8, "bf16", "e4m3", 128), (1, 128, 128, 4, 1, "bf16", "bf16", 16),
])
def test_block_m_choice_and_bounds(T, H, I, E, k, dt, wdt, bm):
    p = moe.make_problem(T, H, I, E, k, dt, wdt)
    assert moe.moe_pick_block_m(p) == bm
    assert moe.moe_max_padded_slots(p) == oracle.max_padded_slots(T * k, E, bm)
    assert moe.moe_max_tiles(p) == oracle.max_tiles(T * k, E, bm)
    for forced in (16, 32, 64, 128) + ((256,) if dt == wdt == "bf16" else ()):
        q = moe.make_problem(T, H, I, E, k, dt, wdt, block_m=forced)
        assert moe.moe_pick_block_m(q) == forced
        assert moe.moe_max_tiles(q) == oracle.max_tiles(T * k, E, forced)
    assert moe.moe_workspace_bytes(p) % 256 == 0


def test_block_m_for_expected_slots():
    """The rule behind moe_pick_block_m, keyed on expected slots per expert; an
    expert-parallel caller passes T*top_k/E_total."""
    bf = [(1, 16), (10, 16), (10.5, 32), (28, 32), (29, 64), (64, 64), (65, 128), (128, 128),
          (129, 256), (1e6, 256), (0, 16)]
    for m, bm in bf:
        assert moe.moe_block_m_for(m, "bf16") == bm, m
    for m, bm in [(8, 16), (20, 32), (40, 64), (41, 128), (1e6, 128)]:
        assert moe.moe_block_m_for(m, "bf16", "e4m3") == bm
        assert moe.moe_block_m_for(m, "f32") == bm
    for T, H, I, E, k, dt, wdt in [(4096, 4096, 14336, 8, 2, "bf16", "bf16"),
                                   (2048, 7168, 2048, 256, 8, "bf16", "e4m3"),
                                   (333, 2880, 2880, 16, 4, "bf16", "bf16"), (16, 128, 256, 8, 2, "f32", "f32")]:
        p = moe.make_problem(T, H, I, E, k, dt, wdt)
        assert moe.moe_pick_block_m(p) == moe.moe_block_m_for(T * k / E, dt, wdt)
    lib = moe.load()
    assert lib.moe_block_m_for(-1.0, moe.MOE_BF16, moe.MOE_BF16) == moe.MOE_ERR_SHAPE
    assert lib.moe_block_m_for(float("nan"), moe.MOE_BF16, moe.MOE_BF16) == moe.MOE_ERR_SHAPE
    assert lib.moe_block_m_for(4.0, moe.MOE_F32, moe.MOE_BF16) == moe.MOE_ERR_DTYPE
    assert lib.moe_block_m_for(4.0, moe.MOE_E4M3, moe.MOE_E4M3) == moe.MOE_ERR_DTYPE


def test_binding_rejects_host_tensors():
    import torch
    p = bad()
    with pytest.raises(ValueError):
        moe.moe_combine(p, torch.zeros(16 * 2 * 128, dtype=torch.bfloat16),
                        torch.zeros(32, dtype=torch.int32), torch.zeros(16 * 128, dtype=torch.bfloat16))


def test_route_entry_points_validate_on_the_host(lib):
    """moe_route / moe_route_align: shape errors, the top_k <= 64 limit, then NULL pointers."""
    p = bad(H=100)
    assert lib.moe_route(ctypes.byref(p), None, 0, None, None, None) == moe.MOE_ERR_SHAPE
    assert lib.moe_route_align(ctypes.byref(p), None, 0, *([None] * 10)) == moe.MOE_ERR_SHAPE
    p = moe.make_problem(4, 128, 128, 100, 65, "bf16")          # top_k above 64
    assert lib.moe_route(ctypes.byref(p), None, 0, None, None, None) == moe.MOE_ERR_SHAPE
    p = bad()
    assert lib.moe_route(ctypes.byref(p), None, 0, None, None, None) == moe.MOE_ERR_NULL
    assert lib.moe_route_align(ctypes.byref(p), None, 1, *([None] * 10)) == moe.MOE_ERR_NULL


def test_mxfp4_problem_validation(lib):
    """MXFP4 weights x e4m3 rows: only the MX up projection (and the dtype-free alignment and
    routing) accept the pair; the MX entry point rejects every other pair."""
    mxp = moe.make_problem(16, 192, 128, 8, 2, "e4m3", "mxfp4")
    assert moe.moe_validate(mxp) == moe.MOE_OK
    assert moe.moe_pick_block_m(mxp) == moe.moe_block_m_for(4, "e4m3", "mxfp4") == 64
    assert moe.moe_block_m_for(128, "e4m3", "mxfp4") == 64
    assert moe.moe_block_m_for(128.5, "e4m3", "mxfp4") == 128
    for kw, code in [(dict(block_m=256), moe.MOE_ERR_SHAPE), (dict(H=96), moe.MOE_ERR_SHAPE),
                     (dict(I=96), moe.MOE_ERR_SHAPE)]:
        base = dict(T=16, H=192, I=128, E=8, top_k=2, dtype="e4m3", w_dtype="mxfp4")
        base.update(kw)
        assert moe.moe_validate(moe.make_problem(**base)) == code, kw
    assert moe.moe_validate(moe.make_problem(16, 192, 128, 8, 2, "bf16", "mxfp4")) == moe.MOE_ERR_DTYPE
    P = ctypes.byref(mxp)
    f = [ctypes.c_void_p(256)] * 16
    assert lib.moe_workspace_bytes(P) == moe.MOE_ERR_DTYPE
    assert lib.moe_grouped_gemm_up(P, *f[:10], None, 0, None) == moe.MOE_ERR_DTYPE
    assert lib.moe_grouped_gemm_down(P, *f[:10], None, 0, None) == moe.MOE_ERR_DTYPE
    assert lib.moe_combine(P, *f[:3], None) == moe.MOE_ERR_DTYPE
    assert lib.moe_quantize_rows_e4m3(P, *f[:3], None) == moe.MOE_ERR_DTYPE
    assert lib.moe_forward(P, *f[:9], 10 ** 12, None) == moe.MOE_ERR_DTYPE
    mxargs = f[:5] + [ctypes.c_float(1.1), ctypes.c_float(1.4)] + f[:6]
    bf = ctypes.byref(bad())
    assert lib.moe_grouped_gemm_up_mxfp4(bf, *mxargs, None) == moe.MOE_ERR_DTYPE
    nulls = [None] * 5 + [ctypes.c_float(1.1), ctypes.c_float(1.4)] + [None] * 6
    assert lib.moe_grouped_gemm_up_mxfp4(P, *nulls, None) == moe.MOE_ERR_NULL


def test_misaligned_pointers_are_rejected_before_any_launch(lib):
    """Data arrays need 16-byte alignment, index/scale arrays 4, the workspace 256; a
    misaligned pointer returns MOE_ERR_ALIGN on the host (no device is touched)."""
    p = bad(T=16, H=128, I=256, E=8, top_k=2)
    P = ctypes.byref(p)
    ok, odd8, odd2 = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8), ctypes.c_void_p(4096 + 2)
    A = moe.MOE_ERR_ALIGN
    assert lib.moe_align(P, odd2, *[ok] * 7, None) == A
    assert lib.moe_align(P, ok, ok, ok, ok, ok, ok, ok, odd2, None) == A
    assert lib.moe_route(P, odd2, 0, ok, ok, None) == A
    assert lib.moe_route_align(P, ok, 0, ok, ok, ok, ok, ok, ok, odd2, ok, ok, None) == A
    assert lib.moe_grouped_gemm_up(P, odd8, None, ok, None, ok, ok, ok, ok, ok, None, None, 0, None) == A
    assert lib.moe_grouped_gemm_up(P, ok, None, ok, None, ok, ok, ok, ok, odd8, None, None, 0, None) == A
    assert lib.moe_grouped_gemm_down(P, ok, None, odd8, None, ok, ok, ok, ok, ok, ok, None, 0, None) == A
    assert lib.moe_grouped_gemm_down(P, ok, None, ok, None, odd2, ok, ok, ok, ok, ok, None, 0, None) == A
    assert lib.moe_combine(P, ok, ok, odd8, None) == A
    need = moe.moe_workspace_bytes(p)
    assert lib.moe_forward(P, ok, ok, ok, ok, None, ok, None, ok, ctypes.c_void_p(4096 + 128),
                           need, None) == A
    assert lib.moe_forward(P, ok, ok, odd2, ok, None, ok, None, ok, ok, need, None) == A
    pf = bad(w_dtype="e4m3")
    assert lib.moe_quantize_rows_e4m3(ctypes.byref(pf), odd8, ok, ok, None) == A
    mxp = ctypes.byref(moe.make_problem(16, 192, 128, 8, 2, "e4m3", "mxfp4"))
    args = [ok, ok, ok, ok, odd8, ctypes.c_float(1.1), ctypes.c_float(1.4), ok, ok, ok, ok, ok, ok]
    assert lib.moe_grouped_gemm_up_mxfp4(mxp, *args, None) == A           # bias
    args[4], args[-1] = ok, odd8
    assert lib.moe_grouped_gemm_up_mxfp4(mxp, *args, None) == A           # act


def test_gemm_workspace_size_and_checks(lib):
    """The GEMMs' optional workspace: 256 fp32 partial tiles of block_m rows x the widest
    partial tile of the two launches (up: gate + up columns; down: the n-block) for bf16
    problems on the 128/256-row kernels, 0 elsewhere; too small -> MOE_ERR_WORKSPACE,
    misaligned -> MOE_ERR_ALIGN, both on the host."""
    big = moe.make_problem(4096, 4096, 14336, 8, 2, "bf16")               # block_m 256
    assert moe.moe_pick_block_m(big) == 256
    assert moe.moe_gemm_workspace_bytes(big) == 256 * 256 * 256 * 4
    # H % 256 != 0: down n-block 128, up 2 x 128
    assert moe.moe_gemm_workspace_bytes(moe.make_problem(4096, 2880, 2880, 8, 2, "bf16")) \
        == 256 * 256 * 256 * 4
    assert moe.moe_gemm_workspace_bytes(moe.make_problem(64, 7168, 2048, 256, 8, "bf16")) == 0
    assert moe.moe_gemm_workspace_bytes(moe.make_problem(2048, 7168, 2048, 256, 8, "bf16", "e4m3")) == 0
    assert moe.moe_gemm_workspace_bytes(moe.make_problem(16, 128, 256, 8, 2, "f32")) == 0
    # moe_forward carves the same buffer out of its own workspace
    assert moe.moe_workspace_bytes(big) - moe.moe_workspace_bytes(moe.make_problem(
        4096, 4096, 14336, 8, 2, "bf16", block_m=64)) >= moe.moe_gemm_workspace_bytes(big)
    small = moe.make_problem(4096, 4096, 14336, 8, 2, "bf16", block_m=128)
    need = moe.moe_gemm_workspace_bytes(small)
    assert need == 256 * 128 * 512 * 4                                       # up: 2 x 256 columns
    assert moe.moe_gemm_workspace_bytes(moe.make_problem(4096, 4096, 2880, 8, 2, "bf16",
                                                         block_m=128)) == 256 * 128 * 256 * 4
    P = ctypes.byref(small)
    ok = ctypes.c_void_p(4096)
    W, A = moe.MOE_ERR_WORKSPACE, moe.MOE_ERR_ALIGN
    odd = ctypes.c_void_p(4096 + 64)
    assert lib.moe_grouped_gemm_down(P, ok, None, ok, None, ok, ok, ok, ok, ok, ok, ok, need - 1,
                                     None) == W
    assert lib.moe_grouped_gemm_down(P, ok, None, ok, None, ok, ok, ok, ok, ok, ok, odd, need,
                                     None) == A
    assert lib.moe_grouped_gemm_up(P, ok, None, ok, None, ok, ok, ok, ok, ok, None, ok, need - 1,
                                   None) == W
    assert lib.moe_grouped_gemm_up(P, ok, None, ok, None, ok, ok, ok, ok, ok, None, odd, need,
                                   None) == A


def test_forward_scratch_host_checks(lib):
    """moe_forward_scratch: validation before any HIP call -- null pointers, and a problem whose
    intermediates exceed the library-owned array (MOE_SCRATCH_MAX_BYTES) is refused."""
    assert moe.moe_scratch_max_bytes() == 128 << 20
    fake = 1 << 20                                   # never dereferenced
    small = moe.make_problem(64, 512, 256, 16, 4, "bf16")
    assert lib.moe_forward_scratch(ctypes.byref(small), None, fake, fake, fake, None, fake, None,
                                   fake, None, None) == moe.MOE_ERR_NULL
    big = moe.make_problem(4096, 4096, 14336, 8, 2, "bf16")
    assert moe.moe_workspace_bytes(big) > moe.moe_scratch_max_bytes()
    assert lib.moe_forward_scratch(ctypes.byref(big), fake, fake, fake, fake, None, fake, None,
                                   fake, None, None) == moe.MOE_ERR_WORKSPACE
    mx = moe.make_problem(64, 512, 256, 16, 4, "e4m3", "mxfp4")
    assert lib.moe_forward_scratch(ctypes.byref(mx), fake, fake, fake, fake, None, fake, None,
                                   fake, None, None) == moe.MOE_ERR_DTYPE
    odd = moe.make_problem(64, 512, 256, 16, 4, "bf16")
    assert lib.moe_forward_scratch(ctypes.byref(odd), fake + 8, fake, fake, fake, None, fake, None,
                                   fake, None, None) == moe.MOE_ERR_ALIGN
