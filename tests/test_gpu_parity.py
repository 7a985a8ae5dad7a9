"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Bars: alignment, quantisation codes and the combine are bit-exact; the layer output
meets max|gpu - oracle| / max|oracle| <= 1e-4 (fp32), 2e-2 (bf16), 6e-2 (fp8 weights).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import CONFIGS, get_config, make_case

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    denom = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (denom if denom > 0 else 1.0))


def problem_of(cfg, block_m=0):
    return moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, cfg.x_dtype, cfg.w_dtype, block_m)


def tol_of(cfg):
    return TOL[cfg.w_dtype] if cfg.w_dtype == "e4m3" else TOL[cfg.x_dtype]


def to_np(t):
    return t.detach().cpu().numpy()


def check_alignment(p, ids_dev, ids_host):
    a = moe.align(p, ids_dev)
    torch.cuda.synchronize()
    bm = moe.moe_pick_block_m(p)
    o = oracle.align(ids_host, p.E, bm)
    assert to_np(a["counts"]).tolist() == o.counts.tolist()
    assert to_np(a["offsets"]).tolist() == o.offsets.tolist()
    assert np.array_equal(to_np(a["sorted_slots"]), o.sorted_slots)
    assert np.array_equal(to_np(a["slot_row"]), o.slot_row)
    assert np.array_equal(to_np(a["tiles"]).reshape(-1, 2), o.tiles)
    assert int(a["num_tiles"].item()) == o.num_tiles
    assert int(a["n_invalid"].item()) == o.n_invalid
    return a, o


# ---------------------------------------------------------------------------------------------
# alignment: bit-exact
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(CONFIGS))
@pytest.mark.parametrize("bm", [0, 16, 64, 128])
def test_align_workloads_bit_exact(device, name, bm):
    cfg = CONFIGS[name]
    from moe_inputs import make_routing
    ids, _, _ = make_routing(cfg, 0)
    say(f"align {name} bm={bm}")
    check_alignment(problem_of(cfg, bm), torch.from_numpy(ids).to(device), ids)


def adversarial():
    rng = np.random.default_rng(7)
    yield "all_on_one_expert", np.full((1000, 3), 5, np.int32), 8
    yield "one_expert_nonempty_E256", np.full((4, 2), 200, np.int32), 256
    yield "E256_fewer_slots", rng.integers(0, 256, (5, 8)).astype(np.int32), 256
    yield "duplicates_in_token", rng.integers(0, 3, (500, 4)).astype(np.int32), 4
    yield "single_slot", np.array([[2]], np.int32), 4
    yield "invalid_ids", np.where(rng.random((300, 2)) < 0.1, -3, rng.integers(0, 6, (300, 2))).astype(np.int32), 6
    yield "id_equal_E", np.array([[0, 6], [6, 1], [5, 6]], np.int32), 6
    yield "many_chunks_E1024", rng.integers(0, 1024, (3000, 8)).astype(np.int32), 1024
    yield "E1", np.zeros((77, 1), np.int32), 1
    # chunked path (more than 8192 slots): ragged last chunk, invalid ids, one hot expert
    yield "chunks_ragged_invalid", np.where(rng.random((5003, 3)) < 0.1, 40,
                                            rng.integers(0, 40, (5003, 3))).astype(np.int32), 40
    yield "chunks_just_above_limit", np.full((4100, 2), 3, np.int32), 8
    yield "small_path_at_limit", rng.integers(0, 8, (4096, 2)).astype(np.int32), 8
    yield "chunks_skewed", np.minimum((64 * rng.random((9000, 6)) ** 3).astype(np.int32), 63), 64


@pytest.mark.parametrize("name,ids,E", list(adversarial()), ids=lambda v: v if isinstance(v, str) else "")
@pytest.mark.parametrize("bm", [16, 128])
def test_align_adversarial_bit_exact(device, name, ids, E, bm):
    T, k = ids.shape
    p = moe.make_problem(T, 128, 128, E, min(k, E), "bf16", block_m=bm)
    if k > E:
        pytest.skip("top_k > E is rejected by validation")
    say(f"align adversarial {name} bm={bm}")
    check_alignment(p, torch.from_numpy(ids).to(device), ids)


# ---------------------------------------------------------------------------------------------
# routing (logits -> top-k ids and weights): ids bit-exact (the selection compares the same fp32
# logits on both sides), weights to fp32 rounding of the softmax
# ---------------------------------------------------------------------------------------------
ROUTE_W_RTOL = 1e-5


def check_route(ids, w, logits32, k, renorm):
    o_ids, o_w = oracle.route(logits32.astype(np.float64), k, renorm)
    assert np.array_equal(to_np(ids), o_ids)
    assert np.allclose(to_np(w), o_w, rtol=ROUTE_W_RTOL, atol=1e-30)
    return o_ids


@pytest.mark.parametrize("name", list(CONFIGS))
def test_route_workloads(device, name):
    cfg = CONFIGS[name]
    from moe_inputs import make_logits
    lg = make_logits(cfg, 0).astype(np.float32)
    p = problem_of(cfg)
    say(f"route {name}")
    ids, w = moe.route(p, torch.from_numpy(lg).to(device), cfg.renormalize)
    torch.cuda.synchronize()
    check_route(ids, w, lg, cfg.top_k, cfg.renormalize)


def route_cases():
    rng = np.random.default_rng(21)
    yield "ties", rng.integers(-2, 3, (300, 16)).astype(np.float32), 4
    yield "E1", rng.standard_normal((50, 1)).astype(np.float32), 1
    yield "k_equals_E", rng.standard_normal((40, 8)).astype(np.float32), 8
    yield "E1024_k8", rng.standard_normal((70, 1024)).astype(np.float32) * 4, 8
    yield "E65_k64", rng.standard_normal((9, 65)).astype(np.float32), 64
    yield "E200_k6_ties", np.repeat(rng.integers(0, 3, (33, 25)).astype(np.float32), 8, axis=1), 6
    yield "T1", rng.standard_normal((1, 256)).astype(np.float32), 8
    yield "T128", rng.standard_normal((128, 256)).astype(np.float32), 8
    yield "T129", rng.standard_normal((129, 256)).astype(np.float32), 8
    yield "large_T", rng.standard_normal((5000, 64)).astype(np.float32) * 2, 6
    yield "E1024_T32", rng.standard_normal((32, 1024)).astype(np.float32), 8
    yield "E512_T64_k16", rng.standard_normal((64, 512)).astype(np.float32), 16


@pytest.mark.parametrize("name,lg,k", list(route_cases()), ids=lambda v: v if isinstance(v, str) else "")
@pytest.mark.parametrize("renorm", [False, True])
def test_route_and_route_align(device, name, lg, k, renorm):
    T, E = lg.shape
    p = moe.make_problem(T, 128, 128, E, k, "bf16")
    d = torch.from_numpy(lg).to(device)
    say(f"route {name} renorm={renorm}")
    ids, w = moe.route(p, d, renorm)
    a = moe.route_align(p, d, renorm)
    torch.cuda.synchronize()
    o_ids = check_route(ids, w, lg, k, renorm)
    assert torch.equal(a["topk_ids"], ids) and torch.equal(a["topk_weights"], w)
    o = oracle.align(o_ids, E, moe.moe_pick_block_m(p))
    assert to_np(a["counts"]).tolist() == o.counts.tolist()
    assert to_np(a["offsets"]).tolist() == o.offsets.tolist()
    assert np.array_equal(to_np(a["sorted_slots"]), o.sorted_slots)
    assert np.array_equal(to_np(a["slot_row"]), o.slot_row)
    assert np.array_equal(to_np(a["tiles"]).reshape(-1, 2), o.tiles)
    assert int(a["num_tiles"].item()) == o.num_tiles and int(a["n_invalid"].item()) == 0


# moe_route_align in one launch (up to 8192 slots): the last workgroup to finish its routing
# aligns the ids the others wrote.  Each call takes the next of the library's 64 completion
# counters and the last workgroup sets it back to zero, so 70 calls in a row use every counter
# and reuse some; calls on two streams at once use different counters.  Every call must equal
# moe_route followed by moe_align, bit for bit, into buffers refilled with junk first.  The
# 8194-slot case is just past the one-launch size (routing, then the alignment launches).
ROUTE_ALIGN_REPEAT = [(64, 256, 8, True), (4096, 8, 2, True), (300, 16, 4, False),
                      (1, 256, 8, True), (4097, 8, 2, True)]


@pytest.mark.parametrize("T,E,k,renorm", ROUTE_ALIGN_REPEAT)
def test_route_align_repeated_two_streams(device, T, E, k, renorm):
    rng = np.random.default_rng([T, E, k])
    lg = torch.from_numpy((rng.standard_normal((T, E)) * 2).astype(np.float32)).to(device)
    p = moe.make_problem(T, 128, 128, E, k, "bf16")
    say(f"route_align repeated T={T} E={E} k={k} N={T * k}")
    ids, w = moe.route(p, lg, renorm)
    ref = moe.align(p, ids)
    torch.cuda.synchronize()
    ref.update(topk_ids=ids, topk_weights=w)

    def buffers():
        b = moe.alloc_align(p, device)
        b["topk_ids"] = torch.empty((T, k), dtype=torch.int32, device=device)
        b["topk_weights"] = torch.empty((T, k), dtype=torch.float32, device=device)
        return b

    def call(b, stream):
        for v in b.values():
            v.fill_(-7 if v.dtype == torch.int32 else float("nan"))
        moe.moe_route_align(p, lg, renorm, b["topk_ids"], b["topk_weights"], b["counts"],
                            b["offsets"], b["sorted_slots"], b["slot_row"], b["tiles"],
                            b["num_tiles"], b["n_invalid"], stream)

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    b1, b2 = buffers(), buffers()
    torch.cuda.synchronize()
    for it in range(35):
        with torch.cuda.stream(s1):
            call(b1, s1)
        with torch.cuda.stream(s2):
            call(b2, s2)
        torch.cuda.synchronize()
        for b in (b1, b2):
            for key, v in ref.items():
                assert torch.equal(b[key], v), f"call {it}: {key}"


def test_align_deterministic_across_streams(device):
    cfg = CONFIGS["skewed_prefill_bf16"]
    from moe_inputs import make_routing
    ids, _, _ = make_routing(cfg, 0)
    p = problem_of(cfg)
    d = torch.from_numpy(ids).to(device)
    a = moe.align(p, d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = moe.align(p, d, stream=s)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


# ---------------------------------------------------------------------------------------------
# fp8 activation quantisation and combine: bit-exact
# ---------------------------------------------------------------------------------------------
def test_quantize_rows_bit_exact(device):
    rng = np.random.default_rng(12)
    T, H = 67, 1024
    x = (rng.standard_normal((T, H)) * 10.0 ** rng.uniform(-6, 3, (T, 1))).astype(np.float32)
    x[3, 256:384] = 0.0
    x[4, :128] = 1e-30
    x[5, 128:256] = -x[5, 128:256]
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xf = xb.to(torch.float32).numpy()
    p = moe.make_problem(T, H, 128, 4, 2, "bf16", "e4m3")
    xq = torch.empty((T, H), dtype=torch.uint8, device=device)
    sc = torch.empty((T, H // 128), dtype=torch.float32, device=device)
    moe.moe_quantize_rows_e4m3(p, xb.to(device), xq, sc)
    torch.cuda.synchronize()
    codes, s = oracle.quantize_groups_e4m3(xf, 128)
    assert np.array_equal(to_np(sc), s)
    assert np.array_equal(to_np(xq), codes)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_combine_bit_exact_ordered(device, dtype):
    rng = np.random.default_rng(13)
    T, k, H = 50, 4, 256
    y = (rng.standard_normal((T * k, H)) * 10.0 ** rng.integers(-3, 8, (T * k, 1))).astype(np.float32)
    y[0:4, 0] = [1e8, 1.0, -1e8, 1.0]          # order-sensitive cancellation
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    yt = torch.from_numpy(y).to(tdt)
    yv = yt.to(torch.float32).numpy()
    slot_row = np.arange(T * k, dtype=np.int32)
    slot_row[[5, 17, 18]] = -1                  # excluded slots are skipped
    p = moe.make_problem(T, H, 128, 8, k, dtype)
    out = torch.empty((T, H), dtype=tdt, device=device)
    moe.moe_combine(p, yt.to(device), torch.from_numpy(slot_row).to(device), out)
    torch.cuda.synchronize()
    yz = yv.copy()
    yz[slot_row < 0] = 0.0
    ref = oracle.combine(yz, k, np.float32)
    if dtype == "bf16":
        ref = oracle.bf16_round(ref)
    got = out.to(torch.float32).cpu().numpy()
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------------------------
# stage parity at small sizes (several tiles, ragged tails, every block size)
# ---------------------------------------------------------------------------------------------
SMALL = {
    "tiny_fp32": dict(),
    "mixtral_prefill_bf16": dict(T=300, H=256, I=384),
    "dsv3_decode_bf16": dict(T=64, H=512, I=256),
    "skewed_prefill_bf16": dict(T=1000, H=256, I=384),
    "dsv3_fp8_e4m3": dict(T=200, H=512, I=256, E=16),
    # H an odd multiple of 128: the widest n-blocks do not divide it
    "dsv3_decode_bf16@h384": dict(T=48, H=384, I=384),
    "dsv3_fp8_e4m3@h384": dict(T=120, H=384, I=384, E=16),
    # H and I odd multiples of 64 (64-wide n-blocks; GPT-OSS has H = I = 2880)
    "mixtral_prefill_bf16@h64": dict(T=300, H=192, I=320),
    "tiny_fp32@h64": dict(H=192, I=320),
}

_cases = {}


def small_case(name, device):
    if name not in _cases:
        cfg = get_config(name.split("@")[0], **SMALL[name])
        _cases[name] = make_case(cfg, device, seed=0)
    return _cases[name]


def expert_getter(case, cache=True):
    if not cache:
        return case.expert_host
    memo = {}

    def get(e):
        if e not in memo:
            memo[e] = case.expert_host(e)
        return memo[e]
    return get


def dequant_act(act, scales, fp8):
    if not fp8:
        return to_np(act.to(torch.float32))
    return oracle.dequantize_groups(to_np(act.view(torch.uint8)), to_np(scales), 128)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_stages_small(device, name, bm):
    case = small_case(name, device)
    cfg = case.cfg
    if bm == 256 and not (cfg.x_dtype == cfg.w_dtype == "bf16"):
        pytest.skip("256-row m-blocks are for bf16 problems only")
    fp8 = cfg.w_dtype == "e4m3"
    p = problem_of(cfg, bm)
    say(f"stages {name} bm={bm} {p}")
    a, o = check_alignment(p, case.topk_ids, case.ids_host)
    rows = moe.moe_max_padded_slots(p)
    if fp8:   # e4m3 code 0x7F is NaN: rows the kernel must write start as NaN
        act = torch.full((rows, cfg.I), 0x7F, dtype=torch.uint8, device=device)
    else:
        act = torch.full((rows, cfg.I), float("nan"), dtype=case.x.dtype, device=device)
    act_scales = torch.zeros((rows, cfg.I // 128), dtype=torch.float32, device=device) if fp8 else None
    x_in, x_sc = case.x, None
    if fp8:
        x_in = torch.empty((cfg.T, cfg.H), dtype=torch.uint8, device=device)
        x_sc = torch.empty((cfg.T, cfg.H // 128), dtype=torch.float32, device=device)
        moe.moe_quantize_rows_e4m3(p, case.x, x_in, x_sc)
    moe.moe_grouped_gemm_up(p, x_in, x_sc, case.w13, case.w13_scales, a["sorted_slots"], a["offsets"], a["tiles"],
                            a["num_tiles"], act, act_scales)
    slot_out = torch.full((cfg.T * cfg.top_k, cfg.H), float("nan"), dtype=case.x.dtype, device=device)
    moe.moe_grouped_gemm_down(p, act, act_scales, case.w2, case.w2_scales, case.topk_weights,
                              a["sorted_slots"], a["offsets"], a["tiles"], a["num_tiles"], slot_out)
    out = torch.empty((cfg.T, cfg.H), dtype=case.x.dtype, device=device)
    moe.moe_combine(p, slot_out, a["slot_row"], out)
    torch.cuda.synchronize()

    get = expert_getter(case)
    xh = case.x_host()
    if fp8:
        xq, sx = oracle.quantize_groups_e4m3(xh, 128)
        x_used = oracle.dequantize_groups(xq, sx, 128)
    else:
        x_used = xh.astype(np.float64)
    act_g = dequant_act(act, act_scales, fp8)
    used = o.offsets[-1]
    assert not np.isnan(act_g[:used]).any()
    # up: each valid row against the oracle's expert_up; padding rows exactly zero
    worst_up = 0.0
    for e in range(cfg.E):
        lo, c, hi = o.offsets[e], o.counts[e], o.offsets[e + 1]
        if c == 0:
            continue
        w13_e = get(e)[0]
        if fp8:
            w13_e = oracle.dequantize_blocks(w13_e, get(e)[2], 128)
        slots = o.sorted_slots[lo:lo + c]
        ref = oracle.expert_up(x_used[slots // cfg.top_k], w13_e)
        worst_up = max(worst_up, rel_err(act_g[lo:lo + c], ref))
        assert np.all(act_g[lo + c:hi] == 0), f"padding rows of expert {e} not zero"
    # down: against the oracle's expert_down applied to the GPU's own act rows
    so = to_np(slot_out.to(torch.float32))
    worst_down = 0.0
    for e in range(cfg.E):
        lo, c = o.offsets[e], o.counts[e]
        if c == 0:
            continue
        w2_e = get(e)[1]
        if fp8:
            w2_e = oracle.dequantize_blocks(w2_e, get(e)[3], 128)
        slots = o.sorted_slots[lo:lo + c]
        ref = oracle.expert_down(act_g[lo:lo + c], w2_e) * case.w_host.reshape(-1)[slots, None]
        worst_down = max(worst_down, rel_err(so[slots], ref))
    # layer
    ref_out = oracle.moe_layer(xh, case.ids_host, case.w_host, get, cfg.E, fp8=fp8)
    err = rel_err(to_np(out.to(torch.float32)), ref_out)
    say(f"  up {worst_up:.3e} down {worst_down:.3e} layer {err:.3e}")
    tol = tol_of(cfg)
    assert worst_up <= tol and worst_down <= tol and err <= tol


# ---------------------------------------------------------------------------------------------
# moe_forward: whole layer, edge cases, determinism
# ---------------------------------------------------------------------------------------------
def run_forward(case, bm=0, stream=None):
    cfg = case.cfg
    p = problem_of(cfg, bm)
    ws = moe.alloc_workspace(p, case.x.device)
    out = moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2,
                      case.w13_scales, case.w2_scales, workspace=ws, stream=stream)
    return out, ws


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_and_deterministic(device, name):
    case = small_case(name, device)
    say(f"forward {name}")
    out1, _ = run_forward(case)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out2, _ = run_forward(case, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, expert_getter(case),
                           case.cfg.E, fp8=case.cfg.w_dtype == "e4m3")
    err = rel_err(to_np(out1.to(torch.float32)), ref)
    say(f"  layer rel err {err:.3e}")
    assert err <= tol_of(case.cfg)


def custom_case(device, cfg, ids):
    case = make_case(cfg, device, seed=3)
    case.ids_host = ids.astype(np.int32)
    case.topk_ids = torch.from_numpy(case.ids_host).to(device)
    return case


@pytest.mark.parametrize("label,kw,ids_fn", [
    ("single_token", dict(T=1, H=256, I=256, E=4, top_k=1), lambda rng, c: np.array([[2]])),
    ("all_to_one_expert", dict(T=700, H=256, I=256, E=8, top_k=2),
     lambda rng, c: np.stack([np.full(c.T, 3), np.full(c.T, 5)], 1)),
    ("E256_fewer_slots", dict(T=3, H=256, I=256, E=256, top_k=8),
     lambda rng, c: np.stack([rng.permutation(256)[:8] for _ in range(c.T)])),
    ("invalid_ids", dict(T=40, H=256, I=256, E=8, top_k=2),
     lambda rng, c: np.where(rng.random((c.T, 2)) < 0.2, 8, rng.integers(0, 8, (c.T, 2)))),
])
@pytest.mark.parametrize("base", ["mixtral_prefill_bf16", "tiny_fp32", "dsv3_fp8_e4m3"])
def test_forward_edge_cases(device, label, kw, ids_fn, base):
    cfg = get_config(base, **kw)
    ids = ids_fn(np.random.default_rng(21), cfg)
    case = custom_case(device, cfg, ids)
    say(f"edge {label} {base}")
    out, ws = run_forward(case)
    torch.cuda.synchronize()
    n_invalid = int(ws[:4].view(torch.int32).item())
    assert n_invalid == int(((ids < 0) | (ids >= cfg.E)).sum())
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, expert_getter(case), cfg.E,
                           fp8=cfg.w_dtype == "e4m3")
    err = rel_err(to_np(out.to(torch.float32)), ref)
    say(f"  rel err {err:.3e}")
    assert err <= tol_of(cfg)


# ---------------------------------------------------------------------------------------------
# full-size workloads: every output row against the oracle, in the launch configuration the
# benchmark times (moe_forward with its workspace, so the GEMMs' K-split tail is active).  The
# oracle streams one expert's weights to the host at a time and evaluates experts on several
# threads (identical arithmetic, see oracle.moe_layer).
# ---------------------------------------------------------------------------------------------
ORACLE_THREADS = 8


@pytest.mark.parametrize("name", list(CONFIGS))
def test_forward_full_size_every_row(device, name):
    import time
    cfg = CONFIGS[name]
    say(f"full-size {name}: generating")
    case = make_case(cfg, device, seed=0)
    torch.cuda.synchronize()
    say(f"full-size {name}: running")
    check_alignment(problem_of(cfg), case.topk_ids, case.ids_host)
    out, ws = run_forward(case)
    torch.cuda.synchronize()
    got = to_np(out.to(torch.float32))
    del ws
    assert np.isfinite(got).all()
    t0 = time.perf_counter()
    say(f"full-size {name}: oracle on all {cfg.T} tokens")
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host,
                           expert_getter(case, cache=False), cfg.E,
                           fp8=cfg.w_dtype == "e4m3", workers=ORACLE_THREADS)
    assert ref.shape == got.shape
    err = rel_err(got, ref)
    # the worst row, to name it if the bar fails
    row_err = np.abs(got - ref).max(axis=1) / np.abs(ref).max()
    worst = int(np.argmax(row_err))
    say(f"  rel err {err:.3e} over {cfg.T} rows x {cfg.H} (worst row {worst}, "
        f"experts {case.ids_host[worst].tolist()}); oracle {time.perf_counter() - t0:.1f} s")
    assert err <= tol_of(cfg)
    del case
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------------
# maximum dimensions: the largest K (H = 32768, the whole zero row) and an expert weight slab
# just under 2^31 bytes (the limit of the kernels' 32-bit in-slab offsets), through every GEMM
# family: streaming (block_m 64), prefill (128, 256) and e4m3
# ---------------------------------------------------------------------------------------------
MAX_DIMS = {
    "bf16_bm64": ("mixtral_prefill_bf16", dict(T=24, H=32768, I=16256, E=2, top_k=2), 64),
    "bf16_bm128": ("mixtral_prefill_bf16", dict(T=24, H=32768, I=16256, E=2, top_k=2), 128),
    "bf16_bm256": ("mixtral_prefill_bf16", dict(T=24, H=32768, I=16256, E=2, top_k=2), 256),
    "e4m3_bm128": ("dsv3_fp8_e4m3", dict(T=24, H=32768, I=32640, E=2, top_k=2), 128),
}


@pytest.mark.parametrize("label", list(MAX_DIMS))
def test_forward_full_size_max_dims(device, label):
    base, kw, bm = MAX_DIMS[label]
    cfg = get_config(base, **kw)
    p = problem_of(cfg, bm)
    assert moe.moe_validate(p) == moe.MOE_OK
    say(f"max dims {label}: generating")
    case = make_case(cfg, device, seed=3)
    torch.cuda.synchronize()
    say(f"max dims {label}: running")
    check_alignment(p, case.topk_ids, case.ids_host)
    out, _ = run_forward(case, bm)
    torch.cuda.synchronize()
    say(f"max dims {label}: oracle")
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host,
                           expert_getter(case, cache=False), cfg.E, fp8=cfg.w_dtype == "e4m3")
    got = to_np(out.to(torch.float32))
    err = rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= tol_of(cfg)
    del case
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------------
# the expert-parallel shard of the batch sweep: 16 local experts of 128, so most slots carry ids
# of other shards (excluded and counted); production-like skew (one expert holds most tokens)
# ---------------------------------------------------------------------------------------------
SHARD = "gptoss_shard_bf16"
SHARD_POINTS = {0: None, 9: None, 20: None, 47: None}   # sweep index -> sampled tokens (None: all)


@pytest.mark.parametrize("idx", list(SHARD_POINTS))
def test_shard_sweep_points(device, idx):
    from moe_inputs import SWEEP_CONFIGS, sweep_batch_sizes
    base = SWEEP_CONFIGS[SHARD]
    T = sweep_batch_sizes(base.route_experts, base.top_k)[idx]
    cfg = get_config(SHARD, T=T)
    say(f"shard T={T}: generating")
    case = make_case(cfg, device, seed=0)
    p = problem_of(cfg)
    check_alignment(p, case.topk_ids, case.ids_host)
    out, ws = run_forward(case)
    torch.cuda.synchronize()
    n_local = int(((case.ids_host >= 0) & (case.ids_host < cfg.E)).sum())
    assert int(ws[:4].view(torch.int32).item()) == cfg.T * cfg.top_k - n_local
    got_all = to_np(out.to(torch.float32))
    # a token none of whose experts is local gets an exactly zero row (at the smallest batches
    # every token reaches the hot local expert, so there may be none)
    foreign = ~((case.ids_host < cfg.E).any(axis=1))
    assert (got_all[foreign] == 0).all()
    n = SHARD_POINTS[idx]
    if n is None:
        toks = list(range(cfg.T))
    else:
        rng = np.random.default_rng(7)
        counts = np.bincount(case.ids_host.reshape(-1), minlength=cfg.route_experts)[:cfg.E]
        lo = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))   # least-loaded active expert
        hot = int(np.argmax(counts))
        pick = {int(np.nonzero((case.ids_host == e).any(axis=1))[0][-1]) for e in (lo, hot)}
        local = np.nonzero(~foreign)[0]
        toks = sorted(set(rng.choice(local, n - 2, replace=False).tolist()) | pick)
    say(f"shard T={T}: oracle on {len(toks)} tokens (block_m {moe.moe_pick_block_m(p)})")
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, expert_getter(case),
                           cfg.E, tokens=toks, workers=ORACLE_THREADS)
    err = rel_err(got_all[toks], ref)
    say(f"  rel err {err:.3e}")
    assert np.isfinite(got_all).all()
    assert err <= tol_of(cfg)
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_shard_every_block_m(device, bm):
    from moe_inputs import SWEEP_CONFIGS, sweep_batch_sizes
    base = SWEEP_CONFIGS[SHARD]
    T = sweep_batch_sizes(base.route_experts, base.top_k)[14]
    cfg = get_config(SHARD, T=T)
    say(f"shard T={T} block_m {bm}")
    case = make_case(cfg, device, seed=1)
    check_alignment(problem_of(cfg, bm), case.topk_ids, case.ids_host)
    out, _ = run_forward(case, bm)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, expert_getter(case), cfg.E)
    err = rel_err(to_np(out.to(torch.float32)), ref)
    say(f"  rel err {err:.3e}")
    assert err <= tol_of(cfg)
    del case
    torch.cuda.empty_cache()
