"""Guard canaries around every output of the HIP path: no store lands outside its buffer.

Each output tensor is a contiguous view cut from the middle of a larger device buffer whose
guard regions (4 KiB on each side) hold a known byte pattern.  After the calls, every guard byte
must be unchanged, and so must the parts of the outputs the entry points promise not to write:
  * act rows past the last valid tile (moe_grouped_gemm_up; also act_scales for e4m3);
  * slot rows of excluded slots (moe_grouped_gemm_down);
  * padding rows and rows past the last tile of the MXFP4 act (moe_grouped_gemm_up_mxfp4);
  * everything past moe_workspace_bytes of moe_forward's workspace.
The cases cover the prefill GEMMs with the K-split tail and ragged last n-blocks (H or I =
2880, not a multiple of the 128-wide n-block), the streaming GEMMs (16- and 64-row m-blocks,
e4m3), the fp32 path, the alignment's one-workgroup and chunked paths, routing and the
combine.  Each case also checks the layer output against the oracle (layer tolerance).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_topk_amd as moe
from moe_inputs import get_config, make_case, make_mx_case

pytestmark = pytest.mark.gpu

G = 4096            # guard bytes on each side (keeps the body 256-byte aligned)
PAT = 0xA5
TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Guarded:
    """A tensor of `shape`/`dtype` inside a uint8 buffer with PAT-filled guards."""

    def __init__(self, shape, dtype, device, fill=None):
        elt = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(shape)) * elt
        self.elt = elt
        self.buf = torch.full((G + self.nbytes + G,), PAT, dtype=torch.uint8, device=device)
        self.t = self.buf[G:G + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)
        self.before = None

    def snapshot(self):
        self.before = self.buf.clone()

    def guards_intact(self) -> bool:
        return bool((self.buf[:G] == PAT).all()) and bool((self.buf[G + self.nbytes:] == PAT).all())

    def untouched(self, lo_byte: int, hi_byte: int) -> bool:
        """Body bytes [lo_byte, hi_byte) equal the snapshot."""
        a, b = G + lo_byte, G + hi_byte
        return torch.equal(self.buf[a:b], self.before[a:b])


def snapshot_all(gs):
    for g in gs:
        g.snapshot()


def assert_guards(named):
    bad = [n for n, g in named.items() if not g.guards_intact()]
    assert not bad, f"stores outside the buffer: {bad}"


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (d if d > 0 else 1.0))


# (base workload, sizes, block_m); ids of ~5% of slots set to E (excluded)
CASES = {
    "ksplit_bm256": ("mixtral_prefill_bf16", dict(T=512, H=1024, I=2048, E=4, top_k=2), 256),
    "ksplit_tail_bm256": ("mixtral_prefill_bf16", dict(T=4096, H=2048, I=1024, E=8, top_k=2), 256),
    "ragged_down_bm128": ("mixtral_prefill_bf16", dict(T=640, H=2880, I=1024, E=4, top_k=2), 128),
    "ragged_down_bm256": ("mixtral_prefill_bf16", dict(T=384, H=2880, I=1024, E=4, top_k=2), 256),
    "ragged_up_bm256": ("mixtral_prefill_bf16", dict(T=384, H=1024, I=2880, E=4, top_k=2), 256),
    "ragged_up_bm128": ("mixtral_prefill_bf16", dict(T=640, H=1024, I=2880, E=4, top_k=2), 128),
    "stream_bm16": ("dsv3_decode_bf16", dict(T=64, H=512, I=256, E=32, top_k=4), 16),
    "stream_bm64_h2880": ("mixtral_prefill_bf16", dict(T=200, H=2880, I=2880, E=16, top_k=4), 64),
    "fp8_bm128": ("dsv3_fp8_e4m3", dict(T=200, H=512, I=384, E=16, top_k=4), 128),
    "fp8_bm32": ("dsv3_fp8_e4m3", dict(T=64, H=384, I=256, E=32, top_k=4), 32),
    "f32_bm16": ("tiny_fp32", dict(), 16),
    "align_chunked_bm128": ("skewed_prefill_bf16", dict(T=3000, H=256, I=256, E=64, top_k=6), 128),
}


def excluded_ids(cfg, seed=11):
    from moe_inputs import make_routing
    ids, _, _ = make_routing(cfg, 0)
    rng = np.random.default_rng(seed)
    ids = ids.copy()
    ids[rng.random(ids.shape) < 0.05] = cfg.E
    ids[0, -1] = cfg.E                    # at least one
    return ids


@pytest.mark.parametrize("label", list(CASES))
def test_stage_outputs_stay_in_bounds(device, label):
    base, kw, bm = CASES[label]
    cfg = get_config(base, **kw)
    case = make_case(cfg, device, seed=2)
    case.ids_host = excluded_ids(cfg)
    case.topk_ids = torch.from_numpy(case.ids_host).to(device)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, cfg.x_dtype, cfg.w_dtype, bm)
    assert moe.moe_pick_block_m(p) == bm
    fp8 = cfg.w_dtype == "e4m3"
    N, rows, mt = cfg.T * cfg.top_k, moe.moe_max_padded_slots(p), moe.moe_max_tiles(p)
    i32, f32 = torch.int32, torch.float32
    dt = case.x.dtype
    say(f"canary {label} {p}")

    g = {"counts": Guarded((cfg.E,), i32, device), "offsets": Guarded((cfg.E + 1,), i32, device),
         "sorted_slots": Guarded((rows,), i32, device), "slot_row": Guarded((N,), i32, device),
         "tiles": Guarded((2 * mt,), i32, device), "num_tiles": Guarded((1,), i32, device),
         "n_invalid": Guarded((1,), i32, device)}
    if fp8:
        g["act"] = Guarded((rows, cfg.I), torch.uint8, device, fill=0x7F)       # e4m3 NaN
        g["act_scales"] = Guarded((rows, cfg.I // 128), f32, device, fill=float("nan"))
        g["xq"] = Guarded((cfg.T, cfg.H), torch.uint8, device, fill=0x7F)
        g["x_scales"] = Guarded((cfg.T, cfg.H // 128), f32, device, fill=float("nan"))
    else:
        g["act"] = Guarded((rows, cfg.I), dt, device, fill=float("nan"))
    g["slot_out"] = Guarded((N, cfg.H), dt, device, fill=float("nan"))
    g["out"] = Guarded((cfg.T, cfg.H), dt, device, fill=float("nan"))
    wsb = moe.moe_gemm_workspace_bytes(p)
    if wsb > 0:
        g["gemm_ws"] = Guarded((wsb,), torch.uint8, device)
    torch.cuda.synchronize()
    snapshot_all(g.values())

    t = {k: v.t for k, v in g.items()}
    moe.moe_align(p, case.topk_ids, t["counts"], t["offsets"], t["sorted_slots"], t["slot_row"],
                  t["tiles"], t["num_tiles"], t["n_invalid"])
    x_in, x_sc = case.x, None
    if fp8:
        moe.moe_quantize_rows_e4m3(p, case.x, t["xq"], t["x_scales"])
        x_in, x_sc = t["xq"], t["x_scales"]
    ws = t.get("gemm_ws")
    moe.moe_grouped_gemm_up(p, x_in, x_sc, case.w13, case.w13_scales, t["sorted_slots"],
                            t["offsets"], t["tiles"], t["num_tiles"], t["act"], t.get("act_scales"), ws)
    moe.moe_grouped_gemm_down(p, t["act"], t.get("act_scales"), case.w2, case.w2_scales,
                              case.topk_weights, t["sorted_slots"], t["offsets"], t["tiles"],
                              t["num_tiles"], t["slot_out"], ws)
    moe.moe_combine(p, t["slot_out"], t["slot_row"], t["out"])
    torch.cuda.synchronize()

    assert_guards(g)
    o = oracle.align(case.ids_host, cfg.E, bm)
    assert np.array_equal(t["sorted_slots"].cpu().numpy(), o.sorted_slots)
    assert int(t["n_invalid"].item()) == o.n_invalid > 0
    used = int(o.offsets[-1])
    act_row = cfg.I * (1 if fp8 else g["act"].elt)
    assert g["act"].untouched(used * act_row, rows * act_row), "act rows past the last tile written"
    assert not torch.isnan(t["act"][:used].float() if not fp8 else
                           t["act"][:used].view(torch.float8_e4m3fn).float()).any()
    if fp8:
        sc_row = 4 * (cfg.I // 128)
        assert g["act_scales"].untouched(used * sc_row, rows * sc_row)
    # slot rows of excluded slots are not written; every other slot row is
    so_row = cfg.H * g["slot_out"].elt
    excl = np.nonzero(case.ids_host.reshape(-1) >= cfg.E)[0]
    for s in excl:
        assert g["slot_out"].untouched(int(s) * so_row, (int(s) + 1) * so_row), f"slot {s} written"
    keep = np.setdiff1d(np.arange(N), excl)
    assert not torch.isnan(t["slot_out"][torch.from_numpy(keep).to(device)].float()).any()
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, case.expert_host, cfg.E,
                           fp8=fp8)
    err = rel_err(t["out"].float().cpu().numpy(), ref)
    say(f"  guards intact; layer rel err {err:.3e}")
    assert err <= TOL[cfg.w_dtype if fp8 else cfg.x_dtype]


@pytest.mark.parametrize("label", ["ksplit_bm256", "ragged_up_bm256", "fp8_bm128", "f32_bm16"])
def test_forward_workspace_and_out_in_bounds(device, label):
    base, kw, bm = CASES[label]
    cfg = get_config(base, **kw)
    case = make_case(cfg, device, seed=4)
    case.ids_host = excluded_ids(cfg, seed=12)
    case.topk_ids = torch.from_numpy(case.ids_host).to(device)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, cfg.x_dtype, cfg.w_dtype, bm)
    say(f"canary forward {label} {p}")
    wsb = moe.moe_workspace_bytes(p)
    ws = Guarded((wsb,), torch.uint8, device)
    out = Guarded((cfg.T, cfg.H), case.x.dtype, device, fill=float("nan"))
    torch.cuda.synchronize()
    ws.snapshot()
    out.snapshot()
    moe.forward(p, case.x, case.topk_ids, case.topk_weights, case.w13, case.w2, case.w13_scales,
                case.w2_scales, out=out.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert ws.guards_intact(), "moe_forward wrote past its workspace"
    assert out.guards_intact(), "moe_forward wrote outside out"
    assert int(ws.t[:4].view(torch.int32).item()) == int((case.ids_host >= cfg.E).sum())
    ref = oracle.moe_layer(case.x_host(), case.ids_host, case.w_host, case.expert_host, cfg.E,
                           fp8=cfg.w_dtype == "e4m3")
    err = rel_err(out.t.float().cpu().numpy(), ref)
    say(f"  guards intact; layer rel err {err:.3e}")
    assert err <= TOL[cfg.w_dtype if cfg.w_dtype == "e4m3" else cfg.x_dtype]


@pytest.mark.parametrize("bm", [16, 64, 128])
def test_mxfp4_act_rows_in_bounds(device, bm):
    """MXFP4 up projection: padding rows and rows past the last valid tile keep their bytes."""
    cfg = get_config("gptoss_shard_mxfp4", T=160, H=192, I=320, E=6, top_k=2, route_experts=0,
                     prod_like=False)
    case = make_mx_case(cfg, device, seed=3)
    p = moe.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, "e4m3", "mxfp4", bm)
    say(f"canary mxfp4 {p}")
    a = moe.align(p, case.topk_ids)
    rows = moe.moe_max_padded_slots(p)
    act = Guarded((rows, cfg.I), torch.uint8, device, fill=0x7F)
    torch.cuda.synchronize()
    act.snapshot()
    moe.moe_grouped_gemm_up_mxfp4(p, case.x_codes, case.x_scale, case.w13, case.w13_scales,
                                  case.bias, case.alpha, case.limit, case.out_scale,
                                  a["sorted_slots"], a["offsets"], a["tiles"], a["num_tiles"], act.t)
    torch.cuda.synchronize()
    assert act.guards_intact()
    ss = a["sorted_slots"].cpu().numpy()
    N = cfg.T * cfg.top_k
    for r in np.nonzero(ss >= N)[0]:                 # padding rows and the unused tail
        assert act.untouched(int(r) * cfg.I, (int(r) + 1) * cfg.I), f"row {r} written"
    valid = np.nonzero(ss < N)[0]
    assert not (act.t.cpu().numpy()[valid] == 0x7F).all(axis=1).any(), "a valid row not written"


def test_route_and_combine_in_bounds(device):
    rng = np.random.default_rng(5)
    T, E, k, H = 300, 64, 6, 256
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(device)
    p = moe.make_problem(T, H, 128, E, k, "bf16")
    N, rows, mt = T * k, moe.moe_max_padded_slots(p), moe.moe_max_tiles(p)
    i32 = torch.int32
    g = {"ids": Guarded((T, k), i32, device), "w": Guarded((T, k), torch.float32, device),
         "counts": Guarded((E,), i32, device), "offsets": Guarded((E + 1,), i32, device),
         "sorted_slots": Guarded((rows,), i32, device), "slot_row": Guarded((N,), i32, device),
         "tiles": Guarded((2 * mt,), i32, device), "num_tiles": Guarded((1,), i32, device),
         "n_invalid": Guarded((1,), i32, device), "out": Guarded((T, H), torch.bfloat16, device)}
    t = {n: v.t for n, v in g.items()}
    moe.moe_route_align(p, lg, True, t["ids"], t["w"], t["counts"], t["offsets"], t["sorted_slots"],
                        t["slot_row"], t["tiles"], t["num_tiles"], t["n_invalid"])
    slot_out = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(torch.bfloat16).to(device)
    moe.moe_combine(p, slot_out, t["slot_row"], t["out"])
    torch.cuda.synchronize()
    assert_guards(g)
    o = oracle.align(t["ids"].cpu().numpy(), E, moe.moe_pick_block_m(p))
    assert np.array_equal(t["sorted_slots"].cpu().numpy(), o.sorted_slots)
    ref = oracle.bf16_round(oracle.combine(slot_out.float().cpu().numpy(), k, np.float32))
    assert np.array_equal(t["out"].float().cpu().numpy(), ref)
