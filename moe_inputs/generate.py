"""Seeded generator for the MoE expert layer's inputs.

Recipe (one source of truth for the oracle tests, the GPU parity tests and the
benchmark):

* Every tensor slab has its own seed ``slab_seed(seed, tag, e)`` derived with
  numpy's SeedSequence from (seed, tag, expert), tag in {X:1, W13:2, W2:3,
  logits:4, bias:5, token clusters:6}.  Slabs can therefore be regenerated one expert at a time.
* Routing is made on the host in float64 with numpy: logits[T,E] ~ N(0,1),
  plus a per-expert bias ~ N(0, logit_bias_std) for the skewed workload, or
  for the expert-parallel shard the production-like logits over all E_r
  experts (recipe in configs.py; Gumbel noise is -log(-log U));
  softmax; the top-k experts in descending probability (ties to the lower
  expert id, so the k experts of a token are distinct); routing weights are the
  chosen probabilities, renormalised to sum 1 only where the workload says so;
  stored as fp32.  The id tensor is int32 [T,k], weights fp32 [T,k].
* X[T,H] ~ N(0,1) is drawn on the host with numpy (float32) and then rounded
  to the workload's activation dtype (bf16 round-to-nearest-even by torch's
  cast, or kept fp32).
* Expert weights ~ N(0, weight_std) are drawn per expert with a seeded torch
  generator on the target device (float32), then rounded to bf16, kept fp32,
  or -- for the fp8 workload -- quantised per 128x128 block:
  s = amax(|block|)/448 (s = 1 for an all-zero block), q = e4m3(w/s) with the
  quotient clamped to +-448 before torch's round-to-nearest-even cast to
  float8_e4m3fn.  The layer receives q and s; its dequantised weight is q*s.

Routing statistics therefore do not depend on the device; weight values do
(torch's CPU and GPU generators differ), so a comparison always uses copies of
the one generated case.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import configs as _c
from .configs import MoEConfig

TAG_X, TAG_W13, TAG_W2, TAG_LOGITS, TAG_BIAS, TAG_CLUSTER = 1, 2, 3, 4, 5, 6
E4M3_MAX = 448.0


def slab_seed(seed: int, tag: int, e: int = 0) -> int:
    """63-bit seed of one tensor slab, from (seed, tag, expert)."""
    st = np.random.SeedSequence([int(seed), int(tag), int(e)]).generate_state(1, dtype=np.uint64)
    return int(st[0] & np.uint64((1 << 63) - 1))


def _rng(seed: int, tag: int, e: int = 0) -> np.random.Generator:
    return np.random.default_rng(slab_seed(seed, tag, e))


def _prod_like_logits(cfg: MoEConfig, seed: int, er: int) -> np.ndarray:
    """Production-like logits [T, er]: expert-level draws (popularity order, clusters, hot
    experts) come from one stream, per-token draws from two others, so the first T' rows do not
    depend on T."""
    g = _rng(seed, TAG_BIAS)
    ranked = np.arange(1, er + 1, dtype=np.float64) ** -_c.PROD_ZIPF_ALPHA
    ranked /= ranked.sum()
    prob = np.empty(er)
    prob[g.permutation(er)] = ranked
    size = min(er, max(2 * cfg.top_k, er // 16))
    clusters = np.stack([g.choice(er, size, replace=False, p=prob)
                         for _ in range(_c.PROD_CLUSTERS)])
    hot = g.choice(er, _c.PROD_HOT_EXPERTS, replace=False, p=prob)
    logits = np.repeat(np.log(np.maximum(prob, 1e-12))[None, :], cfg.T, axis=0)
    tok_cluster = _rng(seed, TAG_CLUSTER).integers(0, _c.PROD_CLUSTERS, cfg.T)
    logits[np.arange(cfg.T)[:, None], clusters[tok_cluster]] += _c.PROD_CLUSTER_BOOST
    logits[:, hot] += _c.PROD_HOT_BOOST
    u = _rng(seed, TAG_LOGITS).random((cfg.T, er))
    logits += _c.PROD_GUMBEL_SCALE * -np.log(-np.log(np.clip(u, 1e-300, None)))
    return logits


def make_logits(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Router logits [T, E_r] (float64), E_r = cfg.route_experts or E: N(0,1), plus the per-expert
    bias of the skewed workload; or the production-like logits."""
    er = cfg.route_experts or cfg.E
    if cfg.prod_like:
        return _prod_like_logits(cfg, seed, er)
    logits = _rng(seed, TAG_LOGITS).standard_normal((cfg.T, er))
    if cfg.logit_bias_std:
        logits = logits + cfg.logit_bias_std * _rng(seed, TAG_BIAS).standard_normal(er)[None, :]
    return logits


def make_routing(cfg: MoEConfig, seed: int = 0):
    """Router output on the host: (ids int32 [T,k], w float32 [T,k], probs float64 [T,E])."""
    logits = make_logits(cfg, seed)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, : cfg.top_k]
    w = np.take_along_axis(p, order, axis=1)
    if cfg.renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32), p


def routing_stats(ids: np.ndarray, E: int) -> dict:
    counts = np.bincount(ids.reshape(-1), minlength=E)[:E]
    return {
        "n_slots": int(ids.size),
        "active_experts": int((counts > 0).sum()),
        "empty_experts": int((counts == 0).sum()),
        "max_per_expert": int(counts.max()),
        "min_per_expert": int(counts.min()),
        "median_per_expert": float(np.median(counts)),
        "mean_per_expert": float(counts.mean()),
    }


def make_x(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """X [T, H] on the host (float32, before rounding to the activation dtype); the first T'
    rows do not depend on T."""
    return _rng(seed, TAG_X).standard_normal((cfg.T, cfg.H), dtype=np.float32)


def _block_quant_e4m3(w: torch.Tensor, block: int):
    """Input preparation for the fp8 workload: 128x128 block scales + e4m3 codes."""
    R, C = w.shape
    blocks = w.reshape(R // block, block, C // block, block)
    amax = blocks.abs().amax(dim=(1, 3))
    s = torch.where(amax == 0, torch.ones_like(amax), amax / E4M3_MAX)
    q = (blocks / s[:, None, :, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.reshape(R, C), s


def _weights(cfg: MoEConfig, tag: int, shape, device, seed: int, experts=None):
    E = cfg.E
    if cfg.w_dtype == "e4m3":
        store = torch.float8_e4m3fn
    elif cfg.w_dtype == "bf16":
        store = torch.bfloat16
    else:
        store = torch.float32
    out = torch.empty((E,) + tuple(shape), dtype=store, device=device)
    scales = None
    if cfg.w_dtype == "e4m3":
        b = cfg.block
        scales = torch.empty((E, shape[0] // b, shape[1] // b), dtype=torch.float32, device=device)
    todo = range(E) if experts is None else experts
    for e in todo:
        g = torch.Generator(device=device)
        g.manual_seed(slab_seed(seed, tag, e))
        w = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
        w.mul_(cfg.weight_std)
        if cfg.w_dtype == "e4m3":
            q, s = _block_quant_e4m3(w, cfg.block)
            out[e].copy_(q)
            scales[e].copy_(s)
        else:
            out[e].copy_(w.to(store))
        del w
    return out, scales


@dataclass
class MoECase:
    """One generated problem: tensors live on ``device``; routing also kept on the host."""
    cfg: MoEConfig
    seed: int
    x: torch.Tensor                 # [T,H] f32 or bf16
    topk_ids: torch.Tensor          # [T,k] int32
    topk_weights: torch.Tensor      # [T,k] f32
    w13: torch.Tensor               # [E,2I,H] f32 / bf16 / float8_e4m3fn
    w2: torch.Tensor                # [E,H,I]
    w13_scales: Optional[torch.Tensor] = None   # [E,2I/128,H/128] f32 (fp8 only)
    w2_scales: Optional[torch.Tensor] = None    # [E,H/128,I/128] f32 (fp8 only)
    ids_host: np.ndarray = field(default=None, repr=False)
    w_host: np.ndarray = field(default=None, repr=False)

    # ---- host copies for the oracle (exact: bf16 and e4m3 widen to f32 exactly) ----
    def x_host(self) -> np.ndarray:
        return self.x.detach().to("cpu", torch.float32).numpy()

    def expert_host(self, e: int):
        """(w13[e], w2[e], s13[e], s2[e]) on the host.  fp8 weights come back as
        their raw uint8 codes, other weights as float32 values."""
        if self.cfg.w_dtype == "e4m3":
            return (self.w13[e].detach().cpu().view(torch.uint8).numpy(),
                    self.w2[e].detach().cpu().view(torch.uint8).numpy(),
                    self.w13_scales[e].detach().cpu().numpy(),
                    self.w2_scales[e].detach().cpu().numpy())
        return (self.w13[e].detach().to("cpu", torch.float32).numpy(),
                self.w2[e].detach().to("cpu", torch.float32).numpy(), None, None)

    def weights_host(self):
        """All experts on the host (small workloads only)."""
        parts = [self.expert_host(e) for e in range(self.cfg.E)]
        w13 = np.stack([p[0] for p in parts])
        w2 = np.stack([p[1] for p in parts])
        if self.cfg.w_dtype == "e4m3":
            return w13, w2, np.stack([p[2] for p in parts]), np.stack([p[3] for p in parts])
        return w13, w2, None, None


def make_case(cfg: MoEConfig, device="cpu", seed: int = 0, experts=None) -> MoECase:
    """Generate one problem on ``device``.  ``experts`` limits weight generation
    to a subset (the rest of the weight tensors is left uninitialised)."""
    device = torch.device(device)
    ids, w, _ = make_routing(cfg, seed)
    xh = make_x(cfg, seed)
    xdt = torch.float32 if cfg.x_dtype == "f32" else torch.bfloat16
    x = torch.from_numpy(xh).to(xdt).to(device)
    w13, s13 = _weights(cfg, TAG_W13, (2 * cfg.I, cfg.H), device, seed, experts)
    w2, s2 = _weights(cfg, TAG_W2, (cfg.H, cfg.I), device, seed, experts)
    return MoECase(cfg=cfg, seed=seed, x=x,
                   topk_ids=torch.from_numpy(ids).to(device),
                   topk_weights=torch.from_numpy(w).to(device),
                   w13=w13, w2=w2, w13_scales=s13, w2_scales=s2,
                   ids_host=ids, w_host=w)


# ---------------------------------------------------------------------------------------------
# MXFP4 weights x e4m3 activations: the first expert GEMM of "MOE Bmm1 Fused Gather" (its
# prepare_case), with the GPT-OSS SwiGLU parameters and per-tensor flex scales.
# ---------------------------------------------------------------------------------------------
TAG_MX_SCALARS, TAG_BIAS13 = 7, 8
E2M1_MAX = 6.0
_E2M1_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)     # codes 0..7 (sign in bit 3)


def mx_quantize(w: torch.Tensor, block: int = 32):
    """Input preparation: float rows [R, K] -> (packed e2m1 [R, K/2] uint8, e8m0 scales
    [R, K/block] uint8) by the OCP MX rule: per block of `block` values along K the shared
    exponent is floor(log2(amax)) - 2 (2 = the largest e2m1 exponent), clamped to [-127, 127]
    (an all-zero block gets -127); each value / 2^exponent is rounded to the nearest e2m1 value,
    ties to the even code, and saturated to +-6.  Element 2i goes to the low nibble of byte i."""
    R, K = w.shape
    b = w.float().reshape(R, K // block, block)
    amax = b.abs().amax(dim=2)
    ex = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                     torch.full_like(amax, -127.0)).clamp(-127, 127)
    q = (b / torch.exp2(ex)[:, :, None]).reshape(R, K)
    a = q.abs().clamp(max=E2M1_MAX)
    mags = torch.tensor(_E2M1_MAGS, device=w.device)
    hi = torch.searchsorted(mags, a.contiguous(), right=False).clamp(max=7)   # first mag >= a
    lo = (hi - 1).clamp(min=0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag_code = torch.where(a == mags[hi], hi, torch.where(pick_hi, hi, lo))
    code = (mag_code | torch.where(torch.signbit(q) & (mag_code > 0), 8, 0)).to(torch.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).to(torch.uint8)
    return packed, (ex + 127).to(torch.uint8)


@dataclass
class MXCase:
    """One MXFP4 problem on ``device``: e4m3 X codes, MXFP4 W13 with interleaved (gate, linear)
    rows, fp32 bias, GPT-OSS SwiGLU parameters, x and output flex scales."""
    cfg: MoEConfig
    seed: int
    x_codes: torch.Tensor           # [T, H] uint8 (e4m3)
    topk_ids: torch.Tensor          # [T, k] int32
    w13: torch.Tensor               # [E, 2I, H/2] uint8: row 2i = gate_i, row 2i+1 = linear_i
    w13_scales: torch.Tensor        # [E, H/32, 2I] uint8 (e8m0)
    bias: torch.Tensor              # [E, 2I] float32, same row order
    x_scale: torch.Tensor           # [1] float32
    out_scale: torch.Tensor         # [1] float32
    alpha: float
    limit: float
    ids_host: np.ndarray = field(default=None, repr=False)

    def x_codes_host(self) -> np.ndarray:
        return self.x_codes.cpu().numpy()

    def expert_host(self, e: int):
        """(packed [2I, H/2], scales [2I, H/32]) of expert e on the host."""
        return (self.w13[e].cpu().numpy(), self.w13_scales[e].cpu().numpy().T.copy())

    def bias_host(self) -> np.ndarray:
        return self.bias.cpu().numpy().astype(np.float64)


def make_mx_case(cfg: MoEConfig, device="cpu", seed: int = 0, ids: Optional[np.ndarray] = None,
                 weight_std: Optional[float] = None) -> MXCase:
    """X ~ N(0,1) rounded to e4m3 (torch's cast); W13 ~ N(0, std) per expert, MX-quantised;
    bias ~ N(0,1); alpha = 1 + u/5, limit = 1.3 + u/5, x_scale = 0.5 + u, out_scale = 3.5 + u
    (u ~ U[0,1), the ranges of the page's prepare_case), each rounded to fp32."""
    device = torch.device(device)
    if ids is None:
        ids, _, _ = make_routing(cfg, seed)
    ids = np.asarray(ids, dtype=np.int32)
    x = torch.from_numpy(make_x(cfg, seed)).to(device)
    x_codes = x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    std = cfg.weight_std if weight_std is None else weight_std
    E, I2, H = cfg.E, 2 * cfg.I, cfg.H
    w13 = torch.empty((E, I2, H // 2), dtype=torch.uint8, device=device)
    sc = torch.empty((E, H // 32, I2), dtype=torch.uint8, device=device)
    for e in range(E):
        g = torch.Generator(device=device)
        g.manual_seed(slab_seed(seed, TAG_W13, e))
        w = torch.randn((I2, H), generator=g, device=device, dtype=torch.float32) * std
        p, s = mx_quantize(w)
        w13[e].copy_(p)
        sc[e].copy_(s.t())
        del w
    bias = torch.from_numpy(_rng(seed, TAG_BIAS13).standard_normal((E, I2)).astype(np.float32)).to(device)
    u = _rng(seed, TAG_MX_SCALARS).random(4)
    alpha, limit = float(np.float32(1.0 + u[0] / 5)), float(np.float32(1.3 + u[1] / 5))
    xs = torch.tensor([0.5 + u[2]], dtype=torch.float32, device=device)
    ys = torch.tensor([3.5 + u[3]], dtype=torch.float32, device=device)
    return MXCase(cfg=cfg, seed=seed, x_codes=x_codes, topk_ids=torch.from_numpy(ids).to(device),
                  w13=w13, w13_scales=sc, bias=bias, x_scale=xs, out_scale=ys, alpha=alpha,
                  limit=limit, ids_host=ids)
