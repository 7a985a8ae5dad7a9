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
