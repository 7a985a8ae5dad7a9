"""The five workload shapes of the MoE expert layer.

Shapes follow the layer definition  out[t] = sum_j w[t,j] * W2[e] (SiLU(W13g[e] x_t) * W13u[e] x_t),
e = ids[t,j], with X[T,H], W13[E,2I,H] (rows [0,I) gate, [I,2I) up) and W2[E,H,I]
("factor_moe_fused_gemm.cu", header comment with the slow PyTorch path).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # experts
    top_k: int
    w_dtype: str      # "f32" | "bf16" | "e4m3" | "mxfp4"  (expert weights)
    x_dtype: str      # "f32" | "bf16" | "e4m3" (mxfp4 only: the gathered activations)
    renormalize: bool  # routing weights renormalised to sum 1 over the chosen experts
    logit_bias_std: float = 0.0  # per-expert router bias ~ N(0, std), skews expert loads
    route_experts: int = 0  # ids are drawn over this many experts (0: E); ids >= E belong to
                            # other expert-parallel shards and are excluded by this one
    prod_like: bool = False  # production-like skew: Zipf expert popularity, token clusters with
                             # preferred experts, batch-hot experts and Gumbel noise (below)
    weight_std: float = 0.02
    block: int = 128   # fp8: weight block edge and activation group width
    description: str = ""

    @property
    def n_slots(self) -> int:
        return self.T * self.top_k

    @property
    def useful_flops_up(self) -> int:
        """Up projection alone: 2 * N * H * 2I = 4*T*k*H*I (padding rows excluded)."""
        return 4 * self.T * self.top_k * self.H * self.I

    @property
    def useful_flops_layer(self) -> int:
        """Both projections: 6*T*k*H*I."""
        return 6 * self.T * self.top_k * self.H * self.I


CONFIGS = {
    c.name: c
    for c in [
        MoEConfig("tiny_fp32", T=16, H=128, I=256, E=8, top_k=2, w_dtype="f32", x_dtype="f32",
                  renormalize=True,
                  description="tiny fp32 layer, top-2 renormalised"),
        MoEConfig("mixtral_prefill_bf16", T=4096, H=4096, I=14336, E=8, top_k=2, w_dtype="bf16",
                  x_dtype="bf16", renormalize=True,
                  description="Mixtral-8x7B-shaped prefill, bf16, top-2 renormalised"),
        MoEConfig("dsv3_decode_bf16", T=64, H=7168, I=2048, E=256, top_k=8, w_dtype="bf16",
                  x_dtype="bf16", renormalize=False,
                  description="DeepSeek-V3-shaped decode batch, bf16, top-8"),
        MoEConfig("skewed_prefill_bf16", T=8192, H=2048, I=1408, E=64, top_k=6, w_dtype="bf16",
                  x_dtype="bf16", renormalize=False, logit_bias_std=2.0,
                  description="skewed-routing prefill, bf16, top-6, router bias ~N(0,2)"),
        MoEConfig("dsv3_fp8_e4m3", T=2048, H=7168, I=2048, E=256, top_k=8, w_dtype="e4m3",
                  x_dtype="bf16", renormalize=False,
                  description="fp8 e4m3 weights with 128x128 fp32 block scales, bf16 X "
                              "quantised per token row in 128-wide groups, top-8"),
    ]
}

# Production-like routing ("MOE Bmm1 Fused Gather", the bench's prod-like logits): expert
# popularity p_e proportional to rank^-1.10 with the ranks in a random order; logits start at
# log p_e; 16 token clusters, each preferring a popularity-weighted sample (without replacement)
# of max(2k, E_r/16) experts (at most E_r), whose logits gain 1.25 for the cluster's tokens; 4
# popularity-weighted batch-hot experts gain 0.6; then 0.75 * Gumbel(0,1) noise per logit.
PROD_ZIPF_ALPHA = 1.10
PROD_CLUSTERS = 16
PROD_CLUSTER_BOOST = 1.25
PROD_HOT_EXPERTS = 4
PROD_HOT_BOOST = 0.6
PROD_GUMBEL_SCALE = 0.75


def sweep_batch_sizes(route_experts: int, top_k: int) -> list:
    """The batch sweep of the same bench: 48 tokens-per-expert levels -- 4..7 by 1, 8..14 by 2,
    16..28 by 4, 32..56 by 8, 64..112 by 16, then by 32 up to 992 -- each times E_r/k tokens."""
    per_expert = []
    for k in range(8):
        per_expert += list(range(2 ** (2 + k), 2 ** (3 + k), min(2 ** k, 32)))
    return [b * route_experts // top_k for b in per_expert]


# Batch-sweep workloads: T is the largest batch of the sweep; a sweep point of T' tokens uses
# the first T' rows of X (the routing of each point is drawn for its own T').
SWEEP_CONFIGS = {
    c.name: c
    for c in [
        MoEConfig("gptoss_shard_bf16", T=31744, H=2880, I=2880, E=16, top_k=4, w_dtype="bf16",
                  x_dtype="bf16", renormalize=True, route_experts=128, prod_like=True,
                  description="one expert-parallel shard (16 of 128 experts) of a GPT-OSS-120B-"
                              "shaped MoE layer, bf16, top-4 of 128, production-like skew"),
        MoEConfig("gptoss_shard_mxfp4", T=31744, H=2880, I=2880, E=16, top_k=4, w_dtype="mxfp4",
                  x_dtype="e4m3", renormalize=True, route_experts=128, prod_like=True,
                  description="the same shard's first expert GEMM as the page runs it: MXFP4 "
                              "weights x e4m3 activations, bias, GPT-OSS SwiGLU, e4m3 output"),
        MoEConfig("gptoss_shard_uniform_mxfp4", T=31744, H=2880, I=2880, E=16, top_k=4,
                  w_dtype="mxfp4", x_dtype="e4m3", renormalize=True, route_experts=128,
                  description="the MXFP4 first expert GEMM of the shard with logits ~N(0,1) "
                              "(the bench's uniform routing)"),
        MoEConfig("gptoss_shard_uniform_bf16", T=31744, H=2880, I=2880, E=16, top_k=4,
                  w_dtype="bf16", x_dtype="bf16", renormalize=True, route_experts=128,
                  description="the same shard with logits ~N(0,1) (the bench's uniform routing)"),
    ]
}

# Order of the workloads as they are listed (the small fp32 case first).
CONFIG_ORDER = ["tiny_fp32", "mixtral_prefill_bf16", "dsv3_decode_bf16",
                "skewed_prefill_bf16", "dsv3_fp8_e4m3"]


def get_config(name: str, **overrides) -> MoEConfig:
    """Look up a workload by name; keyword overrides give a shrunk variant of it."""
    from dataclasses import replace
    base = CONFIGS[name] if name in CONFIGS else SWEEP_CONFIGS[name]
    return replace(base, **overrides) if overrides else base
