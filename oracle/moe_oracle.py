"""Plain CPU definition of the routed grouped-GEMM top-k MoE expert layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, smoke() and the
benchmark's cpu_baseline leg use it; the product path never does.

Sources (page titles as published):
  [slow-path]  "factor_moe_fused_gemm.cu", header comment: the current slow
               PyTorch path -- per active expert, gather the expert's tokens,
               gate_up = linear(tokens, w13[e]) split in two halves with the gate
               first, act = silu(gate) * up, expert_out = linear(act, w2[e]),
               out.index_add_(tok_ids, expert_out * weights).
  [silu-kernel] same page, fused_silu_gate_kernel: gate is the first half of
               the 2I columns, up the second; SiLU(g) = g / (1 + exp(-g)).
  [scatter]    same page, weighted_scatter_add_kernel: each routed row is scaled
               by its routing weight and added into its token's output row.
  [ragged]     "MOE Bmm1 Fused Gather", init_routing_data / load_activations:
               the gather index of an expert-sorted slot is slot // top_k, and
               rows past a slice's end are masked to an out-of-range row
               (zero).  make_ragged_tensor_metadata: per-expert slice sizes,
               offsets and a block schedule of (slice, m-block) pairs.
  [m-blocks]   "moe triton kernel use tma." (review summary): the align kernel
               records, per M block, the expert id and the block's first token
               row; the down projection multiplies by the routed weight
               (MUL_ROUTED_WEIGHT).
  [satfinite]  "MOE Bmm1 Fused Gather", pack_e4m3x2: fp32 -> e4m3 conversion
               rounds to nearest even and saturates to the largest finite value.

Readings where the pages are silent (restated in the tests that pin them):
  * slot s = t*top_k + j (row-major over ids[T,k]);
  * within an expert, slots are kept in ascending s (a stable counting sort);
  * each expert's segment is padded to a multiple of block_m with the
    sentinel N = T*top_k; experts with no slots get no rows and no tiles;
  * tiles are (expert, first row) pairs, expert-major then m-block; unused
    entries of the tile table are (-1, -1);
  * ids outside [0, E) are excluded from every expert and counted;
  * fp8: X and the intermediate activation are quantised per (row, 128-column
    group): s = amax/448 in fp32 (s = 1 when amax = 0), q = e4m3(x/s) with an
    fp32 quotient; dequantised value = q*s.  Weights arrive as e4m3 codes with
    one fp32 scale per 128x128 block;
  * the combine sums a token's k slot outputs in ascending j.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------------------------
# Codecs
# --------------------------------------------------------------------------------------------
def _e4m3_value(codes) -> np.ndarray:
    """OCP FP8 E4M3 ("fn" variant) value of each code, as float64.

    Bit layout s.eeee.mmm, exponent bias 7; exponent 0 holds subnormals
    m/8 * 2^-6; S.1111.111 is NaN and there is no infinity.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7.0)
    sub = (man / 8.0) * 2.0 ** -6
    mag = np.where(ex == 0, sub, normal)
    mag = np.where((ex == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


_E4M3_TABLE = _e4m3_value(np.arange(256))


def e4m3_decode(codes) -> np.ndarray:
    """Decode e4m3 codes (any integer array) to float64 by the table of all 256 values."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


# The 127 non-negative finite magnitudes, ascending; their index is the code.
_E4M3_POS = _E4M3_TABLE[:127]


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code, saturating to
    +-448 ([satfinite]).  The sign bit is the input's sign bit (so -0.0 and
    negative values that round to zero give 0x80).  NaN inputs are not used."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo))
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as
    float32.  bfloat16 keeps the top 16 bits of the binary32 pattern.  Finite
    inputs only."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def quantize_groups_e4m3(x, group: int = 128):
    """Per (row, group of `group` columns): s = amax/448 in fp32 (1 if amax = 0),
    codes = e4m3(x / s) with the quotient formed in fp32.  x: float32 [R, C],
    C a multiple of `group`.  Returns (codes uint8 [R,C], scales float32 [R, C/group])."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    xg = x.reshape(R, C // group, group)
    amax = np.abs(xg).max(axis=2)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    quotient = (xg / s[:, :, None]).astype(np.float32)
    codes = e4m3_encode(quotient).reshape(R, C)
    return codes, s


def dequantize_groups(codes, scales, group: int = 128) -> np.ndarray:
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R, C // group, group)
    return (v * np.asarray(scales, np.float64)[:, :, None]).reshape(R, C)


def dequantize_blocks(codes, scales, block: int = 128) -> np.ndarray:
    """Weight dequantisation: codes [R, C] e4m3, one scale per block x block tile."""
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R // block, block, C // block, block)
    s = np.asarray(scales, np.float64)
    return (v * s[:, None, :, None]).reshape(R, C)


# --------------------------------------------------------------------------------------------
# Routing (the step that produces the layer's ids and weights)
# --------------------------------------------------------------------------------------------
def route(logits, top_k: int, renormalize: bool):
    """Router producer: logits [T, E] -> (ids int32 [T, top_k], weights float64 [T, top_k]).

    [topk-softmax] "MOE Bmm1 Fused Gather" (bench setup: topk(logits, experts_per_token,
    apply_softmax=True), then the expert histogram col_sum) and "factor_moe_fused_gemm.cu"
    ("factor 0", topk_softmax, which yields topk_weights and topk_ids).  The pages fix neither
    the order of softmax and selection nor ties; reading: the softmax over all E logits, the
    top_k experts in descending probability with ties to the lower expert id, their
    probabilities as weights, renormalised to sum 1 when asked (the same as a softmax over
    the selected logits).  Softmax is strictly increasing in the logit, so the selection is
    made on the logits themselves.
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    for t in range(T):
        row = lg[t]
        # descending logit; among equal logits the lower id first
        order = sorted(range(E), key=lambda e: (-row[e], e))[:top_k]
        z = np.exp(row - row.max())
        p = z / z.sum()
        sel = np.array([p[e] for e in order])
        if renormalize:
            sel = sel / sel.sum()
        ids[t] = order
        w[t] = sel
    return ids, w


def expert_histogram(topk_ids, num_experts: int) -> np.ndarray:
    """Slots routed to each expert ("MOE Bmm1 Fused Gather": col_sum of the top-k mask)."""
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in np.asarray(topk_ids).reshape(-1):
        if 0 <= e < num_experts:
            counts[e] += 1
    return counts


# --------------------------------------------------------------------------------------------
# Alignment
# --------------------------------------------------------------------------------------------
def max_padded_slots(n_slots: int, num_experts: int, block_m: int) -> int:
    """Rows the padded, expert-sorted slot list can need: each of at most
    min(E, N) non-empty experts adds at most block_m - 1 padding rows."""
    return n_slots + min(num_experts, n_slots) * (block_m - 1)


def max_tiles(n_slots: int, num_experts: int, block_m: int) -> int:
    return max_padded_slots(n_slots, num_experts, block_m) // block_m


@dataclass
class Alignment:
    counts: np.ndarray        # [E] int32
    offsets: np.ndarray       # [E+1] int32
    sorted_slots: np.ndarray  # [max_padded_slots] int32, sentinel N
    slot_row: np.ndarray      # [N] int32, -1 for excluded slots
    tiles: np.ndarray         # [max_tiles, 2] int32 (expert, first row); (-1,-1) unused
    num_tiles: int
    n_invalid: int


def align(topk_ids, num_experts: int, block_m: int) -> Alignment:
    """Sort routed slots by expert ([ragged], [m-blocks]).

    counts[e]   = number of slots s with ids[s] == e
    offsets     = exclusive prefix sum of counts rounded up to block_m
    sorted_slots[offsets[e] + i] = i-th smallest slot of expert e; padding and
                  the unused tail hold the sentinel N
    slot_row[s] = row of slot s in sorted_slots
    tiles       = (e, offsets[e] + b*block_m) for every m-block b of every expert
    """
    ids = np.asarray(topk_ids).reshape(-1)
    N = int(ids.size)
    E = int(num_experts)
    BM = int(block_m)

    counts = [0] * E
    n_invalid = 0
    for s in range(N):
        e = int(ids[s])
        if 0 <= e < E:
            counts[e] += 1
        else:
            n_invalid += 1

    offsets = [0] * (E + 1)
    for e in range(E):
        padded = -(-counts[e] // BM) * BM
        offsets[e + 1] = offsets[e] + padded

    rows = max_padded_slots(N, E, BM)
    sorted_slots = [N] * rows
    slot_row = [-1] * N
    cursor = list(offsets[:E])
    for s in range(N):                         # ascending s keeps each expert's slots sorted
        e = int(ids[s])
        if 0 <= e < E:
            sorted_slots[cursor[e]] = s
            slot_row[s] = cursor[e]
            cursor[e] += 1

    mt = max_tiles(N, E, BM)
    tiles = [(-1, -1)] * mt
    n = 0
    for e in range(E):
        for b in range((offsets[e + 1] - offsets[e]) // BM):
            tiles[n] = (e, offsets[e] + b * BM)
            n += 1

    return Alignment(
        counts=np.array(counts, dtype=np.int32),
        offsets=np.array(offsets, dtype=np.int32),
        sorted_slots=np.array(sorted_slots, dtype=np.int32),
        slot_row=np.array(slot_row, dtype=np.int32),
        tiles=np.array(tiles, dtype=np.int32).reshape(mt, 2),
        num_tiles=n,
        n_invalid=n_invalid,
    )


# --------------------------------------------------------------------------------------------
# Expert MLP pieces
# --------------------------------------------------------------------------------------------
def silu(g) -> np.ndarray:
    """SiLU(g) = g / (1 + exp(-g))  ([silu-kernel]).  For g -> -inf the quotient is -0."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_up(x_rows, w13_e) -> np.ndarray:
    """act = SiLU(gate) * up with [gate; up] = w13_e @ x  ([slow-path], [silu-kernel]).
    x_rows [n, H], w13_e [2I, H] (rows [0,I) gate, [I,2I) up) -> act [n, I]."""
    x_rows = np.asarray(x_rows, np.float64)
    w13_e = np.asarray(w13_e, np.float64)
    I = w13_e.shape[0] // 2
    gate = x_rows @ w13_e[:I].T
    up = x_rows @ w13_e[I:].T
    return silu(gate) * up


def expert_down(act, w2_e) -> np.ndarray:
    """expert_out = act @ w2_e^T, w2_e [H, I]  ([slow-path])."""
    return np.asarray(act, np.float64) @ np.asarray(w2_e, np.float64).T


def combine(slot_out, top_k: int, acc_dtype=np.float64) -> np.ndarray:
    """out[t] = sum over j = 0..k-1, in that order, of slot_out[t*k + j]
    ([scatter]; every slot of token t lands on row t).  The sum is carried in
    `acc_dtype`, adding one slot at a time."""
    y = np.asarray(slot_out)
    N, H = y.shape
    T = N // top_k
    acc = np.zeros((T, H), dtype=acc_dtype)
    for j in range(top_k):
        acc = (acc + y[j::top_k].astype(acc_dtype)).astype(acc_dtype)
    return acc


# --------------------------------------------------------------------------------------------
# The layer
# --------------------------------------------------------------------------------------------
ExpertGetter = Callable[[int], tuple]


def moe_layer(x, topk_ids, topk_weights, experts, num_experts: Optional[int] = None, *,
              fp8: bool = False, group: int = 128, tokens: Optional[Sequence[int]] = None,
              return_slots: bool = False, workers: int = 1):
    """out[t] = sum_j w[t,j] * W2[e] (SiLU(W13g[e] x_t) * W13u[e] x_t), e = ids[t,j].

    Per active expert: gather the expert's slots' token rows (token = slot // k),
    run the two projections in float64, scale each slot's row by its routing
    weight, then combine each token's k slots ([slow-path], [scatter]).

    x: [T, H] float values.  topk_ids, topk_weights: [T, k].
    experts: either (w13 [E,2I,H], w2 [E,H,I]) float arrays, a 4-tuple
      (w13 codes, w2 codes, s13 [E,2I/b,H/b], s2 [E,H/b,I/b]) when fp8, or a
      callable e -> (w13_e, w2_e, s13_e, s2_e) that fetches one expert.
    fp8: X and the intermediate activation go through per-(row, group)
      e4m3 quantisation (see module docstring); weights are dequantised codes.
    tokens: compute only these token rows (the returned rows follow this order).
    workers: experts are independent of each other, so with workers > 1 they are
      evaluated by that many threads at once; each expert's arithmetic and the
      combine order are the same, so the result is identical bit for bit.
    Returns out [len(tokens), H] float64 (and the per-slot rows if asked).
    """
    x = np.asarray(x)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float64)
    T, H = x.shape
    k = ids.shape[1]
    if callable(experts):
        get = experts
        E = int(num_experts)
    else:
        arrs = experts
        E = int(arrs[0].shape[0]) if num_experts is None else int(num_experts)

        def get(e):
            return tuple(a[e] if a is not None else None for a in arrs) + (None,) * (4 - len(arrs))

    if fp8:
        xq, sx = quantize_groups_e4m3(x.astype(np.float32), group)
        x_in = dequantize_groups(xq, sx, group)
    else:
        x_in = x.astype(np.float64)

    toks = list(range(T)) if tokens is None else [int(t) for t in tokens]
    slots = [t * k + j for t in toks for j in range(k)]
    def one_expert(e):
        """Rows w[s] * W2[e] act(x_{s//k}) of expert e's slots s (ascending s)."""
        mine = [s for s in slots if int(ids.flat[s]) == e]
        if not mine:
            return {}
        w13_e, w2_e, s13_e, s2_e = get(e)
        if fp8:
            w13_e = dequantize_blocks(w13_e, s13_e, group)
            w2_e = dequantize_blocks(w2_e, s2_e, group)
        rows = x_in[[s // k for s in mine]]
        act = expert_up(rows, w13_e)
        if fp8:
            aq, sa = quantize_groups_e4m3(act.astype(np.float32), group)
            act = dequantize_groups(aq, sa, group)
        y = expert_down(act, w2_e)
        return {s: wts.flat[s] * y[i] for i, s in enumerate(mine)}

    slot_vals = {}
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=int(workers)) as ex:
            for part in ex.map(one_expert, range(E)):
                slot_vals.update(part)
    else:
        for e in range(E):
            slot_vals.update(one_expert(e))

    zero = np.zeros(H, dtype=np.float64)
    slot_rows = np.stack([slot_vals.get(s, zero) for s in slots]) if slots else np.zeros((0, H))
    out = combine(slot_rows, k, np.float64)
    if return_slots:
        return out, slot_rows
    return out
