/*
 * moe.h -- C ABI of the MI355X (gfx950) routed grouped-GEMM top-k MoE expert layer.
 *
 * The layer computes, for every token t,
 *     out[t] = sum_{j<top_k} w[t,j] * W2[e] ( SiLU(W13g[e] x_t) * W13u[e] x_t ),  e = ids[t,j]
 * where W13[e] stacks the gate rows [0,I) over the up rows [I,2I)
 * ("factor_moe_fused_gemm.cu", header comment: the slow PyTorch path, and
 * fused_silu_gate_kernel: gate is the first half, SiLU(g) = g / (1 + exp(-g))).
 *
 * It runs as four stages, each an entry point below:
 *   moe_align             expert histogram, padded expert-sorted slot list, tile table
 *   moe_grouped_gemm_up   gathered rows x W13[e]^T with SiLU(gate)*up in the epilogue
 *   moe_grouped_gemm_down act rows x W2[e]^T, scaled by the routing weight in the epilogue
 *   moe_combine           per-token fixed-order sum of the top_k slot rows
 * plus moe_quantize_rows_e4m3 (the fp8 workload's activation quantisation) and
 * moe_forward, which runs the whole chain in a caller-provided workspace.
 *
 * Conventions shared by every entry point
 *   - Pointers named as tensors are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises.  All work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and is asynchronous.
 *   - Tensors are dense row-major with the innermost dimension contiguous.
 *   - A flat slot is s = t*top_k + j (row-major over ids[T,top_k]); N = T*top_k.
 *   - Arguments are validated on the host BEFORE any HIP call; a rejected call
 *     enqueues nothing and returns a negative moe_status.  Launch failures
 *     return MOE_ERR_LAUNCH; faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Reentrant and stateless: calls on different streams may overlap as long
 *     as their output buffers do not.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,       /* a required pointer is NULL                                */
  MOE_ERR_SHAPE = -2,      /* a dimension is out of range or not a supported multiple   */
  MOE_ERR_DTYPE = -3,      /* unsupported dtype or dtype combination                     */
  MOE_ERR_WORKSPACE = -4,  /* workspace smaller than moe_workspace_bytes()               */
  MOE_ERR_LAUNCH = -5,     /* a kernel launch failed (hipGetLastError after the launch)  */
  MOE_ERR_DEVICE = -6,     /* no usable device / not a gfx950 device                    */
  MOE_ERR_ALIGN = -7       /* a device pointer is not aligned as its argument requires  */
} moe_status;

/*
 * Pointer alignment (checked on the host before any launch; MOE_ERR_ALIGN otherwise):
 *   16 bytes: data arrays -- X and its codes, weights, act, slot rows, out, bias;
 *   4 bytes:  int32 and fp32 index, routing-weight, logit and scale arrays;
 *   256 bytes: the workspaces of moe_forward and moe_grouped_gemm_down.
 * Memory from hipMalloc or a torch allocation at offset 0 satisfies all of them.
 */

typedef enum moe_dtype {
  MOE_F32 = 0,   /* IEEE binary32                                                   */
  MOE_BF16 = 1,  /* bfloat16                                                        */
  MOE_E4M3 = 2,  /* OCP FP8 E4M3 ("fn": max 448, no infinities), one byte           */
  MOE_MXFP4 = 3  /* OCP MXFP4: e2m1 values two per byte (the lower K index in the    */
                 /* low nibble) with one e8m0 scale 2^(c-127) per 32 values along K */
} moe_dtype;

/*
 * Problem description.  Supported combinations:
 *   dtype F32,  w_dtype F32  : everything fp32 (X, W, act, slot rows, out).
 *   dtype BF16, w_dtype BF16 : bf16 X, W, act, slot rows and out; fp32 accumulation.
 *   dtype BF16, w_dtype E4M3 : bf16 X and out; W13/W2 e4m3 codes with one fp32
 *                              scale per 128x128 block (dequantised W = code*scale);
 *                              X and act quantised to e4m3 per (row, 128-column
 *                              group) with scale amax/448; bf16 slot rows.
 *   dtype E4M3, w_dtype MXFP4: only moe_grouped_gemm_up_mxfp4 (and the dtype-free
 *                              moe_align / moe_route / moe_route_align); block_m
 *                              at most 128.
 * Limits: 1 <= top_k <= E <= 1024; T >= 1; H and I multiples of 64 (of 128 with E4M3
 *         weights), at most 32768;
 *         T*top_k < 2^31 and per-expert weight slabs < 2^31 bytes.
 * block_m: rows per m-block of the expert-sorted slot list, one of 16, 32, 64,
 *          128, or 256 (bf16 problems only); 0 lets the library choose
 *          (moe_pick_block_m).  Every entry point
 *          resolves 0 the same way, so the same moe_problem describes all stages.
 */
typedef struct moe_problem {
  int32_t T;        /* tokens                              */
  int32_t H;        /* hidden size                         */
  int32_t I;        /* expert intermediate size            */
  int32_t E;        /* number of experts                   */
  int32_t top_k;    /* experts per token                   */
  int32_t block_m;  /* 0 = library choice                  */
  int32_t dtype;    /* moe_dtype of X, act, slot rows, out */
  int32_t w_dtype;  /* moe_dtype of W13 and W2             */
} moe_problem;

/* Human-readable name of a moe_status value (static storage). */
const char* moe_status_str(int status);

/* Host-only validation of a problem; MOE_OK or the negative status the entry
 * points would return for it. */
int moe_validate(const moe_problem* p);

/* Rows per m-block the library uses for `p` (p->block_m if non-zero, else
 * moe_block_m_for(T*top_k/E, dtype, w_dtype)).  Returns a negative moe_status
 * for an invalid problem.  Block size by expected slice size: "MOE Bmm1 Fused
 * Gather", _select_base_config. */
int32_t moe_pick_block_m(const moe_problem* p);

/* The library's block size for `slots_per_expert` expected slots per expert, in
 * the manner of the block-size table of "MOE Bmm1 Fused Gather"
 * (_select_base_config, keyed on the expected slice size): few slots per expert
 * -> small blocks.  moe_pick_block_m assumes every id is a local expert.  A
 * caller whose ids mostly belong to other shards (expert parallelism: E local of
 * E_total experts) passes the slots it received per local expert that received
 * any (from its dispatch counts) and sets block_m to the result: a shard holding
 * popular experts receives several times the global mean.  (The page's bench keys
 * the same choice on the global mean T*top_k/E_total.)
 * Host only, no side effects.  MOE_ERR_DTYPE for an unsupported dtype pair,
 * MOE_ERR_SHAPE for a negative or NaN count. */
int32_t moe_block_m_for(double slots_per_expert, int32_t dtype, int32_t w_dtype);

/* Size queries (library utilities; the pages define no such calls).  They let the
 * caller allocate the outputs of moe_align and the workspaces before any launch, so
 * that no entry point needs the device-side counts on the host. */

/* Upper bound on rows of the padded expert-sorted slot list:
 * N + min(E, N) * (block_m - 1) (each of at most min(E, N) non-empty experts pads
 * fewer than block_m rows).  Negative moe_status if invalid. */
int64_t moe_max_padded_slots(const moe_problem* p);

/* Upper bound on m-blocks (tiles): moe_max_padded_slots / block_m. */
int64_t moe_max_tiles(const moe_problem* p);

/* Bytes of device workspace moe_forward needs (256-byte aligned pieces).  Library
 * utility, no page. */
int64_t moe_workspace_bytes(const moe_problem* p);

/*
 * moe_align -- sort routed slots by expert.
 * ("MOE Bmm1 Fused Gather": make_ragged_tensor_metadata, gather index = slot // top_k;
 *  "moe triton kernel use tma.": per-M-block expert id and first token row;
 *  "factor_moe_fused_gemm.cu": build_expert_map_kernel.)
 * In:  topk_ids     int32 [T, top_k]; ids outside [0,E) are excluded and counted.
 * Out: counts       int32 [E]         slots per expert
 *      offsets      int32 [E+1]       exclusive prefix sum of counts rounded up to block_m
 *      sorted_slots int32 [moe_max_padded_slots]  row offsets[e]+i holds the i-th smallest
 *                                      slot of expert e; padding rows and the unused tail
 *                                      hold the sentinel N
 *      slot_row     int32 [N]         row of each slot in sorted_slots, -1 if excluded
 *      tiles        int32 [moe_max_tiles][2]  (expert, first row) per m-block, expert-major;
 *                                      unused entries (-1,-1)
 *      num_tiles    int32 [1]         number of valid tiles
 *      n_invalid    int32 [1]         number of excluded slots (0 for valid input)
 * Every output element is written; the result is deterministic (bit-identical
 * across runs and streams).
 */
int moe_align(const moe_problem* p, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
              int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles, int32_t* num_tiles,
              int32_t* n_invalid, void* stream);

/*
 * moe_route -- router producer: top-k experts and weights from router logits.
 * ("MOE Bmm1 Fused Gather": topk(logits, experts_per_token, apply_softmax=True);
 *  "factor_moe_fused_gemm.cu": "factor 0", topk_softmax -> topk_weights, topk_ids.)
 * For every token t: p = softmax(logits[t, :]) over all E experts (fp32); topk_ids[t, :]
 * are the top_k experts in descending p, ties to the lower expert id (the selection compares
 * the logits, which softmax keeps in order); topk_weights[t, j] = p of that expert, divided by
 * the sum of the top_k chosen p when renormalize != 0.
 * In:  logits       fp32 [T, E], finite.
 * Out: topk_ids     int32 [T, top_k];  topk_weights fp32 [T, top_k].
 * Needs top_k <= 64 (MOE_ERR_SHAPE otherwise).  Deterministic.
 */
int moe_route(const moe_problem* p, const float* logits, int renormalize, int32_t* topk_ids,
              float* topk_weights, void* stream);

/*
 * moe_route_align -- moe_route followed by moe_align on its ids, as one call.
 * ("MOE Bmm1 Fused Gather": topk(logits, ..., apply_softmax=True), then the expert histogram
 *  col_sum of the routing mask; "factor_moe_fused_gemm.cu": "factor 0", topk_softmax.)
 * Up to 8192 slots (T * top_k) with E <= 1024 it is one launch from the logits to the
 * alignment: the routing stays spread over the GPU (a wavefront per token), and the workgroup
 * that finishes its routing last aligns every id.  The launch hands the ids from workgroup to
 * workgroup through a completion counter, one of 64 that the library keeps per device and
 * takes in turn per call, so at most 64 calls may be in flight at once across all streams of
 * a device.  Larger problems run the routing launch and then the alignment launches on
 * `stream`, with no host synchronisation between them.  Arguments and outputs are those of
 * the two calls; results are identical to calling them in sequence.
 */
int moe_route_align(const moe_problem* p, const float* logits, int renormalize,
                    int32_t* topk_ids, float* topk_weights, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles, int32_t* num_tiles,
                    int32_t* n_invalid, void* stream);

/*
 * moe_quantize_rows_e4m3 -- fp8 workload only (dtype BF16, w_dtype E4M3).
 * ("MOE Bmm1 Fused Gather", pack_e4m3x2: round to nearest even, saturate to finite.)
 * For each token row t and 128-column group g of x (bf16 [T,H]):
 *   scales[t,g] = amax|x[t,g-group]| / 448 in fp32 (1 if the group is all zero),
 *   xq[t,h]     = e4m3(x[t,h] / scales[t,h/128]), IEEE fp32 quotient, RNE, saturating.
 * Out: xq uint8 [T,H] (e4m3 codes), scales fp32 [T, H/128].
 */
int moe_quantize_rows_e4m3(const moe_problem* p, const void* x, uint8_t* xq, float* scales,
                           void* stream);

/*
 * moe_grouped_gemm_up -- gather-fused up projection with the SiLU(gate)*up epilogue.
 * ("MOE Bmm1 Fused Gather": load_activations gathers rows slot // top_k and zero-fills
 *  masked rows; the SwiGLU runs in the GEMM epilogue.  "factor_moe_fused_gemm.cu":
 *  fused_silu_gate_kernel.)
 * For every valid tile (e, row0) and row r in [row0, row0+block_m):
 *   x_r = X[sorted_slots[r] / top_k]  (zero row when sorted_slots[r] is the sentinel)
 *   act[r, n] = SiLU(W13[e, n, :] . x_r) * (W13[e, I+n, :] . x_r),  n in [0, I)
 * In:  x        dtype [T,H]; for E4M3 weights: the e4m3 codes [T,H] from
 *               moe_quantize_rows_e4m3 with x_scales fp32 [T,H/128] (else x_scales NULL)
 *      w13      w_dtype [E, 2I, H]; w13_scales fp32 [E, 2I/128, H/128] for E4M3 (else NULL)
 *      sorted_slots, offsets, tiles, num_tiles: outputs of moe_align for the same problem
 * Out: act      [moe_max_padded_slots, I]: dtype, or e4m3 codes for E4M3 weights with
 *               act_scales fp32 [moe_max_padded_slots, I/128] (amax/448 per row and
 *               128-column group, as above).  Rows of valid tiles are written (padding
 *               rows get 0); rows past the last valid tile are left untouched.
 * workspace: NULL, or the optional GEMM workspace described at moe_gemm_workspace_bytes
 *      (MOE_ERR_WORKSPACE if smaller, MOE_ERR_ALIGN if not 256-byte aligned).
 */
int moe_grouped_gemm_up(const moe_problem* p, const void* x, const float* x_scales,
                        const void* w13, const float* w13_scales, const int32_t* sorted_slots,
                        const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                        void* act, float* act_scales, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * moe_grouped_gemm_up_mxfp4 -- the up projection of the "MOE Bmm1 Fused Gather"
 * example's own variant: MXFP4 weights x e4m3 activations, per-expert bias, the
 * GPT-OSS SwiGLU and an e4m3 output with a flex scale.  (mma_partition: e2m1 weights
 * with 32-wide microscales times e4m3 rows; apply_bias_and_scale: acc * x_scale +
 * bias; _swiglu_step1/2; pack_fp8_out_fragment: RNE and saturation to +-448.)
 * Problem: dtype MOE_E4M3, w_dtype MOE_MXFP4; H and I multiples of 64; block_m <= 128.
 * For every valid tile (e, row0) and row r with sorted_slots[r] != sentinel:
 *   x_r  = X[sorted_slots[r] / top_k]             (e4m3 codes)
 *   h[n] = x_scale * (W13[e, n, :] . x_r) + bias[e, n],   n in [0, 2I)
 *   g = min(h[2c], limit),  l = clamp(h[2c+1], -limit, limit)
 *   act[r, c] = e4m3( g / (1 + exp(-alpha * g)) * (l + 1) / out_scale ),  c in [0, I)
 * In:  x         uint8 [T, H] e4m3 codes; x_scale fp32 [1] (device)
 *      w13       uint8 [E, 2I, H/2]: row n holds W13[e, n, :] as e2m1 pairs; rows come in
 *                (gate, linear) pairs: row 2c is the gate and row 2c+1 the linear part of
 *                act column c (the page's interleaved columns)
 *      w13_scales uint8 [E, H/32, 2I]: e8m0 scale of W13[e, n, 32b .. 32b+31] at [e, b, n]
 *      bias      fp32 [E, 2I], same row order; alpha, limit: host floats; out_scale fp32 [1]
 *      sorted_slots, offsets, tiles, num_tiles: outputs of moe_align for the same problem
 * Out: act       uint8 [moe_max_padded_slots, I] e4m3 codes in padded expert-sorted row
 *                order; padding rows and rows past the last valid tile are not written.
 * All device pointers 16-byte aligned.  MOE_ERR_DTYPE for any other dtype pair.
 */
int moe_grouped_gemm_up_mxfp4(const moe_problem* p, const uint8_t* x, const float* x_scale,
                              const uint8_t* w13, const uint8_t* w13_scales, const float* bias,
                              float alpha, float limit, const float* out_scale,
                              const int32_t* sorted_slots, const int32_t* offsets,
                              const int32_t* tiles, const int32_t* num_tiles, uint8_t* act,
                              void* stream);

/*
 * moe_grouped_gemm_down -- down projection with the routing weight in the epilogue.
 * ("moe triton kernel use tma.": MUL_ROUTED_WEIGHT on the down projection, whose
 *  token rows are contiguous in sorted order.)
 * For every valid tile (e, row0) and row r with s = sorted_slots[r] != sentinel:
 *   slot_out[s, h] = w[s] * (W2[e, h, :] . act[r, :]),  h in [0, H)
 * In:  act, act_scales  as written by moe_grouped_gemm_up
 *      w2  w_dtype [E, H, I]; w2_scales fp32 [E, H/128, I/128] for E4M3 (else NULL)
 *      topk_weights fp32 [T, top_k]
 *      sorted_slots, offsets, tiles, num_tiles: outputs of moe_align for the same problem
 * Out: slot_out dtype [N, H] (bf16 for E4M3 weights).  Rows of excluded slots
 *      are not written.
 * workspace: NULL, or the optional GEMM workspace described at moe_gemm_workspace_bytes
 *      (MOE_ERR_WORKSPACE if smaller, MOE_ERR_ALIGN if not 256-byte aligned).
 */
int moe_grouped_gemm_down(const moe_problem* p, const void* act, const float* act_scales,
                          const void* w2, const float* w2_scales, const float* topk_weights,
                          const int32_t* sorted_slots, const int32_t* offsets,
                          const int32_t* tiles, const int32_t* num_tiles, void* slot_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the optional workspace of moe_grouped_gemm_up and moe_grouped_gemm_down (0: the
 * problem's GEMMs never use one); negative moe_status for an invalid problem.  Library
 * utility, no page (the split it sizes is this library's own, see below).
 * The workspace is device memory, 256-byte aligned, caller-owned scratch whose contents are
 * unspecified afterwards; calls that share one must not overlap.  With it, bf16 problems of
 * 128- or 256-row m-blocks cut the tiles of a GEMM's last, partly filled round of workgroups
 * (one per compute unit) along K into parts whose fp32 partial tiles are added in a fixed
 * order before the epilogue: the result is deterministic, but its rounding differs from a
 * call without workspace.  moe_forward carves the same buffer out of its own workspace.
 */
int64_t moe_gemm_workspace_bytes(const moe_problem* p);

/*
 * moe_combine -- deterministic per-token combine, no atomics.
 * ("factor_moe_fused_gemm.cu": weighted_scatter_add_kernel / index_add_ of the slow path.)
 *   out[t, h] = round( sum over j = 0..top_k-1 in ascending order of slot_out[t*top_k+j, h] )
 * with the sum carried in fp32 and rounded once to dtype; slots with
 * slot_row[s] < 0 (excluded ids) are skipped.
 * In:  slot_out dtype [N, H] (bf16 for E4M3 weights), slot_row int32 [N]
 * Out: out dtype [T, H]
 */
int moe_combine(const moe_problem* p, const void* slot_out, const int32_t* slot_row, void* out,
                void* stream);

/*
 * moe_forward -- the whole layer: align, [quantise X], up, down, combine.
 * In:  x dtype [T,H]; topk_ids int32 [T,top_k]; topk_weights fp32 [T,top_k];
 *      w13, w13_scales, w2, w2_scales as above (scales NULL unless E4M3).
 * Out: out dtype [T,H].
 * workspace: device memory of at least moe_workspace_bytes(p) bytes, 256-byte
 *      aligned.  Its first int32 receives the number of excluded slots
 *      (n_invalid); the rest is scratch whose contents are unspecified.
 * No host synchronisation: all kernels are sized by host-side upper bounds
 * and read the tile count from device memory.
 */
int moe_forward(const moe_problem* p, const void* x, const int32_t* topk_ids,
                const float* topk_weights, const void* w13, const float* w13_scales,
                const void* w2, const float* w2_scales, void* out, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Bytes of the library-owned device array behind moe_forward_scratch (one per GPU the
 * library runs on, held until the process ends).
 */
#define MOE_SCRATCH_MAX_BYTES (128u * 1024u * 1024u)

/* MOE_SCRATCH_MAX_BYTES as a value (host only). */
int64_t moe_scratch_max_bytes(void);

/*
 * moe_forward_scratch -- moe_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels, launch sequence and results (bit for bit) as moe_forward, but the
 * intermediates live in a library-owned device array of MOE_SCRATCH_MAX_BYTES on the current
 * GPU instead of a caller workspace.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); the caller still passes every input and `out`.
 * n_invalid: NULL, or device int32 [1] that receives the number of excluded slots.
 * Errors: MOE_ERR_WORKSPACE when moe_workspace_bytes(p) exceeds MOE_SCRATCH_MAX_BYTES (the
 * problem does not fit: use moe_forward); MOE_ERR_DEVICE if the array's address cannot be
 * obtained; otherwise as moe_forward.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (no part
 * of it needs to start zeroed).  Calls that overlap on one GPU -- on different streams, or
 * from different threads without ordering -- race on it and give undefined results.
 */
int moe_forward_scratch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                        const float* topk_weights, const void* w13, const float* w13_scales,
                        const void* w2, const float* w2_scales, void* out, int32_t* n_invalid,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
