// Internal declarations shared by the HIP translation units of libmoe (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// Vector types for the gfx950 MFMA builtins
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kGroup = 128;      // fp8 weight block edge and activation group width
constexpr int kMaxDim = 32768;   // largest supported H and I
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// OCP E4M3 ("fn") encode: round to nearest even, saturate to +-448, sign kept.
// Written from the format: 4 exponent bits (bias 7), 3 mantissa bits, subnormal
// step 2^-9, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fminf(fabsf(f), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of step 2^-9
    // a * 2^9 is exact; rint rounds half to even
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8 (8 = smallest normal 2^-6)
  } else {
    uint32_t ua = __float_as_uint(a);
    // keep 3 mantissa bits with round-half-even on the 20 discarded bits
    uint32_t lsb = (ua >> 20) & 1u;
    ua += 0x7FFFFu + lsb;
    uint32_t e = (ua >> 23) - 127 + 7;       // rebias; rounding may have bumped the exponent
    uint32_t m = (ua >> 20) & 7u;
    code = (e << 3) | m;
    if (code > 0x7Eu) code = 0x7Eu;          // a <= 448 already; guards the bump past 448
  }
  return sign | code;
}

// ---------------------------------------------------------------------------------------------
// MFMA operand types
// ---------------------------------------------------------------------------------------------
struct OpBf16 {
  static constexpr int ELT = 2;   // bytes per element
  static constexpr int KPM = 32;  // k covered by one MFMA
  static constexpr int LB = 16;   // operand bytes per lane
  using frag = bf16x8;
  __device__ static __forceinline__ frag load(const char* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

struct OpF32 {
  static constexpr int ELT = 4;
  static constexpr int KPM = 4;
  static constexpr int LB = 4;
  using frag = float;
  __device__ static __forceinline__ frag load(const char* p) {
    return *reinterpret_cast<const float*>(p);
  }
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

struct OpE4M3 {
  static constexpr int ELT = 1;
  static constexpr int KPM = 128;
  static constexpr int LB = 32;
  using frag = i32x8;
  __device__ static __forceinline__ frag load(const char* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    frag f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
  }
  // format 0 = e4m3 for both operands; E8M0 scale 127 = 1.0 (no MX scaling here)
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

enum OutKind { OUT_F32 = 0, OUT_BF16 = 1, OUT_E4M3 = 2 };

// Work split over the 8 XCDs (each with its own L2): block b runs on XCD b % 8; each XCD
// takes a contiguous range of the `valid` logical tiles (device-side tile count x n-blocks),
// so no XCD idles on the slack between the host-side tile bound and the real count.  The
// grid must be a multiple of 8 and at least `valid`.  -1: nothing to do for this block.
__device__ __forceinline__ int xcd_logical(int b, int valid) {
  const int per = (valid + 7) >> 3;
  const int i = b >> 3;
  if (i >= per) return -1;
  const int l = (b & 7) * per + i;
  return l < valid ? l : -1;
}

// Logical tile order, expert by expert: inside expert e (m-blocks base..base+M-1) groups of
// G m-blocks sweep the n-blocks, n-block-major inside a group.  A group never holds two
// experts, so concurrent workgroups of one XCD share their weight tiles (each fetched once)
// and their gathered rows.  With one m-block per expert this is n-block order.
// logical / n_blocks is an m-block of the expert that owns `logical`, so one read of the tile
// table gives the expert; offsets are multiples of the m-block size and the tile table lists
// m-blocks expert by expert, so m-block mt starts at row mt * BMT.
struct TileRef {
  int e, mt, nt, row0;   // expert, m-block, n-block, first row of the m-block
};
template <int BMT, int G>
__device__ __forceinline__ TileRef grouped_tile(int logical, int n_blocks, const int32_t* tiles,
                                                const int32_t* offsets) {
  TileRef t;
  t.e = tiles[2 * (logical / n_blocks)];
  const int base = offsets[t.e] / BMT;
  const int M = (offsets[t.e + 1] - offsets[t.e]) / BMT;
  const int r = logical - base * n_blocks;          // 0 <= r < M * n_blocks
  const int full = M / G;
  if (r < full * G * n_blocks) {
    const int g = r / (G * n_blocks), w = r - g * G * n_blocks;
    t.nt = w / G;
    t.mt = base + g * G + (w - t.nt * G);
  } else {
    const int rem = M - full * G, w = r - full * G * n_blocks;
    t.nt = w / rem;
    t.mt = base + full * G + (w - t.nt * rem);
  }
  t.row0 = t.mt * BMT;
  return t;
}

// Block b -> logical tile, in chunks: the logical order is cut into chunks of C tiles that are
// dealt to the XCDs in turn (chunk c to XCD c mod 8), and each XCD runs its chunks in order.
// A chunk keeps tiles that share operands on one L2 at the same time; dealing them in turn
// spreads expensive and cheap parts of the order (a hot expert, the padded last m-blocks of
// small experts) over all XCDs.  The grid must be xcd_chunked_grid(tile bound).
template <int C>
__device__ __forceinline__ int xcd_chunked(int b, int valid) {
  const int x = b & 7, i = b >> 3;
  const int l = ((i / C) * 8 + x) * C + (i % C);
  return l < valid ? l : -1;
}

// Grid for xcd_chunked<C> over at most g logical tiles: every XCD gets as many whole chunks
// of block positions as the XCD with the most chunks needs.
template <int C>
inline int64_t xcd_chunked_grid(int64_t g) {
  return ((g + C - 1) / C + 7) / 8 * 8 * C;
}

// Direct-to-LDS copies (gfx950 global_load_lds_dwordx4 / _dword): each wave instruction lands
// 64 lanes x 16 (or 4) bytes contiguously in LDS at M0.  Issued from inline assembly with
// explicit vmcnt waits: the compiler's own tracking of LDS DMA makes every LDS read wait for
// every outstanding copy, which would drain a multi-stage ring each k-slice.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr)
               : "memory");
}

__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_addr)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


template <class T>
__device__ __forceinline__ uint32_t lds_u32(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)p;
}

// ---------------------------------------------------------------------------------------------
// Launchers (host side), one per translation unit
// ---------------------------------------------------------------------------------------------
struct Resolved {
  int32_t T, H, I, E, K;   // K = top_k
  int32_t BM;
  int32_t dtype, w_dtype;
  int64_t N;               // T*top_k
  int64_t rows_max;        // moe_max_padded_slots
  int64_t tiles_max;       // moe_max_tiles
};

hipError_t launch_route(const Resolved& r, const float* logits, int renorm, int32_t* topk_ids,
                        float* topk_w, hipStream_t s);
hipError_t launch_route_align(const Resolved& r, const float* logits, int renorm, int32_t* topk_ids,
                              float* topk_w, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles,
                              int32_t* num_tiles, int32_t* n_invalid, hipStream_t s);
hipError_t launch_align(const Resolved& r, const int32_t* ids, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles,
                        int32_t* num_tiles, int32_t* n_invalid, hipStream_t s);
// Routing and alignment as one launch (moe_align.hip), for the problems it covers.
bool route_align_one_launch(const Resolved& r);
hipError_t launch_route_align_one(const Resolved& r, const float* logits, int renorm,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  int32_t* offsets, int32_t* sorted_slots, int32_t* slot_row,
                                  int32_t* tiles, int32_t* num_tiles, int32_t* n_invalid,
                                  hipStream_t s);

hipError_t launch_quant_rows(const Resolved& r, const void* x, uint8_t* xq, float* scales,
                             hipStream_t s);

hipError_t launch_up(const Resolved& r, const void* x, const float* x_scales, const void* w13,
                     const float* w13_scales, const int32_t* sorted_slots, const int32_t* offsets,
                     const int32_t* tiles, const int32_t* num_tiles, void* act, float* act_scales,
                     void* split_ws, hipStream_t s);

// split_ws: partial-tile buffer of gemm_split_bytes(r) bytes for the K-split tail of the
// 128/256-row bf16 GEMMs, or null (no split).
hipError_t launch_down(const Resolved& r, const void* act, const float* act_scales,
                       const void* w2, const float* w2_scales, const float* topk_w,
                       const int32_t* sorted_slots, const int32_t* offsets, const int32_t* tiles,
                       const int32_t* num_tiles, void* slot_out, void* split_ws, hipStream_t s);
int64_t gemm_split_bytes(const Resolved& r);
// Compute units of the current device (cached per device ordinal).
int device_cu_count();

// bf16 kernels for 128-row m-blocks (MFMA 32x32x16), used by launch_up / launch_down.
bool prefill_supported(const Resolved& r);
hipError_t launch_up_prefill(const Resolved& r, const void* x, const void* w13,
                             const int32_t* sorted_slots, const int32_t* offsets,
                             const int32_t* tiles, const int32_t* num_tiles, void* act,
                             void* split_ws, hipStream_t s);
hipError_t launch_down_prefill(const Resolved& r, const void* act, const void* w2,
                               const float* topk_w, const int32_t* sorted_slots,
                               const int32_t* offsets, const int32_t* tiles,
                               const int32_t* num_tiles, void* slot_out, void* split_ws,
                               hipStream_t s);

// Weight-streaming kernels (bf16 m-blocks of 16..64 rows, e4m3 m-blocks of 128 rows).
bool stream_supported(const Resolved& r);
hipError_t launch_up_stream(const Resolved& r, const void* x, const float* x_scales,
                            const void* w13, const float* w13_scales, const int32_t* sorted_slots,
                            const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                            void* act, float* act_scales, hipStream_t s);
hipError_t launch_down_stream(const Resolved& r, const void* act, const float* act_scales,
                              const void* w2, const float* w2_scales, const float* topk_w,
                              const int32_t* sorted_slots, const int32_t* offsets,
                              const int32_t* tiles, const int32_t* num_tiles, void* slot_out,
                              hipStream_t s);

hipError_t launch_up_mxfp4(const Resolved& r, const uint8_t* x, const float* x_scale,
                           const uint8_t* w13, const uint8_t* w13_scales, const float* bias,
                           float alpha, float limit, const float* out_scale,
                           const int32_t* sorted_slots, const int32_t* offsets,
                           const int32_t* tiles, const int32_t* num_tiles, uint8_t* act,
                           hipStream_t s);
hipError_t launch_combine(const Resolved& r, const void* slot_out, const int32_t* slot_row,
                          void* out, hipStream_t s);

}  // namespace moe
