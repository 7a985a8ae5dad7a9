// Grouped GEMMs of the MoE expert layer on gfx950 MFMA.
//
//   up   (gather-fused): act[r, n]   = SiLU(W13[e,n,:].x_r) * (W13[e,I+n,:].x_r),
//                         x_r = X[sorted_slots[r] / top_k] (zero row for the sentinel)
//   down (contiguous)  : slot_out[s, h] = w[s] * (W2[e,h,:].act[r,:]),  s = sorted_slots[r]
//
// Sources: "MOE Bmm1 Fused Gather" (load_activations gathers token rows through the
// expert-sorted index and zero-fills masked rows; the SwiGLU runs in the GEMM
// epilogue; a tile is (slice, m-block, n-block) from a block schedule), "moe triton
// kernel use tma." (weights laid out [E, N, K] with K contiguous; the down projection
// multiplies the routed weight; its token rows are contiguous in sorted order) and
// "factor_moe_fused_gemm.cu" (gate is the first half of W13's rows; SiLU(g) =
// g / (1 + exp(-g))).
//
// Kernel shape (one workgroup per (m-block, n-block) tile):
//   * both operands are K-contiguous ("NT"): every lane fetches 16-byte runs of one
//     row, for the gathered A rows as well as the weight rows;
//   * a BK-deep k-slice of A (BM rows) and of the weight tile (2*BN rows for up: gate
//     then up; BN rows for down) is staged through a double-buffered LDS ring with a
//     16-byte row pad (conflict-free ds_read_b128 for 16 rows at one k offset); the
//     next slice's global loads are in flight while the current slice is multiplied;
//   * MFMA 16x16 tiles: bf16 16x16x32, fp32 16x16x4, e4m3 16x16x128.  For e4m3 the
//     k-slice is exactly one 128-wide scale block: each slice's MFMA product is
//     scaled by (row scale x weight block scale) into the fp32 accumulator;
//   * the grid is sized by the host-side tile bound; workgroups past the device-side
//     tile count exit at once (no host synchronisation);
//   * workgroup ids are remapped so each of the 8 XCDs (own L2) runs a contiguous
//     range of the valid tiles, and consecutive tiles share one weight tile (m-blocks
//     at the same n-block).
#include <type_traits>

#include "moe_internal.h"

namespace moe {


struct GemmArgs {
  const char* a_src;          // up: X or its e4m3 codes [T, K]; down: act [rows_max, K]
  const float* a_scales;      // e4m3: up x_scales [T, K/128]; down act_scales [rows, K/128]
  const char* w;              // up: W13 [E, 2I, K]; down: W2 [E, H, K]
  const float* w_scales;      // e4m3: [E, w_rows/128, K/128]
  const int32_t* sorted_slots;
  const int32_t* tiles;
  const int32_t* num_tiles;
  const float* topk_w;        // down only, [N]
  void* out;                  // up: act [rows_max, n_out]; down: slot_out [N, n_out]
  float* out_scales;          // up e4m3: act_scales [rows_max, n_out/128]
  int K;                      // reduction length (up: H, down: I)
  int n_out;                  // output columns (up: I, down: H)
  int top_k;
  int n_slots;                // N = T*top_k (also the sentinel)
  int tiles_max;
  int64_t w_expert_elems;     // elements per expert weight slab
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  // SiLU(g) * u = g / (1 + exp(-g)) * u; exp(-g) = inf for very negative g gives -0.
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <class Op, int BM, int BN, int BK, int WM, int WN, bool UP, int OUT>
__global__ __launch_bounds__(WM* WN* kWave) void moe_gemm_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * kWave;
  constexpr bool SCALED = std::is_same<Op, OpE4M3>::value;
  constexpr int BROWS = UP ? 2 * BN : BN;          // weight rows staged per tile
  constexpr int ROWB = BK * Op::ELT;               // bytes of one row's k-slice
  constexpr int LDSR = ROWB + 16;                  // padded LDS row stride
  constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row slice
  constexpr int A_CH = BM * CPR, B_CH = BROWS * CPR;
  constexpr int A_PT = (A_CH + NT - 1) / NT, B_PT = (B_CH + NT - 1) / NT;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int NF = UP ? 2 * FN : FN;
  constexpr int STAGE = (BM + BROWS) * LDSR;
  static_assert(BK % Op::KPM == 0, "k-slice must hold whole MFMAs");
  static_assert(!SCALED || BK == kGroup, "e4m3 k-slice is one scale block");
  static_assert(!SCALED || BN == kGroup, "e4m3 n-block is one scale block / act group");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile is whole 16x16 MFMA tiles");

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];
  __shared__ float a_scale_lds[SCALED ? 2 * BM : 1];
  __shared__ float red_lds[(SCALED && UP) ? WN * BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  // logical order: m-block fastest, so consecutive workgroups share one weight tile
  const int ntiles = *g.num_tiles;
  const int bid = xcd_logical(blockIdx.x, ntiles * (g.n_out / BN));
  if (bid < 0) return;
  const int mt = bid % ntiles;
  const int nt = bid / ntiles;
  const int e = g.tiles[2 * mt];
  const int row0 = g.tiles[2 * mt + 1];
  const int n0 = nt * BN;
  const int K = g.K;
  const int KT = K / BK;

  // ---- global source pointers (fixed over k) ----------------------------------------------
  const char* a_ptr[A_PT];
  bool a_ok[A_PT];
  int a_tok[A_PT];
  #pragma unroll
  for (int i = 0; i < A_PT; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    a_ok[i] = false;
    a_ptr[i] = g.a_src;
    a_tok[i] = 0;
    if (c < A_CH) {
      if (UP) {
        const int s = g.sorted_slots[row0 + r];
        a_ok[i] = s < g.n_slots;
        const int tok = a_ok[i] ? s / g.top_k : 0;
        a_tok[i] = tok;
        a_ptr[i] = g.a_src + ((size_t)tok * K) * Op::ELT + cc * 16;
      } else {
        a_ok[i] = true;
        a_ptr[i] = g.a_src + ((size_t)(row0 + r) * K) * Op::ELT + cc * 16;
      }
    }
  }
  const char* wbase = g.w + (size_t)e * g.w_expert_elems * Op::ELT;
  const int w_rows_total = UP ? 2 * g.n_out : g.n_out;
  const char* b_ptr[B_PT];
  #pragma unroll
  for (int i = 0; i < B_PT; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    int grow = 0;
    if (c < B_CH) grow = UP ? (r < BN ? n0 + r : g.n_out + n0 + (r - BN)) : n0 + r;
    b_ptr[i] = wbase + ((size_t)grow * K) * Op::ELT + cc * 16;
  }
  (void)w_rows_total;

  // e4m3 row scales: thread r < BM owns row r's scale source
  const float* sa_src = nullptr;
  if (SCALED && tid < BM) {
    if (UP) {
      const int s = g.sorted_slots[row0 + tid];
      const int tok = (s < g.n_slots) ? s / g.top_k : 0;
      sa_src = g.a_scales + (size_t)tok * (K / kGroup);
    } else {
      sa_src = g.a_scales + (size_t)(row0 + tid) * (K / kGroup);
    }
  }
  const float* sw_gate = nullptr;
  const float* sw_up = nullptr;
  if (SCALED) {
    const int kb = K / kGroup;
    const float* se = g.w_scales + (size_t)e * (w_rows_total / kGroup) * kb;
    sw_gate = se + (size_t)(n0 / kGroup) * kb;
    sw_up = UP ? se + (size_t)((g.n_out + n0) / kGroup) * kb : sw_gate;
  }

  i32x4 ra[A_PT], rb[B_PT];
  float rsa = 0.0f;
  auto gload = [&](int kt) {
    const int koff = kt * ROWB;
    #pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      i32x4 v = {0, 0, 0, 0};
      if (a_ok[i]) v = *reinterpret_cast<const i32x4*>(a_ptr[i] + koff);
      ra[i] = v;
    }
    #pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      if (B_CH % NT == 0 || tid + i * NT < B_CH)
        rb[i] = *reinterpret_cast<const i32x4*>(b_ptr[i] + koff);
    }
    if (SCALED && tid < BM) rsa = sa_src[kt];
  };
  auto sstore = [&](int buf) {
    char* st = lds + buf * STAGE;
    #pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * NT;
      if (A_CH % NT == 0 || c < A_CH)
        *reinterpret_cast<i32x4*>(st + (c / CPR) * LDSR + (c % CPR) * 16) = ra[i];
    }
    #pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * NT;
      if (B_CH % NT == 0 || c < B_CH)
        *reinterpret_cast<i32x4*>(st + (BM + c / CPR) * LDSR + (c % CPR) * 16) = rb[i];
    }
    if (SCALED && tid < BM) a_scale_lds[buf * BM + tid] = rsa;
  };

  f32x4 acc[FM][NF];
  #pragma unroll
  for (int i = 0; i < FM; ++i)
    #pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15;           // row of an operand fragment
  const int lk = (lane >> 4) * Op::LB;  // byte offset of this lane's k run in an MFMA step

  auto compute = [&](int buf, int kt) {
    const char* st = lds + buf * STAGE;
    f32x4 part[FM][NF];
    if (SCALED) {
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int j = 0; j < NF; ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    #pragma unroll
    for (int kk = 0; kk < BK / Op::KPM; ++kk) {
      typename Op::frag af[FM], bfr[NF];
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = Op::load(st + (wm * WTM + i * 16 + lrow) * LDSR + kk * Op::KPM * Op::ELT + lk);
      #pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int brow = UP ? ((j < FN) ? wn * WTN + j * 16 : BN + wn * WTN + (j - FN) * 16)
                            : wn * WTN + j * 16;
        bfr[j] = Op::load(st + (BM + brow + lrow) * LDSR + kk * Op::KPM * Op::ELT + lk);
      }
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int j = 0; j < NF; ++j) {
          if (SCALED) part[i][j] = Op::mma(af[i], bfr[j], part[i][j]);
          else acc[i][j] = Op::mma(af[i], bfr[j], acc[i][j]);
        }
    }
    if (SCALED) {
      const float swg = sw_gate[kt];
      const float swu = sw_up[kt];
      #pragma unroll
      for (int i = 0; i < FM; ++i) {
        float sa[4];
        #pragma unroll
        for (int v = 0; v < 4; ++v)
          sa[v] = a_scale_lds[buf * BM + wm * WTM + i * 16 + (lane >> 4) * 4 + v];
        #pragma unroll
        for (int j = 0; j < NF; ++j) {
          const float sw = (UP && j >= FN) ? swu : swg;
          #pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += part[i][j][v] * (sa[v] * sw);
        }
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kt + 1);
    compute(kt & 1, kt);
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------------------
  // MFMA 16x16 result: lane holds rows (lane/16)*4 + v, column lane%16 of each 16x16 tile.
  const int ocol = lane & 15;
  const int orow = (lane >> 4) * 4;
  if (UP) {
    float a[FM][FN][4];
    #pragma unroll
    for (int i = 0; i < FM; ++i)
      #pragma unroll
      for (int j = 0; j < FN; ++j)
        #pragma unroll
        for (int v = 0; v < 4; ++v) a[i][j][v] = silu_mul(acc[i][j][v], acc[i][j + FN][v]);

    if (OUT == OUT_E4M3) {
      // amax per row over the tile's 128 columns (= one activation group)
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          float m = 0.0f;
          #pragma unroll
          for (int j = 0; j < FN; ++j) m = fmaxf(m, fabsf(a[i][j][v]));
          #pragma unroll
          for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
          if (ocol == 0) red_lds[wn * BM + wm * WTM + i * 16 + orow + v] = m;
        }
      __syncthreads();
      uint8_t* act = reinterpret_cast<uint8_t*>(g.out);
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = wm * WTM + i * 16 + orow + v;
          float amax = 0.0f;
          #pragma unroll
          for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red_lds[w * BM + m]);
          const float s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
          const size_t rowoff = (size_t)(row0 + m) * g.n_out + n0;
          #pragma unroll
          for (int j = 0; j < FN; ++j)
            act[rowoff + wn * WTN + j * 16 + ocol] = (uint8_t)f32_to_e4m3(a[i][j][v] / s);
          if (wn == 0 && ocol == 0)
            g.out_scales[(size_t)(row0 + m) * (g.n_out / kGroup) + n0 / kGroup] = s;
        }
    } else {
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          const size_t rowoff = (size_t)(row0 + wm * WTM + i * 16 + orow + v) * g.n_out + n0;
          #pragma unroll
          for (int j = 0; j < FN; ++j) {
            const size_t o = rowoff + wn * WTN + j * 16 + ocol;
            if (OUT == OUT_BF16)
              reinterpret_cast<uint16_t*>(g.out)[o] = (uint16_t)f32_to_bf16_bits(a[i][j][v]);
            else
              reinterpret_cast<float*>(g.out)[o] = a[i][j][v];
          }
        }
    }
  } else {
    #pragma unroll
    for (int i = 0; i < FM; ++i)
      #pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int s = g.sorted_slots[row0 + wm * WTM + i * 16 + orow + v];
        if (s >= g.n_slots) continue;
        const float wt = g.topk_w[s];
        const size_t rowoff = (size_t)s * g.n_out + n0;
        #pragma unroll
        for (int j = 0; j < FN; ++j) {
          const size_t o = rowoff + wn * WTN + j * 16 + ocol;
          const float y = acc[i][j][v] * wt;
          if (OUT == OUT_BF16)
            reinterpret_cast<uint16_t*>(g.out)[o] = (uint16_t)f32_to_bf16_bits(y);
          else
            reinterpret_cast<float*>(g.out)[o] = y;
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Tile configurations per block_m and dtype
// ---------------------------------------------------------------------------------------------
template <class Op, int BM, int BN, int BK, int WM, int WN, bool UP, int OUT>
static hipError_t run(const GemmArgs& a, int n_blocks_n, hipStream_t s) {
  // multiple of 8: every XCD's share of the valid tiles must have blocks to run on
  const int64_t grid = ((int64_t)a.tiles_max * n_blocks_n + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((moe_gemm_kernel<Op, BM, BN, BK, WM, WN, UP, OUT>), dim3((unsigned)grid),
                     dim3(WM * WN * kWave), 0, s, a);
  return hipGetLastError();
}

// BN = 128 output columns per tile for every configuration (H and I are multiples of
// 128).  Waves: 2x2 for 128-row blocks, 1x4 for smaller blocks (all waves along N).
template <class Op, int BK, bool UP, int OUT>
static hipError_t dispatch_bm(const Resolved& r, const GemmArgs& a, hipStream_t s) {
  if constexpr (!std::is_same<Op, OpE4M3>::value) {
    if (a.n_out % 128 != 0) {   // n_out a multiple of 64 only (bf16 / fp32): 64-wide n-blocks
      const int nb = a.n_out / 64;
      switch (r.BM) {
        case 16: return run<Op, 16, 64, BK, 1, 4, UP, OUT>(a, nb, s);
        case 32: return run<Op, 32, 64, BK, 1, 4, UP, OUT>(a, nb, s);
        case 64: return run<Op, 64, 64, BK, 1, 4, UP, OUT>(a, nb, s);
        case 128: return run<Op, 128, 64, BK, 2, 2, UP, OUT>(a, nb, s);
        default: return hipErrorInvalidValue;
      }
    }
  }
  const int nb = a.n_out / 128;
  switch (r.BM) {
    case 16: return run<Op, 16, 128, BK, 1, 4, UP, OUT>(a, nb, s);
    case 32: return run<Op, 32, 128, BK, 1, 4, UP, OUT>(a, nb, s);
    case 64: return run<Op, 64, 128, BK, 1, 4, UP, OUT>(a, nb, s);
    case 128: return run<Op, 128, 128, BK, 2, 2, UP, OUT>(a, nb, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_up(const Resolved& r, const void* x, const float* x_scales, const void* w13,
                     const float* w13_scales, const int32_t* sorted_slots, const int32_t* offsets,
                     const int32_t* tiles, const int32_t* num_tiles, void* act, float* act_scales,
                     void* split_ws, hipStream_t s) {
  if (prefill_supported(r))
    return launch_up_prefill(r, x, w13, sorted_slots, offsets, tiles, num_tiles, act, split_ws, s);
  if (stream_supported(r))
    return launch_up_stream(r, x, x_scales, w13, w13_scales, sorted_slots, offsets, tiles,
                            num_tiles, act, act_scales, s);
  GemmArgs a{};
  a.a_src = (const char*)x;
  a.a_scales = x_scales;
  a.w = (const char*)w13;
  a.w_scales = w13_scales;
  a.sorted_slots = sorted_slots;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.topk_w = nullptr;
  a.out = act;
  a.out_scales = act_scales;
  a.K = r.H;
  a.n_out = r.I;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  a.tiles_max = (int)r.tiles_max;
  a.w_expert_elems = (int64_t)2 * r.I * r.H;
  if (r.w_dtype == MOE_E4M3) return dispatch_bm<OpE4M3, 128, true, OUT_E4M3>(r, a, s);
  if (r.w_dtype == MOE_BF16) return dispatch_bm<OpBf16, 64, true, OUT_BF16>(r, a, s);
  return dispatch_bm<OpF32, 32, true, OUT_F32>(r, a, s);
}

hipError_t launch_down(const Resolved& r, const void* act, const float* act_scales,
                       const void* w2, const float* w2_scales, const float* topk_w,
                       const int32_t* sorted_slots, const int32_t* offsets, const int32_t* tiles,
                       const int32_t* num_tiles, void* slot_out, void* split_ws,
                       hipStream_t s) {
  if (prefill_supported(r))
    return launch_down_prefill(r, act, w2, topk_w, sorted_slots, offsets, tiles, num_tiles,
                               slot_out, split_ws, s);
  if (stream_supported(r))
    return launch_down_stream(r, act, act_scales, w2, w2_scales, topk_w, sorted_slots, offsets,
                              tiles, num_tiles, slot_out, s);
  GemmArgs a{};
  a.a_src = (const char*)act;
  a.a_scales = act_scales;
  a.w = (const char*)w2;
  a.w_scales = w2_scales;
  a.sorted_slots = sorted_slots;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.topk_w = topk_w;
  a.out = slot_out;
  a.out_scales = nullptr;
  a.K = r.I;
  a.n_out = r.H;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  a.tiles_max = (int)r.tiles_max;
  a.w_expert_elems = (int64_t)r.H * r.I;
  if (r.w_dtype == MOE_E4M3) return dispatch_bm<OpE4M3, 128, false, OUT_BF16>(r, a, s);
  if (r.w_dtype == MOE_BF16) return dispatch_bm<OpBf16, 64, false, OUT_BF16>(r, a, s);
  return dispatch_bm<OpF32, 32, false, OUT_F32>(r, a, s);
}

}  // namespace moe
