// MXFP4 x e4m3 grouped up GEMM with the GPT-OSS SwiGLU: the first expert GEMM of the
// "MOE Bmm1 Fused Gather" example's own variant (mma_partition: e2m1 weights with 32-wide
// microscales times e4m3 activations; apply_bias_and_scale: acc * x_scale + bias;
// _swiglu_step1/2: (gate, linear) column pairs, gate capped at limit, linear clamped,
// act = gate / (1 + exp(-alpha * gate)) * (linear + 1); pack_fp8_out_fragment: e4m3 of
// act / out_scale, round to nearest even, saturating).
//
//   act[r, c] = e4m3( swiglu( x_scale * (W13[e, 2c, :] . x_r) + bias[e, 2c],
//                             x_scale * (W13[e, 2c+1, :] . x_r) + bias[e, 2c+1] ) / out_scale )
//   x_r = X[sorted_slots[r] / top_k] (e4m3 codes), W13 rows MXFP4 (e2m1 pairs + e8m0 per 32 K)
//
// MI355X shape:
//   * v_mfma_scale_f32_16x16x128_f8f6f4 with the weights as the first operand (format e2m1,
//     the lane's e8m0 microscale as its scale) and the gathered rows as the second (e4m3,
//     scale 1.0; x_scale is applied in the epilogue).  Weight rows on the first operand put
//     four consecutive W13 rows -- two (gate, linear) pairs -- in each lane's result, so the
//     SwiGLU needs no cross-lane exchange.
//     Operand layout (measured): the e2m1 lane (l >> 4) = q holds the 32 values of microscale
//     block q of the 128-value k-step, low nibble first; the e4m3 lane q holds bytes
//     [16q, 16q + 16) and [64 + 16q, 64 + 16q + 16) of the k-step.
//   * KSL 128-value k-steps per slice (one in the dispatched shapes), NS-stage direct-to-LDS
//     ring: per slice BM rows x 128 B of gathered codes, 2*BNA weight rows x 64 B, and the
//     4 x 2*BNA scale bytes of the slice (scales are stored [E, H/32, 2I], so a slice's scales
//     are 4 contiguous runs);
//   * K need only be a multiple of 64: copies of chunks past K read a static zero area (only
//     the last slice can hold such chunks; the copies of the slices before it advance a
//     pointer per slice and check nothing);
//   * tile order: expert by expert, groups of 4 m-blocks sweep the n-blocks; padding rows
//     read zeros and their 16-row fragments are skipped; their act rows are not written;
//   * epilogue in fp32 with the gfx950 units: exp through v_exp_f32 (__expf) and the
//     reciprocal v_rcp_f32 for the SwiGLU's division, a multiply by 1/out_scale, and the
//     e4m3 convert (v_cvt_pk_fp8_f32, round to nearest even) after a clamp to +-448.  Each of
//     these is within a few ulp of the correctly rounded fp32 operation, so a code can move
//     by one step only for a value within that distance of a rounding midpoint, which the
//     fp32 accumulation order already does against the oracle.
#include "moe_internal.h"

namespace moe {

namespace mx {

constexpr int KM = 128;            // K values per MFMA k-step
constexpr int kGroupM = 4;
constexpr int kWN = 4;             // default waves along the weight rows (times WM along the m-block)

__device__ __attribute__((aligned(16))) char g_zero[256];

// 16-byte chunk swizzle of rows of RB bytes: chunk c of row r sits at c ^ swz<RB>(r), which
// puts the fragment reads (16 consecutive rows at one chunk) in 16 distinct 4-bank groups.
// For 64-byte rows ((r >> 1) ^ (r >> 2)) & 3 also keeps every 8 consecutive rows in 8 distinct
// groups of a 32-bank view ((r >> 2) & 3 alone does not; measured 1-5% faster).
template <int RB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (RB == 64) return ((r >> 1) ^ (r >> 2)) & 3;
  else if constexpr (RB == 128) return (r & 7) ^ ((r >> 3) & 1);
  else return r & 15;
}

struct Args {
  const uint8_t* x;              // [T, K] e4m3 codes
  const float* x_scale;          // [1]
  const uint8_t* w;              // [E, 2I, K/2] e2m1 pairs
  const uint8_t* w_scales;       // [E, K/32, 2I] e8m0
  const float* bias;             // [E, 2I]
  const float* out_scale;        // [1]
  const int32_t* sorted_slots;
  const int32_t* offsets;
  const int32_t* tiles;
  const int32_t* num_tiles;
  uint8_t* act;                  // [rows_max, I] e4m3 codes
  float alpha, limit;
  int K, I, top_k, n_slots;
};

template <int BM, int BNA, int NS, int WM, int KSL, int WN>
__global__ __launch_bounds__(WN * WM * kWave) void mx_up_kernel(Args g) {
  constexpr int KS = KSL * KM;                     // K values per slice
  constexpr int XB = KS;                           // gathered-code bytes per row per slice
  constexpr int WB = KS / 2;                       // weight bytes per row per slice
  constexpr int SB = KS / 32;                      // scale bytes per weight row per slice
  constexpr int XR = 1024 / XB;                    // rows per 1 KB copy
  constexpr int WR = 1024 / WB;
  constexpr int NW = WN * WM;
  constexpr int WROWS = 2 * BNA;                   // weight rows of the tile
  constexpr int WTW = WROWS / WN;                  // weight rows per wave
  constexpr int FW = WTW / 16;
  constexpr int FM = BM / 16;
  constexpr int FMW = FM / WM;
  constexpr int NQ_X = BM * XB / 1024;             // 1 KB copies per slice
  constexpr int NQ_W = WROWS * WB / 1024;
  constexpr int NQ = NQ_X + NQ_W;
  constexpr int NQW = (NQ + NW - 1) / NW;          // per wave; padded slots repeat a real copy
  constexpr int NS_REAL = SB * WROWS / 256;        // 256-byte scale copies per slice
  constexpr int NSW = (NS_REAL + NW - 1) / NW;
  constexpr int OPS = NQW + NSW;
  constexpr int W_OFF = BM * XB;
  constexpr int S_OFF = W_OFF + WROWS * WB;
  constexpr int STAGE = S_OFF + SB * WROWS;
  static_assert(BM % 16 == 0 && FM % WM == 0 && WTW % 16 == 0, "whole MFMA tiles");
  static_assert((SB * WROWS) % 256 == 0 && BM % XR == 0 && NQ_X >= 1, "whole copies");
  static_assert(NS >= 2 && (NS - 1) * OPS <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave % WN;
  const int wm = wave / WN;

  const int ntiles = *g.num_tiles;
  const int nblk = g.I / BNA;
  const int logical = xcd_logical(blockIdx.x, ntiles * nblk);
  if (logical < 0) return;
  const TileRef tr = grouped_tile<BM, kGroupM>(logical, nblk, g.tiles, g.offsets);
  const int e = tr.e;
  const int row0 = tr.row0;
  const int n0 = tr.nt * BNA;                         // first act column; weight rows from 2*n0
  const int K = g.K;
  const int KT = (K + KS - 1) / KS;
  const int KB = K / 32;                           // microscale blocks per row
  const int I2 = 2 * g.I;

  // ---- copies: source of this lane for slice 0, its per-slice byte step, the K offset of
  // its chunk inside a slice (chunks at or past K read zeros), and whether it is live --------
  const char* src[NQW];
  int step[NQW], kof[NQW];
  bool live[NQW];
  #pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = min(wave * NQW + i, NQ - 1);
    if (q < NQ_X) {                                // gathered rows: XR per copy
      const int r = q * XR + lane / (XB / 16);
      const int c = (lane % (XB / 16)) ^ swz<XB>(r);
      const int s = g.sorted_slots[row0 + r];
      live[i] = s < g.n_slots;
      src[i] = reinterpret_cast<const char*>(g.x) + (size_t)(live[i] ? s / g.top_k : 0) * K + c * 16;
      step[i] = XB;
      kof[i] = c * 16;
    } else {                                       // weight rows: WR per copy
      const int r = (q - NQ_X) * WR + lane / (WB / 16);
      const int c = (lane % (WB / 16)) ^ swz<WB>(r);
      live[i] = true;
      src[i] = reinterpret_cast<const char*>(g.w) +
               ((size_t)e * I2 + 2 * n0 + r) * (size_t)(K / 2) + c * 16;
      step[i] = WB;
      kof[i] = c * 32;
    }
  }
  const char* ssrc[NSW];
  int skb[NSW];
  #pragma unroll
  for (int i = 0; i < NSW; ++i) {
    const int q = min(wave * NSW + i, NS_REAL - 1);
    const int b = q * 256 + lane * 4;              // byte of the slice's [SB][WROWS] scale block
    skb[i] = b / WROWS;
    ssrc[i] = reinterpret_cast<const char*>(g.w_scales) +
              ((size_t)e * KB + skb[i]) * I2 + 2 * n0 + (b % WROWS);
  }
  // Slices before KT_full hold no chunk at or past K: their copies read live rows (padding
  // rows read the zero area with no step) from a pointer advanced by one step per slice; the
  // last slice of a K that is not a whole number of slices checks each chunk.
  const int KT_full = K / KS;
  const char* cur[NQW];
  int cstep[NQW];
  uint32_t cdst[NQW];
  #pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = min(wave * NQW + i, NQ - 1);
    cur[i] = live[i] ? src[i] : reinterpret_cast<const char*>(g_zero);
    cstep[i] = live[i] ? step[i] : 0;
    cdst[i] = q < NQ_X ? q * 1024 : W_OFF + (q - NQ_X) * 1024;
  }
  const char* scur[NSW];
  #pragma unroll
  for (int i = 0; i < NSW; ++i) scur[i] = ssrc[i];
  const uint32_t lds_base = lds_u32(lds);
  // copies of slice kt (called with kt = 0, 1, 2, ... in order, then KT for past the end)
  auto issue = [&](int buf, int kt) {
    const uint32_t st = lds_base + buf * STAGE;
    if (kt < KT_full) {
      #pragma unroll
      for (int i = 0; i < NQW; ++i) {
        lds_dma16(cur[i], __builtin_amdgcn_readfirstlane(st + cdst[i]));
        cur[i] += cstep[i];
      }
      #pragma unroll
      for (int i = 0; i < NSW; ++i) {
        const int q = min(wave * NSW + i, NS_REAL - 1);
        lds_dma4(scur[i], __builtin_amdgcn_readfirstlane(st + S_OFF + q * 256));
        scur[i] += (size_t)SB * I2;
      }
    } else {
      const int k0 = kt * KS;
      #pragma unroll
      for (int i = 0; i < NQW; ++i) {
        const bool ok = live[i] && k0 + kof[i] < K;
        lds_dma16(ok ? src[i] + (size_t)kt * step[i] : reinterpret_cast<const char*>(g_zero),
                  __builtin_amdgcn_readfirstlane(st + cdst[i]));
      }
      #pragma unroll
      for (int i = 0; i < NSW; ++i) {
        const int q = min(wave * NSW + i, NS_REAL - 1);
        const bool ok = SB * kt + skb[i] < KB;
        lds_dma4(ok ? ssrc[i] + (size_t)kt * SB * I2 : reinterpret_cast<const char*>(g_zero),
                 __builtin_amdgcn_readfirstlane(st + S_OFF + q * 256));
      }
    }
  };

  // ---- fragments -----------------------------------------------------------------------------
  const int fr = lane & 15;
  const int fq = lane >> 4;
  // weights, k-step kk: row wn*WTW + f*16 + fr, chunk 4kk + fq (16 bytes = microscale block
  // 4kk + fq of the slice); the swizzle of a fragment's rows depends on fr only
  const int sw_w = swz<WB>(fr), sw_x = swz<XB>(fr);
  int w_off[FW], s_off[FW];
  #pragma unroll
  for (int f = 0; f < FW; ++f) {
    const int r = wn * WTW + f * 16 + fr;
    w_off[f] = W_OFF + r * WB;
    s_off[f] = S_OFF + fq * WROWS + r;
  }
  // gathered codes, k-step kk: row fi(i)*16 + fr, chunks 8kk + fq and 8kk + 4 + fq
  auto fi = [&](int i) { return wm + WM * i; };
  int x_off[FMW];
  #pragma unroll
  for (int i = 0; i < FMW; ++i) x_off[i] = (fi(i) * 16 + fr) * XB;

  // 16-row fragments from ceil(valid / 16) on are all padding: skipped
  int fmv;
  {
    int valid = 0;
    #pragma unroll
    for (int r0 = 0; r0 < BM; r0 += kWave)
      valid += __popcll(__ballot(r0 + lane < BM && g.sorted_slots[row0 + min(r0 + lane, BM - 1)] < g.n_slots));
    fmv = __builtin_amdgcn_readfirstlane((valid + 15) >> 4);
  }

  f32x4 acc[FW][FMW];
  #pragma unroll
  for (int f = 0; f < FW; ++f)
    #pragma unroll
    for (int i = 0; i < FMW; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Slices kt+1..kt+NS-2 in flight; the barrier at the top of slice kt publishes it and
  // retires the stage of slice kt-1, which is refilled at once.
  #pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s < KT ? s : KT);
  int buf = 0;
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<(NS - 2) * OPS>();
    __syncthreads();
    // past the end: a slice of zero chunks (the checked path), never read
    issue(buf == 0 ? NS - 1 : buf - 1, kt + NS - 1 < KT ? kt + NS - 1 : KT);
    const char* stg = lds + buf * STAGE;
    #pragma unroll
    for (int kk = 0; kk < KSL; ++kk) {
      i32x8 wf[FW];
      int sc[FW];
      #pragma unroll
      for (int f = 0; f < FW; ++f) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(stg + w_off[f] + (((4 * kk + fq) ^ sw_w) << 4));
        wf[f] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        sc[f] = *reinterpret_cast<const uint8_t*>(stg + s_off[f] + 4 * kk * WROWS);
      }
      #pragma unroll
      for (int i = 0; i < FMW; ++i) {
        if (fi(i) >= fmv) break;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(stg + x_off[i] + (((8 * kk + fq) ^ sw_x) << 4));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(stg + x_off[i] + (((8 * kk + 4 + fq) ^ sw_x) << 4));
        const i32x8 xf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        #pragma unroll
        for (int f = 0; f < FW; ++f)
          acc[f][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[f], xf, acc[f][i], 4, 0,
                                                                       0, sc[f], 0, 127);
      }
    }
    buf = (buf + 1 == NS) ? 0 : buf + 1;
  }
  wait_vmcnt<0>();

  // ---- epilogue: lane holds weight rows 4*fq + v (v = 0..3) of fragment f for token fr:
  // (gate, linear) of act column c and of column c + 1 -----------------------------------------
  const float xs = *g.x_scale;
  const float inv_ys = 1.0f / *g.out_scale;
  bool row_ok[FMW];
  #pragma unroll
  for (int i = 0; i < FMW; ++i) row_ok[i] = g.sorted_slots[row0 + min(fi(i) * 16 + fr, BM - 1)] < g.n_slots;
  #pragma unroll
  for (int f = 0; f < FW; ++f) {
    const int wr = 2 * n0 + wn * WTW + f * 16 + 4 * fq;   // first of this lane's 4 weight rows
    const f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + (size_t)e * I2 + wr);
    const int c = wr / 2;
    #pragma unroll
    for (int i = 0; i < FMW; ++i) {
      if (fi(i) >= fmv) break;
      const int m = fi(i) * 16 + fr;
      if (!row_ok[i]) continue;
      float q[2];
      #pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float h_g = fmaf(acc[f][i][2 * p], xs, b[2 * p]);
        const float h_l = fmaf(acc[f][i][2 * p + 1], xs, b[2 * p + 1]);
        const float gt = fminf(h_g, g.limit);
        const float ln = fminf(fmaxf(h_l, -g.limit), g.limit);
        const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-g.alpha * gt));
        // act / out_scale, clamped to +-448 (the convert then saturates nothing), converted
        // with round to nearest even
        q[p] = fminf(fmaxf(fmaf(a, ln, a) * inv_ys, -kE4M3Max), kE4M3Max);
      }
      const uint32_t codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      *reinterpret_cast<uint16_t*>(g.act + (size_t)(row0 + m) * g.I + c) = (uint16_t)codes;
    }
  }
}

template <int BM, int BNA, int NS, int WM, int KSL, int WN = kWN>
hipError_t run(const Args& a, int64_t tiles_max, hipStream_t s) {
  if (a.I % BNA) return hipErrorInvalidValue;
  const int64_t grid = (tiles_max * (a.I / BNA) + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((mx_up_kernel<BM, BNA, NS, WM, KSL, WN>), dim3((unsigned)grid), dim3(WN * WM * kWave),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace mx

hipError_t launch_up_mxfp4(const Resolved& r, const uint8_t* x, const float* x_scale,
                           const uint8_t* w13, const uint8_t* w13_scales, const float* bias,
                           float alpha, float limit, const float* out_scale,
                           const int32_t* sorted_slots, const int32_t* offsets,
                           const int32_t* tiles, const int32_t* num_tiles, uint8_t* act,
                           hipStream_t s) {
  mx::Args a{};
  a.x = x;
  a.x_scale = x_scale;
  a.w = w13;
  a.w_scales = w13_scales;
  a.bias = bias;
  a.out_scale = out_scale;
  a.sorted_slots = sorted_slots;
  a.offsets = offsets;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.act = act;
  a.alpha = alpha;
  a.limit = limit;
  a.K = r.H;
  a.I = r.I;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  // Three-stage rings of 128-row weight tiles for every block size: occupancy wins here.
  // Measured on the GPT-OSS shard: two to five workgroups per CU beat deeper rings (6 stages:
  // 25% slower at 640 tokens), 256-value slices, and 384-row weight tiles with one workgroup
  // per CU (5-17% slower at 2048-31744 tokens).
  switch (r.BM) {
    case 16: return mx::run<16, 64, 3, 1, 1>(a, r.tiles_max, s);
    case 32: return mx::run<32, 64, 3, 1, 1>(a, r.tiles_max, s);
    case 64: return mx::run<64, 64, 3, 2, 1>(a, r.tiles_max, s);
    // 128-row blocks: 2 x 4 waves (64 weight rows x 32 gathered rows each) read 8 KB of
    // fragments per 8 MFMAs where 4 x 2 waves read 10 KB: 2-5% faster, the loop being bound by
    // LDS reads (each gathered fragment is read by every wave column)
    default: return mx::run<128, 64, 3, 4, 1, 2>(a, r.tiles_max, s);
  }
}

}  // namespace moe
