// Weight-streaming grouped GEMMs (decode-size m-blocks of bf16, and the e4m3 workload):
// gfx950 MFMA 16x16 tiles fed by a direct-to-LDS k-slice ring.
//
//   up   : act[r, n]      = SiLU(W13[e,n,:].x_r) * (W13[e,I+n,:].x_r),  x_r = X[sorted_slots[r] / top_k]
//   down : slot_out[s, h] = w[s] * (W2[e,h,:].act[r,:]),                 s = sorted_slots[r]
//
// Same computation as the generic tile kernel (moe_gemm.hip; sources cited there), shaped
// for the case where the weights dominate the bytes: every weight byte is read from HBM
// once (one m-block per expert at these block sizes), so the kernel is bound by HBM and
// its job is to keep enough bytes in flight.
//   * one m-block (BM rows) x BNA output columns per workgroup (up: BNA gate rows plus the
//     matching BNA up rows of W13), 4 waves side by side along N;
//   * 128-byte k-slices (64 bf16 or 128 e4m3 values per row) copied with
//     global_load_lds_dwordx4 into an NS-stage LDS ring (NS-1 slices in flight), XOR-swizzled
//     so the 16x16 fragment reads are bank-conflict free;
//   * e4m3 ("MOE Bmm1 Fused Gather": pack_e4m3x2 rounds to nearest even and saturates): a
//     slice is exactly one 128-wide scale block, so each slice's MFMA products are scaled by
//     (row scale x weight block scale) into the fp32 accumulators.  Row scales travel with the
//     slice (one dword copy per wave); weight block scales are scalar loads.  The up epilogue
//     quantises act per (row, 128-column group) with an LDS amax across the 4 waves;
//   * the barrier of slice kt+1 sits after the last fragment reads of slice kt, so the stage
//     of slice kt is refilled at once and the next slice's first reads overlap the MFMAs.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace st {

constexpr int kGroupM = 4;   // m-blocks of one expert that sweep the n-blocks together

constexpr int ROWB = 128;   // bytes per row per k-slice
constexpr int WN = 4;       // waves side by side along N (times WM waves along M)

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// All-zero row read by padding slots (largest K: kMaxDim bf16 values).
__device__ __attribute__((aligned(16))) char g_zero_row[2 * kMaxDim];

struct Args {
  const char* a_src;          // up: X or its e4m3 codes [T, K]; down: act [rows_max, K]
  const float* a_scales;      // e4m3: up x_scales [T, K/128]; down act_scales [rows, K/128]
  const char* w;              // up: W13 [E, 2I, K]; down: W2 [E, H, K]
  const float* w_scales;      // e4m3: [E, w_rows/128, K/128]
  const int32_t* sorted_slots;
  const int32_t* offsets;
  const int32_t* tiles;
  const int32_t* num_tiles;
  const float* topk_w;        // down
  void* out;                  // up: act [rows_max, n_out]; down: slot_out [N, n_out]
  float* out_scales;          // up e4m3: act_scales [rows_max, n_out/128]
  int K, n_out, top_k, n_slots, tiles_max;
  int64_t w_expert_elems;
};

template <class Op, int BM, int BNA, int NS, bool UP, int OUT, int WM>
__global__ __launch_bounds__(WN * WM * kWave) void stream_kernel(Args g) {
  constexpr bool SCALED = std::is_same<Op, OpE4M3>::value;
  constexpr int BK = ROWB / Op::ELT;             // values per row per slice
  constexpr int KK = BK / Op::KPM;               // MFMA k-steps per slice
  constexpr int STEPB = Op::KPM * Op::ELT;       // bytes per row per k-step
  constexpr int BROWS = UP ? 2 * BNA : BNA;
  constexpr int WTN = BNA / WN;
  constexpr int NW = WN * WM;                    // waves
  constexpr int NT = NW * kWave;
  constexpr int FM = BM / 16;                    // 16-row fragments of the m-block ...
  constexpr int FMW = FM / WM;                   // ... of which wave row wm holds wm, wm+WM, ...
  constexpr int FN = WTN / 16;
  constexpr int NF = UP ? 2 * FN : FN;
  constexpr int NQ_REAL = (BM + BROWS) * ROWB / 1024;   // 1 KB copies (8 rows) per slice
  constexpr int NQ = (NQ_REAL + NW - 1) / NW * NW;      // padded to whole waves
  constexpr int NQW = NQ / NW;
  constexpr int SC_OFF = NQ * 1024;                     // row scales: one dword copy per wave
  constexpr int STAGE = SC_OFF + (SCALED ? NW * 256 : 0);
  constexpr int OPS = NQW + (SCALED ? 1 : 0);           // copies per wave per slice
  static_assert((BM + BROWS) % 8 == 0 && WTN % 16 == 0, "whole copies and MFMA tiles");
  static_assert(FM % WM == 0, "fragments split evenly over the wave rows");
  static_assert(NS >= 2 && (NS - 1) * OPS <= 63, "vmcnt range");
  static_assert(!SCALED || (KK == 1 && (UP ? BNA == kGroup : BNA % kGroup == 0) &&
                            kGroup % WTN == 0 && BM <= NW * 64),
                "e4m3: one scale block per slice and wave, one act group per up tile");
  static_assert(Op::LB == 16 || Op::LB == 32, "16x16 fragments of one or two 16-byte chunks");

  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave % WN;
  const int wm = wave / WN;

  // ---- tile: expert by expert, groups of kGroupM m-blocks sweep the n-blocks.  At these
  // block sizes an expert usually has about one m-block, so the order is n-block fastest and
  // what workgroups share is the m-block's gathered A rows, which the n-blocks of one m-block
  // (adjacent logical tiles, so on one XCD at the same time) read from that XCD's L2.  An
  // expert with many slots (a hot expert) has many m-blocks; grouping them lets each weight
  // tile serve kGroupM m-blocks from L2 (measured 14-20% faster on such batches). ------------
  const int ntiles = *g.num_tiles;
  const int nblk = g.n_out / BNA;
  const int logical = xcd_logical(blockIdx.x, ntiles * nblk);
  if (logical < 0) return;
  const TileRef tr = grouped_tile<BM, kGroupM>(logical, nblk, g.tiles, g.offsets);
  const int e = tr.e;
  const int row0 = tr.row0;
  const int n0 = tr.nt * BNA;
  const int K = g.K;
  const int KT = K / BK;
  const int KB = K / kGroup;                    // scale blocks along K (e4m3)

  // ---- this wave's copies ------------------------------------------------------------------
  // The gather indices are loaded for every copy (row clamped into the m-block) so that the
  // loads issue together and retire under one wait; weight rows then ignore theirs.
  const char* src[NQW];
  const char* wbase = g.w + (size_t)e * g.w_expert_elems * Op::ELT;
  int slot[NQW];
  #pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = min(wave * NQW + i, NQ_REAL - 1);    // padded tail copies repeat a real one
    const int r = q * 8 + (lane >> 3);
    slot[i] = UP ? g.sorted_slots[row0 + min(r, BM - 1)] : 0;
  }
  #pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = min(wave * NQW + i, NQ_REAL - 1);
    const int r = q * 8 + (lane >> 3);
    const int cc = (lane & 7) ^ swz(r);
    if (r < BM) {
      if (UP) {
        src[i] = (slot[i] < g.n_slots)
                     ? g.a_src + (size_t)(slot[i] / g.top_k) * K * Op::ELT + cc * 16
                     : g_zero_row + cc * 16;
      } else {
        src[i] = g.a_src + (size_t)(row0 + r) * K * Op::ELT + cc * 16;
      }
    } else {
      const int rb = r - BM;
      const int grow = UP ? (rb < BNA ? n0 + rb : g.n_out + n0 + (rb - BNA)) : n0 + rb;
      src[i] = wbase + (size_t)grow * K * Op::ELT + cc * 16;
    }
  }
  const float* sc_src = g.a_scales;             // this lane's row-scale source (e4m3)
  if (SCALED) {
    const int r = min(wave * 64 + lane, BM - 1);   // lanes past the m-block copy a real row
    if (UP) {
      const int s = g.sorted_slots[row0 + r];
      sc_src = g.a_scales + (size_t)((s < g.n_slots) ? s / g.top_k : 0) * KB;
    } else {
      sc_src = g.a_scales + (size_t)(row0 + r) * KB;
    }
  }
  const uint32_t lds_base = lds_u32(lds);
  auto issue = [&](int buf, int kt) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(lds_base + buf * STAGE + wave * NQW * 1024);
    const int koff = kt * ROWB;
    #pragma unroll
    for (int i = 0; i < NQW; ++i) lds_dma16(src[i] + koff, st + i * 1024);
    if (SCALED) {
      const uint32_t ss = __builtin_amdgcn_readfirstlane(lds_base + buf * STAGE + SC_OFF + wave * 256);
      lds_dma4(sc_src + kt, ss);
    }
  };

  // ---- fragments (16x16 MFMA operand: lane holds row lane & 15, bytes
  //      [(lane >> 4) * LB, +LB) of the k-step) ------------------------------------------------
  const int fr = lane & 15;
  const int fsw = swz(fr);                      // fragment bases are multiples of 16 rows
  int off0[KK], off1[KK];
  #pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int c = (kk * STEPB + (lane >> 4) * Op::LB) >> 4;
    off0[kk] = fr * ROWB + ((c ^ fsw) << 4);
    off1[kk] = fr * ROWB + (((c + 1) ^ fsw) << 4);
  }
  int b_row[NF];
  #pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int r = UP ? ((j < FN) ? wn * WTN + j * 16 : BNA + wn * WTN + (j - FN) * 16)
                     : wn * WTN + j * 16;
    b_row[j] = (BM + r) * ROWB;
  }
  using frag = typename Op::frag;
  auto load_frag = [&](const char* p, int kk) -> frag {
    if constexpr (Op::LB == 16) {
      return *reinterpret_cast<const frag*>(p + off0[kk]);
    } else {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(p + off0[kk]);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(p + off1[kk]);
      frag f;
      f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
      f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
      return f;
    }
  };

  // acc[i]: fragment fi(i) = wm + WM * i of the m-block, rows fi(i) * 16 + [0, 16)
  auto fi = [&](int i) { return wm + WM * i; };
  f32x4 acc[FMW][NF];
  #pragma unroll
  for (int i = 0; i < FMW; ++i)
    #pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int fmv = FM;                                 // 16-row fragments holding valid rows (e4m3)
  if constexpr (SCALED) {
    // e4m3: a slice is one k-step and one scale block.  Slices kt+1..kt+NS-2 stay in flight
    // while slice kt is multiplied straight out of its stage; the barrier at the top of each
    // slice both publishes slice kt and retires the stage of slice kt-1 for refilling.
    // The weight-block scales of this tile go to LDS before the ring starts (a compiler-
    // tracked global load inside the loop would wait on the untracked ring copies too,
    // draining the ring every slice): up, the gate and the up row-block (one row of K/128
    // each); down, the BNA/128 row-blocks of the n-block.
    constexpr int NSW = UP ? 2 : BNA / kGroup;
    __shared__ float sws[NSW][kMaxDim / kGroup];
    {
      const int wrows = UP ? 2 * g.n_out : g.n_out;
      const float* se = g.w_scales + (size_t)e * (wrows / kGroup) * KB;
      for (int b = 0; b < NSW; ++b) {
        const int rb = UP ? (b == 0 ? n0 : g.n_out + n0) / kGroup : n0 / kGroup + b;
        for (int i = tid; i < KB; i += NT) sws[b][i] = se[(size_t)rb * KB + i];
      }
    }
    // An m-block holds its expert's rows first and padding after, so 16-row fragments from
    // ceil(valid / 16) on are all padding: their products are skipped (accumulators stay 0).
    {
      const int s_lo = g.sorted_slots[row0 + min(lane, BM - 1)];
      const int s_hi = g.sorted_slots[row0 + min(lane + kWave, BM - 1)];
      const int valid = __popcll(__ballot(lane < BM && s_lo < g.n_slots)) +
                        __popcll(__ballot(lane + kWave < BM && s_hi < g.n_slots));
      fmv = __builtin_amdgcn_readfirstlane((valid + 15) >> 4);
    }
    #pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, min(s, KT - 1));
    int buf = 0;
    for (int kt = 0; kt < KT; ++kt) {
      wait_vmcnt<(NS - 2) * OPS>();                          // this wave's copies of slice kt
      __syncthreads();
      issue(buf == 0 ? NS - 1 : buf - 1, min(kt + NS - 1, KT - 1));   // past the end: repeat, never read
      const char* stg = lds + buf * STAGE;
      const float* sc = reinterpret_cast<const float*>(stg + SC_OFF);
      // up: gate / up block scales; down: the block of this wave's columns
      const float sw_g = UP ? sws[0][kt] : sws[(wn * WTN) / kGroup][kt];
      const float sw_u = UP ? sws[NSW - 1][kt] : sw_g;
      frag bf[NF];
      #pragma unroll
      for (int j = 0; j < NF; ++j) bf[j] = load_frag(stg + b_row[j], 0);
      // every product of the slice first (independent MFMAs back to back), then the scaled
      // accumulation, so no MFMA result is waited for inside the MFMA sequence
      f32x4 part[FMW][NF];
      #pragma unroll
      for (int i = 0; i < FMW; ++i) {
        if (fi(i) >= fmv) break;
        const frag af = load_frag(stg + fi(i) * 16 * ROWB, 0);
        #pragma unroll
        for (int j = 0; j < NF; ++j) part[i][j] = Op::mma(af, bf[j], f32x4{0.f, 0.f, 0.f, 0.f});
      }
      #pragma unroll
      for (int i = 0; i < FMW; ++i) {
        if (fi(i) >= fmv) break;
        const f32x4 sa = *reinterpret_cast<const f32x4*>(sc + fi(i) * 16 + (lane >> 4) * 4);
        #pragma unroll
        for (int j = 0; j < NF; ++j) {
          const float sw = (UP && j >= FN) ? sw_u : sw_g;
          #pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += part[i][j][v] * (sa[v] * sw);
        }
      }
      buf = (buf + 1 == NS) ? 0 : buf + 1;
    }
    wait_vmcnt<0>();
  } else {
    frag a0[FMW], b0[NF], a1[FMW], b1[NF];
    auto read_frags = [&](frag* af, frag* bfr, int buf, int kk) {
      const char* stg = lds + buf * STAGE;
      #pragma unroll
      for (int i = 0; i < FMW; ++i) af[i] = load_frag(stg + fi(i) * 16 * ROWB, kk);
      #pragma unroll
      for (int j = 0; j < NF; ++j) bfr[j] = load_frag(stg + b_row[j], kk);
    };
    auto mfmas = [&](const frag* af, const frag* bfr) {
      #pragma unroll
      for (int i = 0; i < FMW; ++i)
        #pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = Op::mma(af[i], bfr[j], acc[i][j]);
    };
    // One k-step: multiply the fragment set that holds it while reading the next k-step (of
    // this slice, or k-step 0 of the slice in `nbuf`) into the other set.  KK is even, so the
    // set holding k-step kk is fixed by kk's parity.
    static_assert(KK % 2 == 0, "fragment sets alternate within a slice");
    auto step = [&](int kk, int buf, int nbuf) {
      const int nb = (kk + 1 < KK) ? buf : nbuf;
      const int nk = (kk + 1 < KK) ? kk + 1 : 0;
      if (kk & 1) { read_frags(a0, b0, nb, nk); mfmas(a1, b1); }
      else        { read_frags(a1, b1, nb, nk); mfmas(a0, b0); }
    };

    // Slices kt+1..kt+NS-1 in flight; the barrier of slice kt+1 sits after the last fragment
    // reads of slice kt, whose stage is then refilled with slice kt+NS.
    #pragma unroll
    for (int s = 0; s < NS; ++s) issue(s, min(s, KT - 1));
    wait_vmcnt<(NS - 1) * OPS>();
    __syncthreads();
    read_frags(a0, b0, 0, 0);
    int buf = 0;
    for (int kt = 0; kt < KT; ++kt) {
      const int nbuf = (buf + 1 == NS) ? 0 : buf + 1;
      #pragma unroll
      for (int kk = 0; kk < KK - 1; ++kk) step(kk, buf, nbuf);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // all reads of stage buf done
      wait_vmcnt<(NS - 2) * OPS>();                          // this wave's slice kt+1 landed
      __syncthreads();
      issue(buf, min(kt + NS, KT - 1));     // past the last slice: repeat KT-1, never read
      step(KK - 1, buf, nbuf);
      buf = nbuf;
    }
    wait_vmcnt<0>();
  }

  // ---- epilogue: 16x16 result, lane holds column lane & 15, rows (lane >> 4) * 4 + v --------
  const int ocol = lane & 15;
  const int orow = (lane >> 4) * 4;
  if constexpr (UP) {
    float a[FMW][FN][4];
    auto silu_mul = [&](int i) {
      #pragma unroll
      for (int j = 0; j < FN; ++j)
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = acc[i][j][v], up = acc[i][j + FN][v];
          a[i][j][v] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
        }
    };
    if constexpr (OUT == OUT_E4M3) {
      // Fragments from fmv on hold only padding rows, whose accumulators are exactly 0: their
      // codes are 0 and their scales 1 (what amax = 0 gives), stored without the arithmetic.
      // amax of each row over the tile's 128 columns (one activation group), across waves
      __syncthreads();                                   // LDS is free: the ring is drained
      float* red = reinterpret_cast<float*>(lds);
      #pragma unroll
      for (int i = 0; i < FMW; ++i) {
        if (fi(i) >= fmv) break;
        silu_mul(i);
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          float m = 0.0f;
          #pragma unroll
          for (int j = 0; j < FN; ++j) m = fmaxf(m, fabsf(a[i][j][v]));
          #pragma unroll
          for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
          if (ocol == 0) red[wn * BM + fi(i) * 16 + orow + v] = m;
        }
      }
      __syncthreads();
      uint8_t* act = reinterpret_cast<uint8_t*>(g.out);
      #pragma unroll
      for (int i = 0; i < FMW; ++i)
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = fi(i) * 16 + orow + v;
          const size_t rowoff = (size_t)(row0 + m) * g.n_out + n0 + wn * WTN;
          float s = 1.0f;
          if (fi(i) < fmv) {
            float amax = 0.0f;
            #pragma unroll
            for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red[w * BM + m]);
            s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
            // quotient in fp32, then the gfx950 convert (round to nearest even, sign kept);
            // the clamp keeps it within +-448, where the convert saturates nothing and
            // matches f32_to_e4m3 on every value
            #pragma unroll
            for (int j = 0; j < FN; j += 2) {
              const float q0 = fminf(fmaxf(a[i][j][v] / s, -kE4M3Max), kE4M3Max);
              const float q1 =
                  (j + 1 < FN) ? fminf(fmaxf(a[i][j + 1][v] / s, -kE4M3Max), kE4M3Max) : 0.0f;
              const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
              act[rowoff + j * 16 + ocol] = (uint8_t)pk;
              if (j + 1 < FN) act[rowoff + (j + 1) * 16 + ocol] = (uint8_t)(pk >> 8);
            }
          } else {
            #pragma unroll
            for (int j = 0; j < FN; ++j) act[rowoff + j * 16 + ocol] = 0;
          }
          if (wn == 0 && ocol == 0)
            g.out_scales[(size_t)(row0 + m) * (g.n_out / kGroup) + n0 / kGroup] = s;
        }
    } else {
      #pragma unroll
      for (int i = 0; i < FMW; ++i) silu_mul(i);
      #pragma unroll
      for (int i = 0; i < FMW; ++i)
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(g.out) +
                          (size_t)(row0 + fi(i) * 16 + orow + v) * g.n_out + n0 + wn * WTN + ocol;
          #pragma unroll
          for (int j = 0; j < FN; ++j) dst[j * 16] = (uint16_t)f32_to_bf16_bits(a[i][j][v]);
        }
    }
  } else {
    // slots, then routing weights, each batch of loads under one wait
    int sl[FMW][4];
    float wt_[FMW][4];
    #pragma unroll
    for (int i = 0; i < FMW; ++i)
      #pragma unroll
      for (int v = 0; v < 4; ++v) sl[i][v] = g.sorted_slots[row0 + fi(i) * 16 + orow + v];
    #pragma unroll
    for (int i = 0; i < FMW; ++i)
      #pragma unroll
      for (int v = 0; v < 4; ++v) wt_[i][v] = g.topk_w[min(sl[i][v], g.n_slots - 1)];
    #pragma unroll
    for (int i = 0; i < FMW; ++i)
      #pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int s = sl[i][v];
        if (s >= g.n_slots) continue;
        const float wt = wt_[i][v];
        uint16_t* dst = reinterpret_cast<uint16_t*>(g.out) + (size_t)s * g.n_out + n0 + wn * WTN + ocol;
        #pragma unroll
        for (int j = 0; j < FN; ++j) dst[j * 16] = (uint16_t)f32_to_bf16_bits(acc[i][j][v] * wt);
      }
  }
}

template <class Op, int BM, int BNA, int NS, bool UP, int OUT, int WM = 1>
hipError_t run(const Args& a, hipStream_t s) {
  const int64_t grid = ((int64_t)a.tiles_max * (a.n_out / BNA) + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((stream_kernel<Op, BM, BNA, NS, UP, OUT, WM>), dim3((unsigned)grid),
                     dim3(WN * WM * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace st

// bf16 with 16..64-row m-blocks, and e4m3 with any m-block size.
bool stream_supported(const Resolved& r) {
  if (r.w_dtype == MOE_BF16) return r.BM <= 64;
  return r.w_dtype == MOE_E4M3;
}

hipError_t launch_up_stream(const Resolved& r, const void* x, const float* x_scales,
                            const void* w13, const float* w13_scales, const int32_t* sorted_slots,
                            const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                            void* act, float* act_scales, hipStream_t s) {
  st::Args a{};
  a.a_src = (const char*)x;
  a.a_scales = x_scales;
  a.w = (const char*)w13;
  a.w_scales = w13_scales;
  a.sorted_slots = sorted_slots;
  a.offsets = offsets;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.out = act;
  a.out_scales = act_scales;
  a.K = r.H;
  a.n_out = r.I;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  a.tiles_max = (int)r.tiles_max;
  a.w_expert_elems = (int64_t)2 * r.I * r.H;
  if (r.w_dtype == MOE_E4M3) {
    switch (r.BM) {
      case 16: return st::run<OpE4M3, 16, 128, 3, true, OUT_E4M3>(a, s);
      case 32: return st::run<OpE4M3, 32, 128, 3, true, OUT_E4M3, 2>(a, s);
      case 64: return st::run<OpE4M3, 64, 128, 3, true, OUT_E4M3, 2>(a, s);
      default: return st::run<OpE4M3, 128, 128, 3, true, OUT_E4M3, 2>(a, s);
    }
  }
  if (r.I % 128 != 0) {   // I a multiple of 64 only: 64-wide n-blocks
    switch (r.BM) {
      // shallow rings: more workgroups per CU (shard at 1024 tokens: down 0.103 -> 0.070 ms
      // against 5-8 stages)
      case 16: return st::run<OpBf16, 16, 64, 4, true, OUT_BF16>(a, s);
      case 32: return st::run<OpBf16, 32, 64, 4, true, OUT_BF16>(a, s);
      default: return st::run<OpBf16, 64, 64, 3, true, OUT_BF16>(a, s);
    }
  }
  switch (r.BM) {
    // 16-row blocks (decode): 64-wide n-blocks, twice the workgroups (DeepSeek-V3 decode up
    // 2.033 -> 2.001 ms against 128-wide)
    case 16: return st::run<OpBf16, 16, 64, 6, true, OUT_BF16>(a, s);
    case 32: return st::run<OpBf16, 32, 128, 4, true, OUT_BF16>(a, s);
    default: return st::run<OpBf16, 64, 128, 3, true, OUT_BF16>(a, s);
  }
}

hipError_t launch_down_stream(const Resolved& r, const void* act, const float* act_scales,
                              const void* w2, const float* w2_scales, const float* topk_w,
                              const int32_t* sorted_slots, const int32_t* offsets,
                              const int32_t* tiles, const int32_t* num_tiles, void* slot_out,
                              hipStream_t s) {
  st::Args a{};
  a.a_src = (const char*)act;
  a.a_scales = act_scales;
  a.w = (const char*)w2;
  a.w_scales = w2_scales;
  a.sorted_slots = sorted_slots;
  a.offsets = offsets;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.topk_w = topk_w;
  a.out = slot_out;
  a.K = r.I;
  a.n_out = r.H;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  a.tiles_max = (int)r.tiles_max;
  a.w_expert_elems = (int64_t)r.H * r.I;
  if (r.w_dtype == MOE_E4M3 && r.H % 256 == 0 && r.BM >= 64) {
    // 256-wide n-blocks: twice the weight bytes per slice next to the same gathered rows, so
    // more of the ring holds weights in flight
    if (r.BM == 64) return st::run<OpE4M3, 64, 256, 3, false, OUT_BF16, 2>(a, s);
    return st::run<OpE4M3, 128, 256, 3, false, OUT_BF16, 2>(a, s);
  }
  if (r.w_dtype == MOE_E4M3) {
    switch (r.BM) {
      case 16: return st::run<OpE4M3, 16, 128, 4, false, OUT_BF16>(a, s);
      case 32: return st::run<OpE4M3, 32, 128, 4, false, OUT_BF16, 2>(a, s);
      case 64: return st::run<OpE4M3, 64, 128, 4, false, OUT_BF16, 2>(a, s);
      default: return st::run<OpE4M3, 128, 128, 4, false, OUT_BF16, 2>(a, s);
    }
  }
  if (r.H % 256 == 0) {
    switch (r.BM) {
      // 16-row blocks: 128-wide n-blocks and 3 stages, two workgroups per CU (decode down
      // with K = 2048: 1.063 -> 0.999 ms against 256-wide, 4 stages)
      case 16: return st::run<OpBf16, 16, 128, 3, false, OUT_BF16>(a, s);
      case 32: return st::run<OpBf16, 32, 256, 4, false, OUT_BF16>(a, s);
      default: return st::run<OpBf16, 64, 256, 3, false, OUT_BF16>(a, s);
    }
  }
  if (r.H % 128 != 0) {   // H a multiple of 64 only: 64-wide n-blocks
    switch (r.BM) {
      case 16: return st::run<OpBf16, 16, 64, 4, false, OUT_BF16>(a, s);
      case 32: return st::run<OpBf16, 32, 64, 4, false, OUT_BF16>(a, s);
      default: return st::run<OpBf16, 64, 64, 3, false, OUT_BF16>(a, s);
    }
  }
  switch (r.BM) {   // H is a multiple of 128 only
    case 16: return st::run<OpBf16, 16, 128, 4, false, OUT_BF16>(a, s);
    case 32: return st::run<OpBf16, 32, 128, 4, false, OUT_BF16>(a, s);
    default: return st::run<OpBf16, 64, 128, 3, false, OUT_BF16>(a, s);
  }
}

}  // namespace moe
