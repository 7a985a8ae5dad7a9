// bf16 grouped GEMMs for 128-row m-blocks (prefill): gfx950 MFMA 32x32x16.
//
//   up   : act[r, n]      = SiLU(W13[e,n,:].x_r) * (W13[e,I+n,:].x_r),  x_r = X[sorted_slots[r] / top_k]
//   down : slot_out[s, h] = w[s] * (W2[e,h,:].act[r,:]),                 s = sorted_slots[r]
//
// Same computation as the generic tile kernel (moe_gemm.hip; sources cited there:
// "MOE Bmm1 Fused Gather" load_activations / SwiGLU epilogue, "moe triton kernel use
// tma." MUL_ROUTED_WEIGHT, "factor_moe_fused_gemm.cu" gate-first SiLU), shaped for
// large per-expert row counts on MI355X:
//   * v_mfma_f32_32x32x16_bf16 -- on gfx950 it sustains the dense bf16 rate, the
//     16x16x32 form only about half of it;
//   * one 128-row m-block x BNA output columns per workgroup (up: BNA gate rows plus
//     the matching BNA up rows of W13), 4 waves side by side along N, each wave
//     128 rows x (up: BNA/4 gate + BNA/4 up | down: BNA/4) columns.  Wide tiles keep
//     the L2->CU bytes per flop low (L2 hits cost about a microsecond under load, so
//     bytes in flight, not peak bandwidth, bound a narrow tile) and the LDS traffic
//     per MFMA below what the LDS sustains;
//   * k-slices of BK = 32 (64 bytes per row) in two LDS stages without padding: the
//     16-byte chunk c of row r sits at position c ^ (((r >> 1) ^ (r >> 3)) & 3) (for
//     128-byte rows c ^ ((r & 7) ^ ((r >> 3) & 1))), conflict-free for the fragment
//     reads (16 consecutive rows at one k offset) and for the row-wise writes;
//   * global loads run two k-slices ahead through two register sets: slice kt+2 is
//     requested before slice kt is multiplied, slice kt+1 (requested one slice earlier)
//     is written to the free LDS stage after the multiply;
//   * fragment reads of the next 16-wide k step overlap the MFMAs of the current one;
//   * tile order: expert by expert, groups of 8 m-blocks of one expert sweep the n-blocks,
//     and each XCD (own L2) runs a contiguous range of that order, so concurrent workgroups
//     share rows and weights and each weight tile leaves HBM about once.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace pf {

constexpr int BM = 128;        // rows per m-block
constexpr int GROUP_M = 8;     // m-blocks that sweep the n-blocks together

// One all-zero bf16 row of the largest supported K (kMaxDim): the padding rows of an
// m-block (sentinel slots) read it instead of a token row, so the gathered loads need
// no select -- a select right after a load makes the compiler wait for that load.
__device__ __attribute__((aligned(16))) char g_zero_row[2 * kMaxDim];

template <int ROWB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (ROWB == 128) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

// Logical tile order, expert by expert: inside expert e (m-blocks base..base+M-1) groups of
// GROUP_M m-blocks sweep the n-blocks, n-block-major inside a group.  A group never holds two
// experts, so one XCD's concurrent workgroups share their weight tiles (each fetched once) and
// their gathered rows.  logical / n_blocks is an m-block of the expert that owns `logical`.
template <int BMT>
__device__ __forceinline__ void tile_of(int logical, int n_blocks, const int32_t* tiles,
                                        const int32_t* offsets, int& mt, int& nt) {
  const int e = tiles[2 * (logical / n_blocks)];
  const int base = offsets[e] / BMT;
  const int M = (offsets[e + 1] - offsets[e]) / BMT;
  const int r = logical - base * n_blocks;          // 0 <= r < M * n_blocks
  const int full = M / GROUP_M;
  if (r < full * GROUP_M * n_blocks) {
    const int g = r / (GROUP_M * n_blocks), w = r - g * GROUP_M * n_blocks;
    nt = w / GROUP_M;
    mt = base + g * GROUP_M + (w - nt * GROUP_M);
  } else {
    const int rem = M - full * GROUP_M, w = r - full * GROUP_M * n_blocks;
    nt = w / rem;
    mt = base + full * GROUP_M + (w - nt * rem);
  }
}

struct Args {
  const char* a_src;        // up: X [T, K]; down: act [rows_max, K]   (bf16)
  const char* w;            // up: W13 [E, 2I, K]; down: W2 [E, H, K]  (bf16)
  const int32_t* sorted_slots;
  const int32_t* offsets;
  const int32_t* tiles;
  const int32_t* num_tiles;
  const float* topk_w;      // down
  uint16_t* out;            // up: act [rows_max, I]; down: slot_out [N, H]  (bf16 bits)
  int K, n_out, top_k, n_slots, tiles_max;
  int64_t w_expert_elems;
};

template <int BK, int WM, int WN, int BNA, bool UP>
__global__ __launch_bounds__(WM* WN* kWave) void gemm_kernel(Args g) {
  constexpr int NT = WM * WN * kWave;
  constexpr int ROWB = BK * 2;                  // bytes of one row's k-slice
  constexpr int CPR = ROWB / 16;                // 16-byte chunks per row slice
  constexpr int KK = BK / 16;                   // MFMA k-steps per slice
  constexpr int BROWS = UP ? 2 * BNA : BNA;     // weight rows per stage
  constexpr int WTM = BM / WM;                  // wave tile rows
  constexpr int WTN = BNA / WN;                 // wave tile output columns
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int NF = UP ? 2 * FN : FN;
  constexpr int A_PT = BM * CPR / NT;           // 16-byte chunks per thread per stage
  constexpr int B_PT = BROWS * CPR / NT;
  constexpr int STAGE = (BM + BROWS) * ROWB;
  static_assert(BM * CPR % NT == 0 && BROWS * CPR % NT == 0, "whole chunks per thread");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole 32x32 MFMA tiles");

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  const int nblk = g.n_out / BNA;
  const int logical = xcd_logical(blockIdx.x, *g.num_tiles * nblk);
  if (logical < 0) return;
  int mt, nt;
  tile_of<BM>(logical, nblk, g.tiles, g.offsets, mt, nt);
  const int e = g.tiles[2 * mt];
  const int row0 = g.tiles[2 * mt + 1];
  const int n0 = nt * BNA;
  const int K = g.K;
  const int KT = K / BK;                         // even: K is a multiple of 128

  // ---- per-thread global sources and LDS destinations (fixed over k) ---------------------
  const char* a_ptr[A_PT];
  int a_dst[A_PT];
  #pragma unroll
  for (int i = 0; i < A_PT; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    a_dst[i] = r * ROWB + ((cc ^ swz<ROWB>(r)) << 4);
    if (UP) {
      const int s = g.sorted_slots[row0 + r];
      a_ptr[i] = (s < g.n_slots) ? g.a_src + (size_t)(s / g.top_k) * K * 2 + cc * 16
                                 : g_zero_row + cc * 16;
    } else {
      a_ptr[i] = g.a_src + (size_t)(row0 + r) * K * 2 + cc * 16;
    }
  }
  const char* wbase = g.w + (size_t)e * g.w_expert_elems * 2;
  const char* b_ptr[B_PT];
  int b_dst[B_PT];
  #pragma unroll
  for (int i = 0; i < B_PT; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    b_dst[i] = (BM + r) * ROWB + ((cc ^ swz<ROWB>(r)) << 4);
    const int grow = UP ? (r < BNA ? n0 + r : g.n_out + n0 + (r - BNA)) : n0 + r;
    b_ptr[i] = wbase + (size_t)grow * K * 2 + cc * 16;
  }

  i32x4 ra0[A_PT], rb0[B_PT], ra1[A_PT], rb1[B_PT];
  auto gload = [&](i32x4* ra, i32x4* rb, int kt) {
    const int koff = kt * ROWB;
    #pragma unroll
    for (int i = 0; i < A_PT; ++i) ra[i] = *reinterpret_cast<const i32x4*>(a_ptr[i] + koff);
    #pragma unroll
    for (int i = 0; i < B_PT; ++i) rb[i] = *reinterpret_cast<const i32x4*>(b_ptr[i] + koff);
  };
  auto sstore = [&](const i32x4* ra, const i32x4* rb, int buf) {
    char* st = lds + buf * STAGE;
    #pragma unroll
    for (int i = 0; i < A_PT; ++i) *reinterpret_cast<i32x4*>(st + a_dst[i]) = ra[i];
    #pragma unroll
    for (int i = 0; i < B_PT; ++i) *reinterpret_cast<i32x4*>(st + b_dst[i]) = rb[i];
  };

  // ---- fragment addressing --------------------------------------------------------------
  // 32x32x16 operand: lane holds row (lane & 31), 8 consecutive k at chunk 2*kk + (lane >> 5).
  // Fragment bases are multiples of 32 rows, so the swizzle depends on lane & 31 only.
  const int fr = lane & 31;
  const int fsw = swz<ROWB>(fr);
  const int fq = lane >> 5;
  int lane_off[KK];
  #pragma unroll
  for (int kk = 0; kk < KK; ++kk) lane_off[kk] = fr * ROWB + (((2 * kk + fq) ^ fsw) << 4);
  int a_row[FM], b_row[NF];
  #pragma unroll
  for (int i = 0; i < FM; ++i) a_row[i] = (wm * WTM + i * 32) * ROWB;
  #pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int r = UP ? ((j < FN) ? wn * WTN + j * 32 : BNA + wn * WTN + (j - FN) * 32)
                     : wn * WTN + j * 32;
    b_row[j] = (BM + r) * ROWB;
  }

  f32x16 acc[FM][NF];
  #pragma unroll
  for (int i = 0; i < FM; ++i)
    #pragma unroll
    for (int j = 0; j < NF; ++j)
      #pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Instruction order inside one k-slice region (hints to the scheduler): fragments of
  // k-step 0, then each k-step's MFMAs interleaved with the next k-step's fragment reads
  // and the next slices' global loads; the LDS writes of the next slice ride along the
  // last k-step.
  auto schedule = [&]() {
    constexpr int MF = FM * NF;           // MFMAs per k-step
    constexpr int RD = FM + NF;           // fragment reads per k-step
    constexpr int GL = A_PT + B_PT;       // global loads (and LDS writes) per slice
    constexpr int GL_PER = (GL + KK - 2) / (KK - 1 > 0 ? KK - 1 : 1);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
    #pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
      #pragma unroll
      for (int q = 0; q < MF; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q < GL_PER) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    #pragma unroll
    for (int q = 0; q < MF; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < GL) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
  };

  auto compute = [&](int buf) {
    const char* st = lds + buf * STAGE;
    bf16x8 af[2][FM], bfr[2][NF];
    #pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(st + a_row[i] + lane_off[0]);
    #pragma unroll
    for (int j = 0; j < NF; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8*>(st + b_row[j] + lane_off[0]);
    #pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk + 1 < KK) {
        #pragma unroll
        for (int i = 0; i < FM; ++i)
          af[nxt][i] = *reinterpret_cast<const bf16x8*>(st + a_row[i] + lane_off[kk + 1]);
        #pragma unroll
        for (int j = 0; j < NF; ++j)
          bfr[nxt][j] = *reinterpret_cast<const bf16x8*>(st + b_row[j] + lane_off[kk + 1]);
      }
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int j = 0; j < NF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- main loop: slice kt in LDS, kt+1 in flight in one register set, kt+2 requested --------
  gload(ra0, rb0, 0);
  sstore(ra0, rb0, 0);
  gload(ra1, rb1, 1);
  __syncthreads();
  for (int kt = 0; kt < KT; kt += 2) {
    // even slice kt: LDS stage 0; slice kt+1 arrives in set 1; request kt+2 into set 0
    // (past the last slice the requests repeat slice KT-1: in bounds, never consumed)
    gload(ra0, rb0, min(kt + 2, KT - 1));
    compute(0);
    sstore(ra1, rb1, 1);
    schedule();
    __syncthreads();
    // odd slice kt+1: LDS stage 1; slice kt+2 arrives in set 0; request kt+3 into set 1
    gload(ra1, rb1, min(kt + 3, KT - 1));
    compute(1);
    sstore(ra0, rb0, 0);
    schedule();
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------------------
  // 32x32 result: lane holds column lane & 31 and rows 8*(v/4) + 4*(lane>>5) + (v&3), v < 16.
  const int ocol = lane & 31;
  const int orow = 4 * (lane >> 5);
  if (UP) {
    #pragma unroll
    for (int i = 0; i < FM; ++i)
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * WTM + i * 32 + 8 * (v >> 2) + orow + (v & 3);
        uint16_t* dst = g.out + (size_t)(row0 + m) * g.n_out + n0 + wn * WTN + ocol;
        #pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float gt = acc[i][j][v], up = acc[i][j + FN][v];
          const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
          dst[j * 32] = (uint16_t)f32_to_bf16_bits(a);
        }
      }
  } else {
    #pragma unroll
    for (int i = 0; i < FM; ++i)
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * WTM + i * 32 + 8 * (v >> 2) + orow + (v & 3);
        const int s = g.sorted_slots[row0 + m];
        if (s >= g.n_slots) continue;
        const float wt = g.topk_w[s];
        uint16_t* dst = g.out + (size_t)s * g.n_out + n0 + wn * WTN + ocol;
        #pragma unroll
        for (int j = 0; j < FN; ++j) dst[j * 32] = (uint16_t)f32_to_bf16_bits(acc[i][j][v] * wt);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Direct-to-LDS variant: the global -> LDS copies are global_load_lds_dwordx4 (each wave
// instruction lands 64 x 16 bytes contiguously in LDS at M0), so no registers stage the
// k-slices and the LDS ring can hold NS slices, NS-1 of them in flight.  The copies are
// issued from inline assembly with explicit vmcnt waits: the compiler's own tracking of
// LDS DMA waits for every outstanding copy before any LDS read, which would drain the
// ring each k-slice.  The per-lane source address is chosen so that the fixed
// lane -> LDS position mapping realises the same XOR swizzle as above.
// ---------------------------------------------------------------------------------------------
template <int BMT, int BK, int NS, int BNA, bool UP, int WM, int WN>
__global__ __launch_bounds__(WN * WM * kWave) void gemm_dma_kernel(Args g) {
  constexpr int ROWB = BK * 2, KK = BK / 16, NW = WN * WM;
  constexpr int BROWS = UP ? 2 * BNA : BNA;
  constexpr int WTN = BNA / WN;
  constexpr int FM = BMT / 32 / WM;                // 32-row fragments per wave (rows wm*BMT/WM ...)
  constexpr int FN = WTN / 32;
  constexpr int NF = UP ? 2 * FN : FN;
  constexpr int STAGE = (BMT + BROWS) * ROWB;
  constexpr int NQ = STAGE / 1024;                // 1 KB wave copies per slice
  constexpr int NQW = NQ / NW;                    // per wave
  constexpr int ROWS_PER_Q = 1024 / ROWB;
  constexpr int CPR = ROWB / 16;
  static_assert(NQ % NW == 0, "copies split evenly over the waves");
  static_assert(NS >= 2 && (NS - 1) * NQW <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave % WN;
  const int wm = wave / WN;
  const int mrow0 = wm * (BMT / WM);               // this wave's first row of the m-block

  const int nblk = g.n_out / BNA;
  const int logical = xcd_logical(blockIdx.x, *g.num_tiles * nblk);
  if (logical < 0) return;
  int mt, nt;
  tile_of<BMT>(logical, nblk, g.tiles, g.offsets, mt, nt);
  const int e = g.tiles[2 * mt];
  const int row0 = g.tiles[2 * mt + 1];
  const int n0 = nt * BNA;
  const int K = g.K;
  const int KT = K / BK;

  // ---- this wave's copies: source row pointers (k-slice 0) and LDS offsets -----------------
  const char* src[NQW];
  const char* wbase = g.w + (size_t)e * g.w_expert_elems * 2;
  #pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = wave * NQW + i;
    const int r = q * ROWS_PER_Q + lane / CPR;      // row of the stage this lane fills
    const int cc = (lane % CPR) ^ swz<ROWB>(r);      // chunk that belongs at this position
    if (r < BMT) {
      if (UP) {
        const int s = g.sorted_slots[row0 + r];
        src[i] = (s < g.n_slots) ? g.a_src + (size_t)(s / g.top_k) * K * 2 + cc * 16
                                 : g_zero_row + cc * 16;
      } else {
        src[i] = g.a_src + (size_t)(row0 + r) * K * 2 + cc * 16;
      }
    } else {
      const int rb = r - BMT;
      const int grow = UP ? (rb < BNA ? n0 + rb : g.n_out + n0 + (rb - BNA)) : n0 + rb;
      src[i] = wbase + (size_t)grow * K * 2 + cc * 16;
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  auto issue = [&](int buf, int kt) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(lds_base + buf * STAGE + wave * NQW * 1024);
    const int koff = kt * ROWB;
    #pragma unroll
    for (int i = 0; i < NQW; ++i) lds_dma16(src[i] + koff, st + i * 1024);
  };

  // ---- fragments -----------------------------------------------------------------------------
  const int fr = lane & 31;
  const int fsw = swz<ROWB>(fr);
  const int fq = lane >> 5;
  int lane_off[KK];
  #pragma unroll
  for (int kk = 0; kk < KK; ++kk) lane_off[kk] = fr * ROWB + (((2 * kk + fq) ^ fsw) << 4);
  int b_row[NF];
  #pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int r = UP ? ((j < FN) ? wn * WTN + j * 32 : BNA + wn * WTN + (j - FN) * 32)
                     : wn * WTN + j * 32;
    b_row[j] = (BMT + r) * ROWB;
  }

  f32x16 acc[FM][NF];
  #pragma unroll
  for (int i = 0; i < FM; ++i)
    #pragma unroll
    for (int j = 0; j < NF; ++j)
      #pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Rows of the m-block that hold slots come first, padding after: this wave's 32-row
  // fragments from fmv on are all padding, and their reads and MFMAs are skipped.
  int fmv;
  {
    int valid = 0;
    #pragma unroll
    for (int r0 = 0; r0 < BMT; r0 += kWave)
      valid += __popcll(__ballot(g.sorted_slots[row0 + r0 + lane] < g.n_slots));
    fmv = __builtin_amdgcn_readfirstlane(min(FM, max(0, (valid - mrow0 + 31) / 32)));
  }

  // Two fragment sets: one being multiplied, one being read.
  bf16x8 a0[FM], b0[NF], a1[FM], b1[NF];
  // PARTIAL: some of this wave's fragments are padding (checked per fragment, no schedule hint)
  auto main_loop = [&](auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    auto read_frags = [&](bf16x8* af, bf16x8* bfr, int buf, int kk) {
      const char* st = lds + buf * STAGE;
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        if (!PARTIAL || i < fmv)
          af[i] = *reinterpret_cast<const bf16x8*>(st + (mrow0 + i * 32) * ROWB + lane_off[kk]);
      if (PARTIAL && fmv == 0) return;
      #pragma unroll
      for (int j = 0; j < NF; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(st + b_row[j] + lane_off[kk]);
    };
    auto mfmas = [&](const bf16x8* af, const bf16x8* bfr) {
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        if (!PARTIAL || i < fmv)
          #pragma unroll
          for (int j = 0; j < NF; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // Scheduler hint: two MFMAs, then all of the next k-step's fragment reads back to back
    // (each wave needs many LDS reads in flight to cover LDS latency), then the rest of the
    // MFMAs.
    auto interleave = [&]() {
      if constexpr (!PARTIAL) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, FM + NF, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FM * NF - 2, 0);
      }
    };
    // k-step kk of the slice in `buf`: multiply set (kk & 1) while reading the next k-step
    // (of this slice, or k-step 0 of the slice in `nbuf`) into the other set.
    auto step = [&](int kk, int buf, int nbuf) {
      const int nb = (kk + 1 < KK) ? buf : nbuf;
      const int nk = (kk + 1 < KK) ? kk + 1 : 0;
      if (kk & 1) { read_frags(a0, b0, nb, nk); mfmas(a1, b1); }
      else        { read_frags(a1, b1, nb, nk); mfmas(a0, b0); }
      interleave();
    };

    // Ring of NS stages.  After the fragments of a slice's last k-step are read, one barrier
    // (a) publishes slice kt+1 (every wave waited for its own copies of it) and (b) frees the
    // stage of slice kt, which is refilled at once with slice kt+NS; the last k-step's MFMAs
    // then overlap the reads of slice kt+1's first fragments.  NS-1 slices stay in flight.
    #pragma unroll
    for (int s = 0; s < NS; ++s) issue(s, min(s, KT - 1));
    wait_vmcnt<(NS - 1) * NQW>();
    __syncthreads();
    read_frags(a0, b0, 0, 0);
    int buf = 0;
    for (int kt = 0; kt < KT; ++kt) {
      const int nbuf = (buf + 1 == NS) ? 0 : buf + 1;
      #pragma unroll
      for (int kk = 0; kk < KK - 1; ++kk) step(kk, buf, nbuf);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // all reads of stage buf done
      wait_vmcnt<(NS - 2) * NQW>();                          // this wave's slice kt+1 landed
      __syncthreads();
      // past the last slice repeat slice KT-1 (in bounds, never read) so every iteration
      // leaves the same number of copies outstanding
      issue(buf, min(kt + NS, KT - 1));
      step(KK - 1, buf, nbuf);              // after the last slice the reads are stale, unused
      buf = nbuf;
    }
    wait_vmcnt<0>();
  };
  if (fmv == FM) main_loop(std::false_type{});
  else           main_loop(std::true_type{});

  // ---- epilogue (as in gemm_kernel) ---------------------------------------------------------
  const int ocol = lane & 31;
  const int orow = 4 * (lane >> 5);
  if (UP) {
    #pragma unroll
    for (int i = 0; i < FM; ++i)
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mrow0 + i * 32 + 8 * (v >> 2) + orow + (v & 3);
        uint16_t* dst = g.out + (size_t)(row0 + m) * g.n_out + n0 + wn * WTN + ocol;
        #pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float gt = acc[i][j][v], up = acc[i][j + FN][v];
          const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
          dst[j * 32] = (uint16_t)f32_to_bf16_bits(a);
        }
      }
  } else {
    #pragma unroll
    for (int i = 0; i < FM; ++i)
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mrow0 + i * 32 + 8 * (v >> 2) + orow + (v & 3);
        const int s = g.sorted_slots[row0 + m];
        if (s >= g.n_slots) continue;
        const float wt = g.topk_w[s];
        uint16_t* dst = g.out + (size_t)s * g.n_out + n0 + wn * WTN + ocol;
        #pragma unroll
        for (int j = 0; j < FN; ++j) dst[j * 32] = (uint16_t)f32_to_bf16_bits(acc[i][j][v] * wt);
      }
  }
}

template <int BK, int NS, int BNA, bool UP, int WM = 1, int BMT = BM, int WN = 4>
hipError_t run_dma(const Args& a, hipStream_t s) {
  // multiple of 8: every XCD's share of the valid tiles must have blocks to run on
  const int64_t grid = ((int64_t)a.tiles_max * (a.n_out / BNA) + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_dma_kernel<BMT, BK, NS, BNA, UP, WM, WN>), dim3((unsigned)grid),
                     dim3(WN * WM * kWave), 0, s, a);
  return hipGetLastError();
}

template <int BK, int WM, int WN, int BNA, bool UP>
hipError_t run(const Args& a, hipStream_t s) {
  // multiple of 8: every XCD's share of the valid tiles must have blocks to run on
  const int64_t grid = ((int64_t)a.tiles_max * (a.n_out / BNA) + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<BK, WM, WN, BNA, UP>), dim3((unsigned)grid), dim3(WM * WN * kWave),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace pf

// bf16 with 128- or 256-row m-blocks.
bool prefill_supported(const Resolved& r) {
  return r.w_dtype == MOE_BF16 && (r.BM == pf::BM || r.BM == 2 * pf::BM);
}

hipError_t launch_up_prefill(const Resolved& r, const void* x, const void* w13,
                             const int32_t* sorted_slots, const int32_t* offsets,
                             const int32_t* tiles, const int32_t* num_tiles, void* act,
                             hipStream_t s) {
  pf::Args a{};
  a.offsets = offsets;
  a.a_src = (const char*)x;
  a.w = (const char*)w13;
  a.sorted_slots = sorted_slots;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.out = (uint16_t*)act;
  a.K = r.H;
  a.n_out = r.I;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  a.tiles_max = (int)r.tiles_max;
  a.w_expert_elems = (int64_t)2 * r.I * r.H;
  // 256-row m-blocks: 8 waves, 4 along M (64 rows each) x 2 along N
  if (r.I % 128 != 0) {   // I a multiple of 64 only: 64-wide n-blocks, 2 waves along N
    if (r.BM == 256) return pf::run_dma<64, 3, 64, true, 4, 256, 2>(a, s);
    return pf::run_dma<64, 4, 64, true, 4, 128, 2>(a, s);
  }
  if (r.BM == 256) return pf::run_dma<64, 2, 128, true, 4, 256, 2>(a, s);
  if (r.I % 256 == 0) return pf::run_dma<64, 2, 256, true, 2>(a, s);
  return pf::run_dma<64, 3, 128, true>(a, s);
}

hipError_t launch_down_prefill(const Resolved& r, const void* act, const void* w2,
                               const float* topk_w, const int32_t* sorted_slots,
                               const int32_t* offsets, const int32_t* tiles,
                               const int32_t* num_tiles, void* slot_out, hipStream_t s) {
  pf::Args a{};
  a.offsets = offsets;
  a.a_src = (const char*)act;
  a.w = (const char*)w2;
  a.sorted_slots = sorted_slots;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.topk_w = topk_w;
  a.out = (uint16_t*)slot_out;
  a.K = r.I;
  a.n_out = r.H;
  a.top_k = r.K;
  a.n_slots = (int)r.N;
  a.tiles_max = (int)r.tiles_max;
  a.w_expert_elems = (int64_t)r.H * r.I;
  if (r.H % 128 != 0) {   // H a multiple of 64 only
    if (r.BM == 256) return pf::run_dma<64, 3, 64, false, 4, 256, 2>(a, s);
    return pf::run_dma<64, 4, 64, false, 4, 128, 2>(a, s);
  }
  if (r.BM == 256) {
    if (r.H % 256 == 0) return pf::run_dma<64, 2, 256, false, 4, 256, 2>(a, s);
    return pf::run_dma<64, 2, 128, false, 4, 256, 2>(a, s);
  }
  if (r.H % 256 == 0) return pf::run_dma<64, 3, 256, false, 2>(a, s);
  return pf::run_dma<64, 4, 128, false>(a, s);
}

}  // namespace moe
