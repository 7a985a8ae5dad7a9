// bf16 grouped GEMMs for 128- and 256-row m-blocks (prefill): gfx950 MFMA 32x32x16.
//
//   up   : act[r, n]      = SiLU(W13[e,n,:].x_r) * (W13[e,I+n,:].x_r),  x_r = X[sorted_slots[r] / top_k]
//   down : slot_out[s, h] = w[s] * (W2[e,h,:].act[r,:]),                 s = sorted_slots[r]
//
// Same computation as the generic tile kernel (moe_gemm.hip; sources cited there:
// "MOE Bmm1 Fused Gather" load_activations / SwiGLU epilogue, "moe triton kernel use
// tma." MUL_ROUTED_WEIGHT, "factor_moe_fused_gemm.cu" gate-first SiLU), shaped for
// large per-expert row counts on MI355X:
//   * v_mfma_f32_32x32x16_bf16: a 32x32 output tile per instruction reads half the LDS
//     bytes per flop of the 16x16 forms;
//   * one m-block x BNA output columns per workgroup (up: BNA gate rows plus the matching
//     BNA up rows of W13), WM x WN waves; wide tiles keep the L2->CU and LDS bytes per
//     flop low.  The last n-block may be ragged (n_out a multiple of 64, BNA of 128 or
//     256): its weight rows past n_out re-read the last row and its columns past n_out
//     are not stored;
//   * k-slices of BK = 64 (128 bytes per row) in a ring of NS LDS stages without padding:
//     the 16-byte chunk c of row r sits at position c ^ ((r & 7) ^ ((r >> 3) & 1)),
//     conflict-free for the fragment reads (32 consecutive rows at one k offset);
//   * global -> LDS copies by direct-to-LDS DMA (below), NS-1 slices in flight; the 256-row
//     tiles give the m-block rows a ring of two stages and the weight rows one of three, and
//     spread each slice's copies over the k-steps of the next slice;
//   * fragment reads of the next 16-wide k step overlap the MFMAs of the current one, one
//     read after each MFMA;
//   * with a workspace, the tiles of the last, partly filled round of workgroups are cut
//     along K (tail_split below), their fp32 partials added by split_reduce_kernel;
//   * tile order: expert by expert, groups of 8 m-blocks of one expert sweep the n-blocks;
//     that order is dealt to the XCDs (own L2 each) in chunks of 32 tiles, so concurrent
//     workgroups of an XCD share rows and weights, and a hot expert's tiles spread over all
//     XCDs (one contiguous range per XCD measured about 3% slower on large batches).
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace pf {

constexpr int BM = 128;        // rows per m-block
constexpr int kChunk = 32;     // logical tiles per chunk dealt to one XCD (xcd_chunked)
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

struct Args {
  const char* a_src;        // up: X [T, K]; down: act [rows_max, K]   (bf16)
  const char* w;            // up: W13 [E, 2I, K]; down: W2 [E, H, K]  (bf16)
  const int32_t* sorted_slots;
  const int32_t* offsets;
  const int32_t* tiles;
  const int32_t* num_tiles;
  const float* topk_w;      // down
  uint16_t* out;            // up: act [rows_max, I]; down: slot_out [N, H]  (bf16 bits)
  float* part;              // fp32 partial tiles of the K-split tail, or null
  int K, n_out, top_k, n_slots, tiles_max;
  int slots;                // with part: workgroup slots of the device (one per CU), else 0
  int grid_tiles;           // blocks [0, grid_tiles) run whole tiles, the rest K-split units
  int64_t w_expert_elems;
};

// K-split of the last round.  The logical tiles run in rounds of `slots`
// workgroups (one per CU); when the last round holds only r < slots tiles, those r tiles
// are cut along K into S parts, S = min(slots / r, K slices / kMinSplitSlices, kMaxSplit),
// so the last round is r*S short units instead of r whole tiles beside idle CUs.  Each unit
// writes its fp32 partial tile; split_reduce_kernel adds the S partials of a row in
// ascending part order (fixed, so the result does not depend on timing), then applies the
// epilogue (up: SiLU(gate) * up; down: the routing weight) and rounds once.
constexpr int kSplitBK = 64;          // k-slice of every prefill launch that may split
constexpr int kMinSplitSlices = 8;    // at least 512 of K per part
constexpr int kMaxSplit = 16;
constexpr int kMaxSplitUnits = 256;   // r*S <= slots <= this (sizes the partial buffer)

struct TailSplit { int full, r, S; };

__device__ __forceinline__ TailSplit tail_split(int total, int slots, int kt_all) {
  TailSplit t{total, 0, 1};
  if (slots <= 0) return t;
  const int r = total % slots;
  if (r == 0) return t;
  const int S = min(min(slots / r, kt_all / kMinSplitSlices), kMaxSplit);
  if (S < 2) return t;
  t.full = total - r;
  t.r = r;
  t.S = S;
  return t;
}

// Raw buffer descriptor of [base, base + bytes): 32-bit offsets, no stride; a lane whose offset
// is past `bytes` reads zeros without touching memory.
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, uint32_t bytes) {
  const unsigned long long a = (unsigned long long)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);                 // num_records (bytes)
  r[3] = 0x00020000;                                                 // raw 32-bit data
  return r;
}

// 64 lanes x 16 bytes from the buffer at voff + soff straight to LDS at M0 (MUBUF
// buffer_load_dwordx4 ... lds).
__device__ __forceinline__ void buf_dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory");
}

// ---------------------------------------------------------------------------------------------
// Direct-to-LDS variant: the global -> LDS copies are global_load_lds_dwordx4 (each wave
// instruction lands 64 x 16 bytes contiguously in LDS at M0), so no registers stage the
// k-slices and the LDS ring can hold NS slices, NS-1 of them in flight.  The copies are
// issued from inline assembly with explicit vmcnt waits: the compiler's own tracking of
// LDS DMA waits for every outstanding copy before any LDS read, which would drain the
// ring each k-slice.  The per-lane source address is chosen so that the fixed
// lane -> LDS position mapping realises the XOR swizzle above.
// ---------------------------------------------------------------------------------------------
// BUF: the copies are MUBUF buffer_load_dwordx4 ... lds against one buffer descriptor per wave
// (its copies are all gathered/act rows or all weight rows): 32-bit offsets instead of 64-bit
// addresses per lane (24 fewer VGPRs at 256-row blocks), the k offset in the scalar soffset,
// and padding rows of the gathered operand at an offset past the end of X, read as zeros
// without a memory access.  Measured against the global_load_lds form on the Mixtral-shaped
// workload: 2% faster, bit-identical.
// WS: stages of a separate weight ring (0: rows and weights share the NS-stage ring)
template <int BMT, int BK, int NS, int BNA, bool UP, int WM, int WN, bool BUF = false, int WS = 0>
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
  // SPLIT (WS > NS): the m-block rows and the weight rows have rings of their own, of NS = 2
  // and WS = 3 stages, and each wave copies only rows or only weights (BUF); see the k-loop.
  constexpr bool SPLIT = WS > NS;
  constexpr int ASTAGE = BMT * ROWB, WSTAGE = BROWS * ROWB;
  static_assert(!SPLIT || (BUF && NS == 2 && WS == 3 && KK == 4 && NQW == 8), "split rings");
  constexpr int LDS_BYTES = SPLIT ? NS * ASTAGE + WS * WSTAGE : NS * STAGE;

  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave % WN;
  const int wm = wave / WN;
  const int mrow0 = wm * (BMT / WM);               // this wave's first row of the m-block

  const int nblk = (g.n_out + BNA - 1) / BNA;      // the last n-block may be ragged
  const int KT_all = g.K / BK;
  const TailSplit ts = tail_split(*g.num_tiles * nblk, g.slots, KT_all);
  int logical, kbeg = 0, kend = KT_all, unit = -1;
  if ((int)blockIdx.x < g.grid_tiles) {
    logical = xcd_chunked<kChunk>(blockIdx.x, ts.full);
    if (logical < 0) return;
  } else {                                         // K-split unit of a last-round tile
    const int u = (int)blockIdx.x - g.grid_tiles;
    if (u >= ts.r * ts.S) return;
    const int ti = u % ts.r, part = u / ts.r;
    logical = ts.full + ti;
    kbeg = part * KT_all / ts.S;
    kend = (part + 1) * KT_all / ts.S;
    unit = ti * ts.S + part;
  }
  const TileRef tr = grouped_tile<BMT, GROUP_M>(logical, nblk, g.tiles, g.offsets);
  const int e = tr.e;
  const int row0 = tr.row0;
  const int n0 = tr.nt * BNA;
  const int K = g.K;
  const int KT = kend - kbeg;                       // k-slices of this workgroup, from kbeg

  // ---- this wave's copies: source of each row chunk (k-slice 0) and LDS offsets -----------
  // FLAT: a 64-bit address per copy; BUF: a 32-bit offset into this wave's buffer (X or the
  // m-block's act rows for A copies, the expert's weight slab for weight copies).
  static_assert(!BUF || BMT % (NQW * ROWS_PER_Q) == 0, "BUF: a wave copies only A or only weight rows");
  const char* wbase = g.w + (size_t)e * g.w_expert_elems * 2;
  const bool a_wave = wave * NQW * ROWS_PER_Q < BMT;
  i32x4 rsrc{};
  if (BUF) {
    if (!a_wave)
      rsrc = buf_rsrc(wbase, (uint32_t)(g.w_expert_elems * 2));
    else if (UP)
      rsrc = buf_rsrc(g.a_src, (uint32_t)((size_t)(g.n_slots / g.top_k) * K * 2));
    else
      rsrc = buf_rsrc(g.a_src + (size_t)row0 * K * 2, (uint32_t)(BMT * K * 2));
  }
  const char* src[BUF ? 1 : NQW];
  uint32_t voff[BUF ? NQW : 1];
  // Slots of the m-block (to count its rows that hold slots) and of the rows this wave
  // gathers, all loaded before any is used: one memory round trip per tile (a slot loaded
  // where it is used made the compiler wait for each in turn: one round trip per copy).
  int mslot[BMT / kWave];
  #pragma unroll
  for (int r0 = 0; r0 < BMT; r0 += kWave) mslot[r0 / kWave] = g.sorted_slots[row0 + r0 + lane];
  int slot[UP ? NQW : 1];
  if constexpr (UP) {
    #pragma unroll
    for (int i = 0; i < NQW; ++i)
      if ((wave * NQW + i) * ROWS_PER_Q < BMT)    // wave-uniform: copy i gathers rows
        slot[i] = g.sorted_slots[row0 + (wave * NQW + i) * ROWS_PER_Q + lane / CPR];
  }
  // Rows of the m-block that hold slots come first, padding after: this wave's 32-row
  // fragments from fmv on are all padding, and their reads and MFMAs are skipped.
  int valid = 0;
  #pragma unroll
  for (int r0 = 0; r0 < BMT; r0 += kWave) valid += __popcll(__ballot(mslot[r0 / kWave] < g.n_slots));
  const int fmv = __builtin_amdgcn_readfirstlane(min(FM, max(0, (valid - mrow0 + 31) / 32)));
  #pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = wave * NQW + i;
    const int r = q * ROWS_PER_Q + lane / CPR;      // row of the stage this lane fills
    const int cc = (lane % CPR) ^ swz<ROWB>(r);      // chunk that belongs at this position
    if (q * ROWS_PER_Q < BMT) {
      if (UP) {
        const int s = slot[i];
        const int t = s / g.top_k;                   // sentinel slots too: no branch
        if constexpr (BUF)
          voff[i] = (s < g.n_slots) ? (uint32_t)(t * K * 2 + cc * 16) : 0x80000000u;
        else
          src[i] = (s < g.n_slots) ? g.a_src + (size_t)t * K * 2 + cc * 16
                                   : g_zero_row + cc * 16;
      } else {
        if constexpr (BUF) voff[i] = (uint32_t)(r * K * 2 + cc * 16);
        else src[i] = g.a_src + (size_t)(row0 + r) * K * 2 + cc * 16;
      }
    } else {
      // weight row; past n_out (ragged last n-block) the last row is re-read, its products
      // are not stored
      const int rb = r - BMT;
      const int nr = min(n0 + (UP && rb >= BNA ? rb - BNA : rb), g.n_out - 1);
      const int grow = (UP && rb >= BNA) ? g.n_out + nr : nr;
      if constexpr (BUF) voff[i] = (uint32_t)(grow * K * 2 + cc * 16);
      else src[i] = wbase + (size_t)grow * K * 2 + cc * 16;
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  // copies [I0, I0 + N) of this wave for slice kt into stage buf of the wave's ring
  auto issue_part = [&](auto i0_tag, auto n_tag, int buf, int kt) {
    constexpr int I0 = decltype(i0_tag)::value, N = decltype(n_tag)::value;
    uint32_t st;
    if constexpr (SPLIT)
      st = a_wave ? lds_base + buf * ASTAGE + wave * NQW * 1024
                  : lds_base + NS * ASTAGE + buf * WSTAGE + wave * NQW * 1024 - ASTAGE;
    else
      st = lds_base + buf * STAGE + wave * NQW * 1024;
    st = __builtin_amdgcn_readfirstlane(st);
    const int koff = kt * ROWB;
    #pragma unroll
    for (int i = I0; i < I0 + N; ++i) {
      if constexpr (BUF) buf_dma16(rsrc, voff[i], (uint32_t)koff, st + i * 1024);
      else lds_dma16(src[i] + koff, st + i * 1024);
    }
  };
  auto issue = [&](int buf, int kt) {
    issue_part(std::integral_constant<int, 0>{}, std::integral_constant<int, NQW>{}, buf, kt);
  };
  // SPLIT: a slice's copies go out in parts, part p before k-step p-1 of the next slice (part
  // 0 right after the barrier): rows in parts of 3, 3, 2 (p = 0..2), weights of 2 (p = 0..3).
  auto issue_p = [&](int p, int buf, int kt) {
    if constexpr (SPLIT) {
      using C0 = std::integral_constant<int, 0>;
      using C2 = std::integral_constant<int, 2>;
      using C3 = std::integral_constant<int, 3>;
      using C4 = std::integral_constant<int, 4>;
      using C6 = std::integral_constant<int, 6>;
      if (a_wave) {
        if (p == 0)      issue_part(C0{}, C3{}, buf, kt);
        else if (p == 1) issue_part(C3{}, C3{}, buf, kt);
        else if (p == 2) issue_part(C6{}, C2{}, buf, kt);
      } else {
        if (p == 0)      issue_part(C0{}, C2{}, buf, kt);
        else if (p == 1) issue_part(C2{}, C2{}, buf, kt);
        else if (p == 2) issue_part(C4{}, C2{}, buf, kt);
        else             issue_part(C6{}, C2{}, buf, kt);
      }
    }
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


  // Two fragment sets: one being multiplied, one being read.
  bf16x8 a0[FM], b0[NF], a1[FM], b1[NF];
  // PARTIAL: some of this wave's fragments are padding (checked per fragment, no schedule hint)
  auto main_loop = [&](auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    // buf: stage of the m-block rows; wbuf: stage of the weight rows (the same unless SPLIT)
    auto read_frags = [&](bf16x8* af, bf16x8* bfr, int buf, int wbuf, int kk) {
      const char* st = lds + (SPLIT ? buf * ASTAGE : buf * STAGE);
      const char* sw = SPLIT ? lds + NS * ASTAGE + wbuf * WSTAGE - ASTAGE : st;
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        if (!PARTIAL || i < fmv)
          af[i] = *reinterpret_cast<const bf16x8*>(st + (mrow0 + i * 32) * ROWB + lane_off[kk]);
      if (PARTIAL && fmv == 0) return;
      #pragma unroll
      for (int j = 0; j < NF; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(sw + b_row[j] + lane_off[kk]);
    };
    auto mfmas = [&](const bf16x8* af, const bf16x8* bfr) {
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        if (!PARTIAL || i < fmv)
          #pragma unroll
          for (int j = 0; j < NF; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // Scheduler hint: each MFMA is followed by one of the next k-step's fragment reads until
    // the reads run out, then the remaining MFMAs (or reads).  Measured against two MFMAs,
    // all reads back to back, then the rest: bit-identical results, the Mixtral-shaped up
    // GEMM 3% and the skewed up GEMM 4% faster; reads issued before their MFMA, or spread
    // evenly over the MFMAs, were no better.
    auto interleave = [&]() {
      if constexpr (!PARTIAL) {
        constexpr int NM = FM * NF, ND = FM + NF, NP = NM < ND ? NM : ND;
        #pragma unroll
        for (int q = 0; q < NP; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (ND > NP) __builtin_amdgcn_sched_group_barrier(0x100, ND - NP, 0);
        if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
      }
    };
    // k-step kk of the slice in `buf`: multiply set (kk & 1) while reading the next k-step
    // (of this slice, or k-step 0 of the slice in `nbuf`) into the other set.
    auto step = [&](int kk, int buf, int nbuf, int wbuf, int nwbuf) {
      const int nb = (kk + 1 < KK) ? buf : nbuf;
      const int nw = (kk + 1 < KK) ? wbuf : nwbuf;
      const int nk = (kk + 1 < KK) ? kk + 1 : 0;
      if (kk & 1) { read_frags(a0, b0, nb, nw, nk); mfmas(a1, b1); }
      else        { read_frags(a1, b1, nb, nw, nk); mfmas(a0, b0); }
      interleave();
    };

    // Ring of NS stages.  After the fragments of a slice's last k-step are read, one barrier
    // (a) publishes slice kt+1 (every wave waited for its own copies of it) and (b) frees the
    // stage of slice kt, which is refilled with slice kt+NS; the last k-step's MFMAs then
    // overlap the reads of slice kt+1's first fragments.  NS-1 slices stay in flight.
    //
    // SPLIT: the freed rows stage takes rows slice kt+2 and the freed weight stage weight
    // slice kt+3, both in parts spread over the next k-steps (issue_p), so rows slice kt+2
    // is complete before barrier kt+1 and weight slices kt+2 and kt+3 may be in flight
    // there.  Measured against the single ring whose 64 copies all went out right after the
    // barrier (timers in the loop: the waves whose copies were accepted last reached the next
    // barrier last, the others waited there 35-42% of the time): down GEMM 4-6% faster, up
    // GEMM unchanged, bit-identical.  Copying rows and weights in every wave, or only in the
    // four waves that the issue arbiter favours, or the weights alone spread, was slower.
    if constexpr (SPLIT) {
      // rows: slice 0 and part 0 of slice 1; weights: slices 0, 1 and part 0 of slice 2
      const int last = a_wave ? NS - 1 : WS - 1;
      #pragma unroll
      for (int s = 0; s < WS - 1; ++s)
        if (s < last) issue(s, kbeg + min(s, KT - 1));
      issue_p(0, last, kbeg + min(last, KT - 1));
      if (a_wave) wait_vmcnt<3>();                 // rows slice 0 landed
      else        wait_vmcnt<NQW + 2>();           // weight slice 0 landed
    } else {
      #pragma unroll
      for (int s = 0; s < NS; ++s) issue(s, kbeg + min(s, KT - 1));
      wait_vmcnt<(NS - 1) * NQW>();
    }
    __syncthreads();
    read_frags(a0, b0, 0, 0, 0);
    // stage and slice whose parts are being issued (SPLIT)
    int buf = 0, wbuf = 0, qbuf = a_wave ? NS - 1 : WS - 1, qslice = qbuf;
    for (int kt = 0; kt < KT; ++kt) {
      const int nbuf = (buf + 1 == NS) ? 0 : buf + 1;
      const int nwbuf = SPLIT ? ((wbuf + 1 == WS) ? 0 : wbuf + 1) : nbuf;
      #pragma unroll
      for (int kk = 0; kk < KK - 1; ++kk) {
        if constexpr (SPLIT) issue_p(kk + 1, qbuf, kbeg + min(qslice, KT - 1));
        step(kk, buf, nbuf, SPLIT ? wbuf : buf, nwbuf);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // all reads of stage buf done
      // this wave's copies of slice kt+1 landed (SPLIT weights: slice kt+2 may be in flight)
      if (SPLIT && !a_wave) wait_vmcnt<NQW>();
      else                  wait_vmcnt<(NS - 2) * NQW>();
      __syncthreads();
      // past the last slice repeat slice KT-1 (in bounds, never read) so every iteration
      // leaves the same number of copies outstanding
      if constexpr (SPLIT) {
        qbuf = a_wave ? buf : wbuf;
        qslice = kt + (a_wave ? NS : WS);
        issue_p(0, qbuf, kbeg + min(qslice, KT - 1));
      } else {
        issue(buf, kbeg + min(kt + NS, KT - 1));
      }
      step(KK - 1, buf, nbuf, SPLIT ? wbuf : buf, nwbuf);   // after the last slice: stale, unused
      buf = nbuf;
      wbuf = nwbuf;
    }
    wait_vmcnt<0>();
  };
  if (fmv == FM) main_loop(std::false_type{});
  else           main_loop(std::true_type{});

  // ---- epilogue -------------------------------------------------------------------------------
  // up: act = SiLU(gate) * up in bf16; down: slot row = w[s] * acc in bf16, padding rows skipped.
  // In the ragged last n-block, 32-column fragments past n_out are not stored; that check is a
  // separate copy of the epilogue, so the common copy's stores carry no column test.  Staging
  // the tile in LDS for whole-row 16-byte stores (also with non-temporal stores) was measured:
  // bit-identical and no faster, so the stores go straight from the MFMA layout.
  const int ocol = lane & 31;
  const int orow = 4 * (lane >> 5);
  const int ncol0 = n0 + wn * WTN;
  if (unit >= 0) {
    // K-split unit: the fp32 partial tile [BMT][PW] (up: gate columns, then up columns);
    // all-padding fragments are not stored (split_reduce_kernel reads only rows that hold
    // slots)
    constexpr int PW = UP ? 2 * BNA : BNA;
    float* pb = g.part + (size_t)unit * BMT * PW + wn * WTN + ocol;
    #pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fmv) continue;
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mrow0 + i * 32 + 8 * (v >> 2) + orow + (v & 3);
        #pragma unroll
        for (int j = 0; j < NF; ++j)
          pb[(size_t)m * PW + (j < FN ? j * 32 : BNA + (j - FN) * 32)] = acc[i][j][v];
      }
    }
    return;
  }
  auto epilogue = [&](auto ragged_tag) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    if (UP) {
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = mrow0 + i * 32 + 8 * (v >> 2) + orow + (v & 3);
          uint16_t* dst = g.out + (size_t)(row0 + m) * g.n_out + ncol0 + ocol;
          #pragma unroll
          for (int j = 0; j < FN; ++j) {
            if (RAGGED && ncol0 + j * 32 >= g.n_out) continue;
            const float gt = acc[i][j][v], up = acc[i][j + FN][v];
            const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
            dst[j * 32] = (uint16_t)f32_to_bf16_bits(a);
          }
        }
    } else {
      // All slots of this lane's rows first, then all their routing weights (the index is
      // clamped so the load needs no branch), then the stores.  Loaded row by row behind the
      // padding test, each row cost two dependent global round trips: the skewed-routing down
      // GEMM took 13% longer.
      int srow[FM][16];
      float wrow[FM][16];
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 16; ++v)
          srow[i][v] = g.sorted_slots[row0 + mrow0 + i * 32 + 8 * (v >> 2) + orow + (v & 3)];
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 16; ++v) wrow[i][v] = g.topk_w[min(srow[i][v], g.n_slots - 1)];
      #pragma unroll
      for (int i = 0; i < FM; ++i)
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int s = srow[i][v];
          if (s >= g.n_slots) continue;
          uint16_t* dst = g.out + (size_t)s * g.n_out + ncol0 + ocol;
          #pragma unroll
          for (int j = 0; j < FN; ++j) {
            if (RAGGED && ncol0 + j * 32 >= g.n_out) continue;
            dst[j * 32] = (uint16_t)f32_to_bf16_bits(acc[i][j][v] * wrow[i][v]);
          }
        }
    }
  };
  if (ncol0 + WTN <= g.n_out) epilogue(std::false_type{});
  else                        epilogue(std::true_type{});
}

// Sum of the S partial tiles of each K-split tile (ascending part order), then the epilogue
// (up: SiLU(gate) * up, padding rows 0; down: times the routing weight, padding rows not
// stored), rounded once to bf16: one wave per row, BNA/64 columns per lane, 16 rows per block.
template <int BMT, int BNA, bool UP>
__global__ __launch_bounds__(256) void split_reduce_kernel(Args g) {
  constexpr int CPL = BNA / kWave;
  constexpr int RPB = 16;
  constexpr int PW = UP ? 2 * BNA : BNA;
  const int nblk = (g.n_out + BNA - 1) / BNA;
  const TailSplit ts = tail_split(*g.num_tiles * nblk, g.slots, g.K / kSplitBK);
  const int ti = (int)blockIdx.x / (BMT / RPB);
  if (ti >= ts.r) return;
  const TileRef tr = grouped_tile<BMT, GROUP_M>(ts.full + ti, nblk, g.tiles, g.offsets);
  const int row0 = tr.row0;
  const int n0 = tr.nt * BNA;
  const int lane = threadIdx.x & (kWave - 1);
  const int c0 = lane * CPL;
  const size_t pstride = (size_t)BMT * PW;
  for (int m = ((int)blockIdx.x % (BMT / RPB)) * RPB + (int)threadIdx.x / kWave;
       m < ((int)blockIdx.x % (BMT / RPB) + 1) * RPB; m += 256 / kWave) {
    const int s = g.sorted_slots[row0 + m];
    if (UP) {
      uint16_t* dst = g.out + (size_t)(row0 + m) * g.n_out + n0 + c0;
      float gt[CPL], up[CPL];
      #pragma unroll
      for (int c = 0; c < CPL; ++c) gt[c] = up[c] = 0.0f;
      if (s < g.n_slots) {
        const float* pb = g.part + (size_t)ti * ts.S * pstride + (size_t)m * PW + c0;
        for (int p = 0; p < ts.S; ++p)
          #pragma unroll
          for (int c = 0; c < CPL; ++c) {
            gt[c] += pb[p * pstride + c];
            up[c] += pb[p * pstride + BNA + c];
          }
      }
      #pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (n0 + c0 + c < g.n_out) {
          const float a = gt[c] * __builtin_amdgcn_rcpf(1.0f + __expf(-gt[c])) * up[c];
          dst[c] = (uint16_t)f32_to_bf16_bits(a);
        }
    } else {
      if (s >= g.n_slots) continue;
      const float* pb = g.part + (size_t)ti * ts.S * pstride + (size_t)m * PW + c0;
      float sum[CPL];
      #pragma unroll
      for (int c = 0; c < CPL; ++c) sum[c] = pb[c];
      for (int p = 1; p < ts.S; ++p)
        #pragma unroll
        for (int c = 0; c < CPL; ++c) sum[c] += pb[p * pstride + c];
      const float wt = g.topk_w[s];
      uint16_t* dst = g.out + (size_t)s * g.n_out + n0 + c0;
      #pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (n0 + c0 + c < g.n_out) dst[c] = (uint16_t)f32_to_bf16_bits(sum[c] * wt);
    }
  }
}

template <int BK, int NS, int BNA, bool UP, int WM = 1, int BMT = BM, int WN = 4, bool BUF = false, int WS = 0>
hipError_t run_dma(Args a, hipStream_t s) {
  // sized by the host-side tile bound; blocks past the device-side tile count exit at once
  const int64_t grid = xcd_chunked_grid<kChunk>((int64_t)a.tiles_max * ((a.n_out + BNA - 1) / BNA));
  if (grid <= 0) return hipSuccess;
  const bool split = a.part != nullptr && a.slots >= 2;
  if (!split) a.slots = 0;
  static_assert(BK == kSplitBK, "the K-split tail assumes 64-wide k-slices");
  a.grid_tiles = (int)grid;
  hipLaunchKernelGGL((gemm_dma_kernel<BMT, BK, NS, BNA, UP, WM, WN, BUF, WS>),
                     dim3((unsigned)(grid + (split ? a.slots : 0))), dim3(WN * WM * kWave), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  // S >= 2 needs r <= slots / 2 tiles to reduce
  hipLaunchKernelGGL((split_reduce_kernel<BMT, BNA, UP>), dim3((unsigned)(a.slots / 2 * (BMT / 16))),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pf

// bf16 with 128- or 256-row m-blocks.
bool prefill_supported(const Resolved& r) {
  return r.w_dtype == MOE_BF16 && (r.BM == pf::BM || r.BM == 2 * pf::BM);
}

// Partial-tile buffer of the GEMMs' K-split tail: kMaxSplitUnits fp32 tiles of block_m rows
// x the widest partial tile of the two launches (up: gate + up columns, 2 x 128 at 256-row
// m-blocks, 2 x 256 or 2 x 128 at 128-row ones; down: 256 when H allows, else 128).
int64_t gemm_split_bytes(const Resolved& r) {
  if (!prefill_supported(r)) return 0;
  const int64_t up = r.BM == 256 ? 256 : (r.I % 256 == 0 ? 512 : 256);
  const int64_t down = r.H % 256 == 0 ? 256 : 128;
  return (int64_t)pf::kMaxSplitUnits * r.BM * (up > down ? up : down) * 4;
}

hipError_t launch_up_prefill(const Resolved& r, const void* x, const void* w13,
                             const int32_t* sorted_slots, const int32_t* offsets,
                             const int32_t* tiles, const int32_t* num_tiles, void* act,
                             void* split_ws, hipStream_t s) {
  pf::Args a{};
  a.part = (float*)split_ws;
  a.slots = split_ws ? std::min(device_cu_count(), pf::kMaxSplitUnits) : 0;
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
  // 256-row m-blocks: 8 waves, 4 along M (64 rows each) x 2 along N.  I a multiple of 64
  // but not of 128: the last 128-wide n-block is half used.
  // MUBUF copies need X's byte size below 2^31 (32-bit offsets; padding at 2^31 reads zeros)
  if (r.BM == 256) {
    if ((int64_t)r.T * r.H * 2 < ((int64_t)1 << 31))
      return pf::run_dma<64, 2, 128, true, 4, 256, 2, true, 3>(a, s);
    return pf::run_dma<64, 2, 128, true, 4, 256, 2>(a, s);
  }
  if (r.I % 256 == 0) return pf::run_dma<64, 2, 256, true, 2>(a, s);
  return pf::run_dma<64, 3, 128, true>(a, s);
}

hipError_t launch_down_prefill(const Resolved& r, const void* act, const void* w2,
                               const float* topk_w, const int32_t* sorted_slots,
                               const int32_t* offsets, const int32_t* tiles,
                               const int32_t* num_tiles, void* slot_out, void* split_ws,
                               hipStream_t s) {
  pf::Args a{};
  a.part = (float*)split_ws;
  a.slots = split_ws ? std::min(device_cu_count(), pf::kMaxSplitUnits) : 0;
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
  // H a multiple of 64 but not of 128: the last 128-wide n-block is half used
  if (r.BM == 256) {
    if (r.H % 256 == 0) return pf::run_dma<64, 2, 256, false, 4, 256, 2, true, 3>(a, s);
    return pf::run_dma<64, 2, 128, false, 4, 256, 2>(a, s);
  }
  if (r.H % 256 == 0) return pf::run_dma<64, 3, 256, false, 2>(a, s);
  return pf::run_dma<64, 4, 128, false>(a, s);
}

}  // namespace moe
