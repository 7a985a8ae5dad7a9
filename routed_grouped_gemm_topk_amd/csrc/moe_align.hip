// Expert alignment: histogram, padded prefix offsets, stable expert-sorted slot list,
// inverse map and (expert, first row) tile table.
//
// Sources: "MOE Bmm1 Fused Gather" (make_ragged_tensor_metadata: slice sizes, slice
// offsets and a block schedule; gather index = slot // top_k), "moe triton kernel use
// tma." (the align kernel records per M block the expert id and first token row) and
// "factor_moe_fused_gemm.cu" (build_expert_map_kernel counts slots per expert with
// atomics and leaves the positions unfinished).  Here the counts still come from LDS
// integer atomics (order-free), but each slot's position is a stable rank: the number
// of lower-numbered slots routed to the same expert.  Within a wavefront that rank
// comes from a bit-sliced ballot match (lanes holding the same key), across wavefronts
// and chunks from LDS prefix counts, so the output is bit-identical on every run.
//
// One workgroup of 1024 threads does the whole pass (the slot count of an MoE batch
// is tens of thousands at most); it is latency-bound and takes a few microseconds.
#include "moe_internal.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kAlignMaxExperts = 1024;

// Largest index i in [0, n) with v[i] <= x, for non-decreasing v with v[0] <= x.
__device__ __forceinline__ int upper_index(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (v[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int N, int E, int BM, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  __shared__ int cnt[kAlignMaxExperts];
  __shared__ int tb[kAlignMaxExperts + 1];    // first tile of each expert (exclusive scan)
  __shared__ int off[kAlignMaxExperts + 1];   // first row of each expert
  __shared__ int base[kAlignMaxExperts];      // slots of each expert placed by earlier chunks
  __shared__ int ctot[kAlignMaxExperts];      // slots of each expert in the current chunk
  __shared__ uint16_t hist[kAlignWaves][kAlignMaxExperts];  // per-wave counts -> prefixes
  __shared__ int wsum[kAlignWaves];
  __shared__ int s_invalid;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int e = tid; e < E; e += kAlignThreads) { cnt[e] = 0; base[e] = 0; }
  if (tid == 0) s_invalid = 0;
  __syncthreads();

  // ---- pass 1: histogram -------------------------------------------------------------------
  int my_invalid = 0;
  for (int s = tid; s < N; s += kAlignThreads) {
    int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1); else ++my_invalid;
  }
  if (my_invalid) atomicAdd(&s_invalid, my_invalid);
  __syncthreads();

  // ---- exclusive scan of m-blocks per expert (E <= 1024: one expert per thread) ------------
  const int nb = (tid < E) ? (cnt[tid] + BM - 1) / BM : 0;
  int incl = nb;
  #pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int v = (lane < kAlignWaves) ? wsum[lane] : 0;
    int iv = v;
    #pragma unroll
    for (int d = 1; d < kAlignWaves; d <<= 1) {
      int y = __shfl_up(iv, d, kWave);
      if (lane >= d) iv += y;
    }
    if (lane < kAlignWaves) wsum[lane] = iv - v;   // exclusive wave prefix
  }
  __syncthreads();
  const int excl = incl - nb + wsum[wave];
  if (tid < E) {
    tb[tid] = excl;
    off[tid] = excl * BM;
    if (tid == E - 1) { tb[E] = excl + nb; off[E] = (excl + nb) * BM; }
  }
  __syncthreads();

  const int total_tiles = tb[E];
  for (int e = tid; e <= E; e += kAlignThreads) {
    offsets[e] = off[e];
    if (e < E) counts[e] = cnt[e];
  }
  if (tid == 0) { *num_tiles = total_tiles; *n_invalid = s_invalid; }

  // ---- tile table ---------------------------------------------------------------------------
  for (int i = tid; i < tiles_max; i += kAlignThreads) {
    int e = -1, r = -1;
    if (i < total_tiles) {
      e = upper_index(tb, E, i);
      r = off[e] + (i - tb[e]) * BM;
    }
    tiles[2 * i] = e;
    tiles[2 * i + 1] = r;
  }

  // ---- sentinel in padding rows and the unused tail ------------------------------------------
  const int rows_used = off[E];
  for (int r = tid; r < rows_max; r += kAlignThreads) {
    bool pad = true;
    if (r < rows_used) {
      int e = upper_index(off, E, r);
      pad = (r - off[e]) >= cnt[e];
    }
    if (pad) sorted_slots[r] = N;
  }

  // ---- pass 2: stable placement, 1024 slots per chunk ----------------------------------------
  const int key_bits = 32 - __clz(E);   // keys 0..E (E = excluded / past the end)
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int chunk = 0; chunk < N; chunk += kAlignThreads) {
    const int s = chunk + tid;
    int key = (s < N) ? ids[s] : E;
    if ((unsigned)key >= (unsigned)E) key = E;

    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) (&hist[0][0])[(i / E) * kAlignMaxExperts + (i % E)] = 0;

    // lanes of this wave holding the same key
    uint64_t same = ~0ull;
    for (int b = 0; b < key_bits; ++b) {
      const int bit = (key >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    const int rank = __popcll(same & lanes_below);
    const int group = __popcll(same);
    __syncthreads();                                  // hist cleared
    if (key < E && rank == 0) hist[wave][key] = (uint16_t)group;
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) {    // per expert: prefix over waves
      int run = 0;
      #pragma unroll
      for (int w = 0; w < kAlignWaves; ++w) {
        int c = hist[w][e];
        hist[w][e] = (uint16_t)run;
        run += c;
      }
      ctot[e] = run;
    }
    __syncthreads();
    if (s < N) {
      if (key < E) {
        const int r = off[key] + base[key] + hist[wave][key] + rank;
        sorted_slots[r] = s;
        slot_row[s] = r;
      } else {
        slot_row[s] = -1;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) base[e] += ctot[e];
    __syncthreads();
  }
}

hipError_t launch_align(const Resolved& r, const int32_t* ids, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles,
                        int32_t* num_tiles, int32_t* n_invalid, hipStream_t s) {
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, (int)r.N, r.E, r.BM,
                     (int)r.rows_max, (int)r.tiles_max, counts, offsets, sorted_slots, slot_row,
                     tiles, num_tiles, n_invalid);
  return hipGetLastError();
}

}  // namespace moe
