// Expert alignment: histogram, padded prefix offsets, stable expert-sorted slot list,
// inverse map and (expert, first row) tile table.
//
// Sources: "MOE Bmm1 Fused Gather" (make_ragged_tensor_metadata: slice sizes, slice
// offsets and a block schedule; gather index = slot // top_k), "moe triton kernel use
// tma." (the align kernel records per M block the expert id and first token row) and
// "factor_moe_fused_gemm.cu" (build_expert_map_kernel counts slots per expert with
// atomics and leaves the positions unfinished).  Here every slot's position is a stable
// rank: the number of lower-numbered slots routed to the same expert, so the output is
// bit-identical on every run.
//
// Ranks inside a workgroup: each of its 16 waves owns a contiguous run of the workgroup's
// slots and walks it 64 slots per step.  Within a step the lanes holding the same expert
// find each other with a bit-sliced ballot match (one ballot per key bit), which gives each
// lane its rank among them and the group size; the group's lowest lane adds the size to the
// wave's per-expert count in LDS.  Counting pass, one prefix over the waves, placing pass
// (the lowest lane's atomic add returns the group's first row, shared by a lane shuffle).
// All of a wave's ids are loaded at once, and no step waits on the previous one.
//
// Up to kSmallN slots one workgroup does everything.  Above that the slots are cut into
// chunks of at least kChunk (the last chunk takes the remainder) and three launches run:
// count (one workgroup per chunk), scan (one workgroup: per-expert prefix over the chunks,
// offsets, tiles, padding) and place (one workgroup per chunk).  The per-chunk counts are
// parked in the chunk's own part of slot_row, which only that chunk's place workgroup
// overwrites, after reading them.
#include "moe_internal.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kAlignMaxExperts = 1024;
constexpr int kSmallBatch = 8;                                   // steps per wave, one kernel
constexpr int kSmallN = kAlignWaves * kSmallBatch * kWave;       // 8192
constexpr int kChunk = 2048;                                     // >= E + 1 words of slot_row
constexpr int kChunkBatch = (2 * kChunk + kAlignThreads - 1) / kAlignThreads;  // 4 steps
static_assert(kChunk >= kAlignMaxExperts + 1, "chunk holds its counts and invalid count");

// Largest index i in [0, n) with v[i] <= x, for non-decreasing v with v[0] <= x.
__device__ __forceinline__ int upper_index(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (v[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Lanes of this wave holding the same key (keys < 2^key_bits).
__device__ __forceinline__ uint64_t match_any(int key, int key_bits) {
  uint64_t same = ~0ull;
  for (int b = 0; b < key_bits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  return same;
}

// This wave's part of the slot range [c0, c1): whole 64-slot steps, at most BATCH of them.
struct WaveRange {
  int begin, end;
};
template <int BATCH>
__device__ __forceinline__ WaveRange wave_range(int c0, int c1, int wave) {
  const int R = ((c1 - c0 + kAlignWaves - 1) / kAlignWaves + kWave - 1) / kWave * kWave;
  const int b = min(c0 + wave * R, c1);
  return {b, min(b + R, c1)};
}

// Keys of the wave's slots: k[u] = ids[begin + 64u + lane] (E past the range or invalid).
template <int BATCH>
__device__ __forceinline__ void load_keys(const int32_t* ids, WaveRange w, int E, int lane,
                                          int* k) {
  #pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    const int s = w.begin + u * kWave + lane;
    k[u] = (s < w.end) ? ids[s] : E;
  }
}

// Counting pass: adds this wave's per-expert counts into row[]; returns its invalid count.
template <int BATCH>
__device__ __forceinline__ int count_keys(const int* k, WaveRange w, int E, int key_bits,
                                          int lane, int* row) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int invalid = 0;
  #pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    if (w.begin + u * kWave >= w.end) break;
    int key = k[u];
    if ((unsigned)key >= (unsigned)E) {
      if (w.begin + u * kWave + lane < w.end) ++invalid;
      key = E;
    }
    const uint64_t same = match_any(key, key_bits);
    if (key < E && __popcll(same & below) == 0) atomicAdd(&row[key], __popcll(same));
  }
  #pragma unroll
  for (int d = 1; d < kWave; d <<= 1) invalid += __shfl_xor(invalid, d, kWave);
  return invalid;
}

// Placing pass: row[e] holds the next row for expert e; writes sorted_slots and slot_row.
template <int BATCH>
__device__ __forceinline__ void place_keys(const int* k, WaveRange w, int E, int key_bits,
                                           int lane, int* row, int32_t* sorted_slots,
                                           int32_t* slot_row) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  #pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    if (w.begin + u * kWave >= w.end) break;
    const int s = w.begin + u * kWave + lane;
    int key = k[u];
    if ((unsigned)key >= (unsigned)E) key = E;
    const uint64_t same = match_any(key, key_bits);
    const int rank = __popcll(same & below);
    int first = 0;
    if (key < E && rank == 0) first = atomicAdd(&row[key], __popcll(same));
    first = __shfl(first, (int)__builtin_ctzll(same), kWave);   // the group's lowest lane
    if (s < w.end) {
      if (key < E) {
        sorted_slots[first + rank] = s;
        slot_row[s] = first + rank;
      } else {
        slot_row[s] = -1;
      }
    }
  }
}

// hist[w][e] (counts of wave w) -> base[e] + counts of waves before w; returns nothing, the
// totals go to tot[e] when tot is given.  Called by the whole workgroup between barriers.
__device__ __forceinline__ void wave_prefix(int (*hist)[kAlignMaxExperts], int E, const int* base,
                                            int* tot) {
  for (int e = threadIdx.x; e < E; e += kAlignThreads) {
    int run = base ? base[e] : 0;
    #pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    if (tot) tot[e] = run;
  }
}

// From cnt[e] (LDS): offsets, counts, tiles, num_tiles and the sentinel in every row that
// holds no slot.  Leaves off[] (first row of each expert, E+1 entries) in LDS.  Whole
// workgroup; starts and ends with a barrier.
__device__ void finish_layout(const int* cnt, int* tb, int* off, int* wsum, int N, int E, int BM,
                              int rows_max, int tiles_max, int32_t* counts, int32_t* offsets,
                              int32_t* tiles, int32_t* num_tiles, int32_t* sorted_slots) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  __syncthreads();
  // exclusive scan of m-blocks per expert (E <= 1024: one expert per thread)
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
  if (tid == 0) *num_tiles = total_tiles;
  for (int i = tid; i < tiles_max; i += kAlignThreads) {
    int e = -1, r = -1;
    if (i < total_tiles) {
      e = upper_index(tb, E, i);
      r = off[e] + (i - tb[e]) * BM;
    }
    tiles[2 * i] = e;
    tiles[2 * i + 1] = r;
  }
  // sentinel in padding rows (after each expert's slots) and the unused tail.  An expert has
  // fewer than BM padding rows: from 64-row blocks on, wave w takes experts w, w + 16, ...,
  // its lanes writing an expert's padding rows 64 at a time (whole stores instead of one row
  // per lane per store); below that each thread writes its expert's few rows.
  if (BM >= kWave) {
    for (int e = wave; e < E; e += kAlignWaves)
      for (int r = off[e] + cnt[e] + lane; r < off[e + 1]; r += kWave) sorted_slots[r] = N;
  } else {
    for (int e = tid; e < E; e += kAlignThreads)
      for (int r = off[e] + cnt[e]; r < off[e + 1]; ++r) sorted_slots[r] = N;
  }
  for (int r = off[E] + tid; r < rows_max; r += kAlignThreads) sorted_slots[r] = N;
  __syncthreads();
}

// ---- up to kSmallN slots: one workgroup ---------------------------------------------------
__device__ __forceinline__ void align_small(
    const int32_t* ids, int N, int E, int BM, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  __shared__ int hist[kAlignWaves][kAlignMaxExperts];  // per-wave counts -> next rows
  __shared__ int cnt[kAlignMaxExperts];
  __shared__ int tb[kAlignMaxExperts + 1];
  __shared__ int off[kAlignMaxExperts + 1];
  __shared__ int wsum[kAlignWaves];
  __shared__ int winv[kAlignWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int key_bits = 32 - __clz(E);        // keys 0..E (E = excluded / past the end)

  const WaveRange w = wave_range<kSmallBatch>(0, N, wave);
  int k[kSmallBatch];
  load_keys<kSmallBatch>(ids, w, E, lane, k);
  for (int i = lane; i < E; i += kWave) hist[wave][i] = 0;   // own row: no barrier needed
  const int inv = count_keys<kSmallBatch>(k, w, E, key_bits, lane, hist[wave]);
  if (lane == 0) winv[wave] = inv;
  __syncthreads();
  wave_prefix(hist, E, nullptr, cnt);
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kAlignWaves; ++i) t += winv[i];
    *n_invalid = t;
  }
  finish_layout(cnt, tb, off, wsum, N, E, BM, rows_max, tiles_max, counts, offsets, tiles,
                num_tiles, sorted_slots);
  for (int i = lane; i < E; i += kWave) hist[wave][i] += off[i];   // this wave's next rows
  place_keys<kSmallBatch>(k, w, E, key_bits, lane, hist[wave], sorted_slots, slot_row);
}

__global__ __launch_bounds__(kAlignThreads) void align_small_kernel(
    const int32_t* __restrict__ ids, int N, int E, int BM, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  align_small(ids, N, E, BM, rows_max, tiles_max, counts, offsets, sorted_slots, slot_row, tiles,
              num_tiles, n_invalid);
}

// ---- more slots: count / scan / place ---------------------------------------------------
__device__ __forceinline__ void chunk_bounds(int c, int nchunks, int N, int& c0, int& c1) {
  c0 = c * kChunk;
  c1 = (c + 1 == nchunks) ? N : c0 + kChunk;
}

__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int N, int E, int nchunks, int32_t* __restrict__ slot_row) {
  __shared__ int hist[kAlignWaves][kAlignMaxExperts];
  __shared__ int winv[kAlignWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int key_bits = 32 - __clz(E);
  int c0, c1;
  chunk_bounds(blockIdx.x, nchunks, N, c0, c1);
  const WaveRange w = wave_range<kChunkBatch>(c0, c1, wave);
  int k[kChunkBatch];
  load_keys<kChunkBatch>(ids, w, E, lane, k);
  for (int i = lane; i < E; i += kWave) hist[wave][i] = 0;
  const int inv = count_keys<kChunkBatch>(k, w, E, key_bits, lane, hist[wave]);
  if (lane == 0) winv[wave] = inv;
  __syncthreads();
  // the chunk's counts (and invalid count) go to slot_row[c0 .. c0 + E]
  for (int e = threadIdx.x; e < E; e += kAlignThreads) {
    int t = 0;
    #pragma unroll
    for (int i = 0; i < kAlignWaves; ++i) t += hist[i][e];
    slot_row[c0 + e] = t;
  }
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kAlignWaves; ++i) t += winv[i];
    slot_row[c0 + E] = t;
  }
}

__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(
    int N, int E, int BM, int nchunks, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  __shared__ int cnt[kAlignMaxExperts];
  __shared__ int tb[kAlignMaxExperts + 1];
  __shared__ int off[kAlignMaxExperts + 1];
  __shared__ int wsum[kAlignWaves];
  // per expert: chunk counts -> chunk's first row within the expert (8 loads in flight)
  constexpr int U = 8;
  for (int e = threadIdx.x; e <= E; e += kAlignThreads) {   // e == E: the invalid counts
    int run = 0;
    for (int c = 0; c < nchunks; c += U) {
      int v[U];
      #pragma unroll
      for (int u = 0; u < U; ++u) v[u] = (c + u < nchunks) ? slot_row[(c + u) * kChunk + e] : 0;
      #pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c + u < nchunks && e < E) slot_row[(c + u) * kChunk + e] = run;
        run += v[u];
      }
    }
    if (e < E) cnt[e] = run; else *n_invalid = run;
  }
  finish_layout(cnt, tb, off, wsum, N, E, BM, rows_max, tiles_max, counts, offsets, tiles,
                num_tiles, sorted_slots);
}

__global__ __launch_bounds__(kAlignThreads) void align_place_kernel(
    const int32_t* __restrict__ ids, int N, int E, int nchunks,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ slot_row) {
  __shared__ int hist[kAlignWaves][kAlignMaxExperts];
  __shared__ int base[kAlignMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int key_bits = 32 - __clz(E);
  int c0, c1;
  chunk_bounds(blockIdx.x, nchunks, N, c0, c1);
  const WaveRange w = wave_range<kChunkBatch>(c0, c1, wave);
  int k[kChunkBatch];
  load_keys<kChunkBatch>(ids, w, E, lane, k);
  for (int e = threadIdx.x; e < E; e += kAlignThreads) base[e] = offsets[e] + slot_row[c0 + e];
  for (int i = lane; i < E; i += kWave) hist[wave][i] = 0;
  count_keys<kChunkBatch>(k, w, E, key_bits, lane, hist[wave]);
  __syncthreads();   // base[] read from slot_row before any of it is overwritten
  wave_prefix(hist, E, base, nullptr);
  __syncthreads();
  place_keys<kChunkBatch>(k, w, E, key_bits, lane, hist[wave], sorted_slots, slot_row);
}

hipError_t launch_align(const Resolved& r, const int32_t* ids, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles,
                        int32_t* num_tiles, int32_t* n_invalid, hipStream_t s) {
  const int N = (int)r.N;
  if (N <= kSmallN) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, N, r.E, r.BM,
                       (int)r.rows_max, (int)r.tiles_max, counts, offsets, sorted_slots, slot_row,
                       tiles, num_tiles, n_invalid);
    return hipGetLastError();
  }
  const int nchunks = N / kChunk;   // >= 4; the last chunk takes the remainder (< 2 * kChunk)
  hipLaunchKernelGGL(align_count_kernel, dim3(nchunks), dim3(kAlignThreads), 0, s, ids, N, r.E,
                     nchunks, slot_row);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kAlignThreads), 0, s, N, r.E, r.BM, nchunks,
                     (int)r.rows_max, (int)r.tiles_max, counts, offsets, sorted_slots, slot_row,
                     tiles, num_tiles, n_invalid);
  hipLaunchKernelGGL(align_place_kernel, dim3(nchunks), dim3(kAlignThreads), 0, s, ids, N, r.E,
                     nchunks, offsets, sorted_slots, slot_row);
  return hipGetLastError();
}

}  // namespace moe
