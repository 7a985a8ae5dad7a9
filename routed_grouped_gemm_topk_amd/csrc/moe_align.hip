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
//
// moe_route_align's one-launch form (router producer, then this alignment) is here too:
// route_align_kernel, below.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_route.h"


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
// COHERENT: device-scope loads, for ids that other workgroups of the same launch wrote with
// device-scope stores (they bypass a stale line in this XCD's L2).
template <int BATCH, bool COHERENT = false>
__device__ __forceinline__ void load_keys(const int32_t* ids, WaveRange w, int E, int lane,
                                          int* k) {
  #pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    const int s = w.begin + u * kWave + lane;
    if constexpr (COHERENT) {
      // unconditional (in-bounds) loads: a load under the condition is waited for on its own
      const int v = __hip_atomic_load(ids + (s < w.end ? s : 0), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      k[u] = (s < w.end) ? v : E;
    } else {
      k[u] = (s < w.end) ? ids[s] : E;
    }
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

// Scratch of an alignment workgroup (LDS), shared by every stage below.
struct AlignLds {
  int hist[kAlignWaves][kAlignMaxExperts];   // per-wave counts -> next rows
  int cnt[kAlignMaxExperts];                 // counts per expert (place: first row per expert)
  int tb[kAlignMaxExperts + 1];              // first tile per expert
  int off[kAlignMaxExperts + 1];             // first row per expert
  int wsum[kAlignWaves];
  int winv[kAlignWaves];
};

// Loads and stores of values that other workgroups of the same launch read or wrote: device
// scope, so they go past a stale line in this XCD's L2 (see route_align_kernel).
template <bool COHERENT>
__device__ __forceinline__ int ld_i32(const int32_t* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COHERENT>
__device__ __forceinline__ void st_i32(int32_t* p, int v) {
  if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// From L.cnt[e]: offsets, counts, tiles, num_tiles and the sentinel in every row that holds no
// slot.  Leaves L.off[] (first row of each expert, E+1 entries) in LDS.  Whole workgroup;
// starts and ends with a barrier.  COHERENT: offsets are read by other workgroups of the launch.
template <bool COHERENT = false>
__device__ void finish_layout(AlignLds& L, int N, int E, int BM, int rows_max, int tiles_max,
                              int32_t* counts, int32_t* offsets, int32_t* tiles,
                              int32_t* num_tiles, int32_t* sorted_slots) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  __syncthreads();
  // exclusive scan of m-blocks per expert (E <= 1024: one expert per thread)
  const int nb = (tid < E) ? (L.cnt[tid] + BM - 1) / BM : 0;
  int incl = nb;
  #pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) L.wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int v = (lane < kAlignWaves) ? L.wsum[lane] : 0;
    int iv = v;
    #pragma unroll
    for (int d = 1; d < kAlignWaves; d <<= 1) {
      int y = __shfl_up(iv, d, kWave);
      if (lane >= d) iv += y;
    }
    if (lane < kAlignWaves) L.wsum[lane] = iv - v;   // exclusive wave prefix
  }
  __syncthreads();
  const int excl = incl - nb + L.wsum[wave];
  if (tid < E) {
    L.tb[tid] = excl;
    L.off[tid] = excl * BM;
    if (tid == E - 1) { L.tb[E] = excl + nb; L.off[E] = (excl + nb) * BM; }
  }
  __syncthreads();

  const int total_tiles = L.tb[E];
  for (int e = tid; e <= E; e += kAlignThreads) {
    st_i32<COHERENT>(offsets + e, L.off[e]);
    if (e < E) counts[e] = L.cnt[e];
  }
  if (tid == 0) *num_tiles = total_tiles;
  for (int i = tid; i < tiles_max; i += kAlignThreads) {
    int e = -1, r = -1;
    if (i < total_tiles) {
      e = upper_index(L.tb, E, i);
      r = L.off[e] + (i - L.tb[e]) * BM;
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
      for (int r = L.off[e] + L.cnt[e] + lane; r < L.off[e + 1]; r += kWave) sorted_slots[r] = N;
  } else {
    for (int e = tid; e < E; e += kAlignThreads)
      for (int r = L.off[e] + L.cnt[e]; r < L.off[e + 1]; ++r) sorted_slots[r] = N;
  }
  for (int r = L.off[E] + tid; r < rows_max; r += kAlignThreads) sorted_slots[r] = N;
  __syncthreads();
}

// ---- up to kSmallN slots: one workgroup ---------------------------------------------------
// Each wave holds up to BATCH steps of 64 keys: N <= 16 * 64 * BATCH.
template <int BATCH, bool COHERENT = false>
__device__ __forceinline__ void align_small(
    AlignLds& L, const int32_t* ids, int N, int E, int BM, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int key_bits = 32 - __clz(E);        // keys 0..E (E = excluded / past the end)

  const WaveRange w = wave_range<BATCH>(0, N, wave);
  int k[BATCH];
  load_keys<BATCH, COHERENT>(ids, w, E, lane, k);
  for (int i = lane; i < E; i += kWave) L.hist[wave][i] = 0;   // own row: no barrier needed
  const int inv = count_keys<BATCH>(k, w, E, key_bits, lane, L.hist[wave]);
  if (lane == 0) L.winv[wave] = inv;
  __syncthreads();
  wave_prefix(L.hist, E, nullptr, L.cnt);
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kAlignWaves; ++i) t += L.winv[i];
    *n_invalid = t;
  }
  finish_layout(L, N, E, BM, rows_max, tiles_max, counts, offsets, tiles, num_tiles, sorted_slots);
  for (int i = lane; i < E; i += kWave) L.hist[wave][i] += L.off[i];   // this wave's next rows
  place_keys<BATCH>(k, w, E, key_bits, lane, L.hist[wave], sorted_slots, slot_row);
}

__global__ __launch_bounds__(kAlignThreads) void align_small_kernel(
    const int32_t* __restrict__ ids, int N, int E, int BM, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  __shared__ AlignLds L;
  align_small<kSmallBatch>(L, ids, N, E, BM, rows_max, tiles_max, counts, offsets, sorted_slots,
                           slot_row, tiles, num_tiles, n_invalid);
}

// ---- more slots: count / scan / place ---------------------------------------------------
__device__ __forceinline__ void chunk_bounds(int c, int nchunks, int N, int& c0, int& c1) {
  c0 = c * kChunk;
  c1 = (c + 1 == nchunks) ? N : c0 + kChunk;
}

// Chunk c's counts (and invalid count) -> slot_row[c0 .. c0 + E].
template <bool COHERENT = false>
__device__ void count_chunk(AlignLds& L, const int32_t* ids, int N, int E, int nchunks, int c,
                            int32_t* slot_row) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int key_bits = 32 - __clz(E);
  int c0, c1;
  chunk_bounds(c, nchunks, N, c0, c1);
  const WaveRange w = wave_range<kChunkBatch>(c0, c1, wave);
  int k[kChunkBatch];
  load_keys<kChunkBatch, COHERENT>(ids, w, E, lane, k);
  for (int i = lane; i < E; i += kWave) L.hist[wave][i] = 0;
  const int inv = count_keys<kChunkBatch>(k, w, E, key_bits, lane, L.hist[wave]);
  if (lane == 0) L.winv[wave] = inv;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kAlignThreads) {
    int t = 0;
    #pragma unroll
    for (int i = 0; i < kAlignWaves; ++i) t += L.hist[i][e];
    st_i32<COHERENT>(slot_row + c0 + e, t);
  }
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kAlignWaves; ++i) t += L.winv[i];
    st_i32<COHERENT>(slot_row + c0 + E, t);
  }
}

// Per expert: chunk counts -> each chunk's first row within the expert (in place), then the
// layout.  One workgroup.
template <bool COHERENT = false>
__device__ void scan_chunks(AlignLds& L, int N, int E, int BM, int nchunks, int rows_max,
                            int tiles_max, int32_t* counts, int32_t* offsets,
                            int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles,
                            int32_t* num_tiles, int32_t* n_invalid) {
  constexpr int U = 8;   // loads in flight
  for (int e = threadIdx.x; e <= E; e += kAlignThreads) {   // e == E: the invalid counts
    int run = 0;
    for (int c = 0; c < nchunks; c += U) {
      int v[U];
      #pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x = ld_i32<COHERENT>(slot_row + min(c + u, nchunks - 1) * kChunk + e);
        v[u] = (c + u < nchunks) ? x : 0;
      }
      #pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c + u < nchunks && e < E) st_i32<COHERENT>(slot_row + (c + u) * kChunk + e, run);
        run += v[u];
      }
    }
    if (e < E) L.cnt[e] = run; else *n_invalid = run;
  }
  finish_layout<COHERENT>(L, N, E, BM, rows_max, tiles_max, counts, offsets, tiles, num_tiles,
                          sorted_slots);
}

// Chunk c's slots to their rows: offsets[e] + the chunk's first row within expert e
// (slot_row[c0 + e], left by scan_chunks) + the slot's rank within the chunk.
template <bool COHERENT = false>
__device__ void place_chunk(AlignLds& L, const int32_t* ids, int N, int E, int nchunks, int c,
                            const int32_t* offsets, int32_t* sorted_slots, int32_t* slot_row) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int key_bits = 32 - __clz(E);
  int c0, c1;
  chunk_bounds(c, nchunks, N, c0, c1);
  const WaveRange w = wave_range<kChunkBatch>(c0, c1, wave);
  int k[kChunkBatch];
  load_keys<kChunkBatch, COHERENT>(ids, w, E, lane, k);
  for (int e = threadIdx.x; e < E; e += kAlignThreads)
    L.cnt[e] = ld_i32<COHERENT>(offsets + e) + ld_i32<COHERENT>(slot_row + c0 + e);
  for (int i = lane; i < E; i += kWave) L.hist[wave][i] = 0;
  count_keys<kChunkBatch>(k, w, E, key_bits, lane, L.hist[wave]);
  __syncthreads();   // L.cnt[] read from slot_row before any of it is overwritten
  wave_prefix(L.hist, E, L.cnt, nullptr);
  __syncthreads();
  place_keys<kChunkBatch>(k, w, E, key_bits, lane, L.hist[wave], sorted_slots, slot_row);
}

__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int N, int E, int nchunks, int32_t* __restrict__ slot_row) {
  __shared__ AlignLds L;
  count_chunk(L, ids, N, E, nchunks, blockIdx.x, slot_row);
}

__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(
    int N, int E, int BM, int nchunks, int rows_max, int tiles_max,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid) {
  __shared__ AlignLds L;
  scan_chunks(L, N, E, BM, nchunks, rows_max, tiles_max, counts, offsets, sorted_slots, slot_row,
              tiles, num_tiles, n_invalid);
}

__global__ __launch_bounds__(kAlignThreads) void align_place_kernel(
    const int32_t* __restrict__ ids, int N, int E, int nchunks,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ slot_row) {
  __shared__ AlignLds L;
  place_chunk(L, ids, N, E, nchunks, blockIdx.x, offsets, sorted_slots, slot_row);
}

// ---- routing and alignment in one launch (up to kSmallN slots) ----------------------------
// The routing stays spread over the GPU: workgroup b routes tokens tpw*b .. tpw*b + tpw - 1,
// one wave per token (route_token), and writes their ids and weights; then it takes a ticket
// from a completion counter.  The workgroup that draws the last ticket has every other
// workgroup's ids in hand and aligns them (align_small).  No workgroup waits for another, so
// the launch ends whatever the order and residency of its workgroups.
//
// Hand-over of the ids across the XCDs' L2 caches: they are written with device-scope stores
// (coherent across the XCDs), each wave waits for its stores to complete before the workgroup
// barrier that precedes the ticket, the ticket is a device-scope atomic, and the aligning
// workgroup reads the ids with device-scope loads, which do not return a stale line of its
// own XCD's L2.
// A release/acquire pair on the ticket (a write-back of the whole L2 in every workgroup, an
// invalidation in the last) gives the same result and was measured slower.
//
// The counter is one of kTicketSlots, taken in turn per call on the host; the workgroup that
// draws the last ticket sets it back to zero.  Calls that run at the same time (several
// streams) use different counters as long as fewer than kTicketSlots of them overlap.  (A
// two-level ticket, workgroups counting into 8 group counters and the last of each group into
// a top counter, was measured: 1 us slower, one more dependent atomic.)
constexpr int kTicketSlots = 64;
__device__ int g_route_ticket[kTicketSlots];

template <int LPL>
__global__ __launch_bounds__(kAlignThreads) void route_align_kernel(
    const float* __restrict__ logits, int T, int K, int renorm, int E, int BM, int rows_max,
    int tiles_max, int tpw, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ n_invalid, int* __restrict__ ticket) {
  __shared__ AlignLds L;
  __shared__ int last;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * tpw + wave;
  if (wave < tpw && t < T) {                       // wave-uniform
    int id;
    float w;
    route_token<LPL>(logits + (size_t)t * E, E, K, renorm != 0, lane, id, w);
    if (lane < K) {
      st_i32<true>(topk_ids + (size_t)t * K + lane, id);
      topk_w[(size_t)t * K + lane] = w;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    last = (__hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (int)gridDim.x - 1);
    if (last) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  align_small<kSmallBatch, true>(L, topk_ids, T * K, E, BM, rows_max, tiles_max, counts, offsets,
                                 sorted_slots, slot_row, tiles, num_tiles, n_invalid);
}

namespace {
std::mutex g_ticket_mu;
int* g_ticket_base[64];   // device address of g_route_ticket per device ordinal
std::atomic<unsigned> g_ticket_calls{0};

// This call's ticket on the current device (null on failure).
int* next_ticket() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  int* base;
  {
    std::lock_guard<std::mutex> g(g_ticket_mu);
    if (!g_ticket_base[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_route_ticket)) != hipSuccess || !p) return nullptr;
      g_ticket_base[dev] = (int*)p;
    }
    base = g_ticket_base[dev];
  }
  return base + g_ticket_calls.fetch_add(1, std::memory_order_relaxed) % kTicketSlots;
}
}  // namespace

bool route_align_one_launch(const Resolved& r) {
  return r.N <= kSmallN && r.K <= kRouteMaxK && r.E <= 16 * kWave;
}

hipError_t launch_route_align_one(const Resolved& r, const float* logits, int renorm,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  int32_t* offsets, int32_t* sorted_slots, int32_t* slot_row,
                                  int32_t* tiles, int32_t* num_tiles, int32_t* n_invalid,
                                  hipStream_t s) {
  if (!route_align_one_launch(r)) return hipErrorInvalidValue;
  int* ticket = next_ticket();
  if (!ticket) return hipErrorInvalidSymbol;
  // tokens per workgroup: one per compute unit up to 256 tokens (a token's routing is a
  // chain of dependent wavefront steps; waves sharing a SIMD would take turns), at most 16
  const int tpw = std::min(kAlignWaves, std::max(1, (r.T + 255) / 256));
  const unsigned blocks = (unsigned)((r.T + tpw - 1) / tpw);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kAlignThreads), 0, s, logits, (int)r.T, r.K,
                       renorm, r.E, r.BM, (int)r.rows_max, (int)r.tiles_max, tpw, topk_ids, topk_w,
                       counts, offsets, sorted_slots, slot_row, tiles, num_tiles, n_invalid,
                       ticket);
    return hipGetLastError();
  };
  switch (route_lpl(r.E)) {
    case 1: return go(route_align_kernel<1>);
    case 2: return go(route_align_kernel<2>);
    case 4: return go(route_align_kernel<4>);
    case 8: return go(route_align_kernel<8>);
    case 16: return go(route_align_kernel<16>);
    default: return hipErrorInvalidValue;
  }
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
