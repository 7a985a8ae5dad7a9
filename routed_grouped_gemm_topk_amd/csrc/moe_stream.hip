// HBM-streaming kernels: the per-(row, 128-group) e4m3 quantisation of X and the
// deterministic per-token combine.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// X quantisation ("MOE Bmm1 Fused Gather", pack_e4m3x2: round to nearest even with
// saturation to the largest finite e4m3 value).  16 lanes per 128-column group, 8 bf16
// values (16 bytes) per lane, 4 groups per wavefront: the group amax is a 16-lane max
// reduction, s = amax/448 (IEEE division), codes = e4m3(x/s) (IEEE division).
// ---------------------------------------------------------------------------------------------
constexpr int kQuantThreads = 256;
constexpr int kQuantLanes = kGroup / 8;                            // lanes per group
constexpr int kQuantGroupsPerBlock = kQuantThreads / kQuantLanes;  // 16

__global__ __launch_bounds__(kQuantThreads) void quant_rows_e4m3_kernel(
    const i32x4* __restrict__ x8, uint2* __restrict__ xq8, float* __restrict__ scales,
    int64_t n_groups) {
  const int sub = threadIdx.x & (kQuantLanes - 1);
  const int64_t grp = (int64_t)blockIdx.x * kQuantGroupsPerBlock + threadIdx.x / kQuantLanes;
  const bool live = grp < n_groups;
  float v[8];
  float m = 0.0f;
  if (live) {
    const i32x4 w = x8[grp * kQuantLanes + sub];
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32((uint32_t)w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32((uint32_t)w[i] >> 16);
    }
    #pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  // the 16 lanes of a group are aligned within the wavefront: xor offsets below 16 stay in it
  #pragma unroll
  for (int d = kQuantLanes / 2; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
  if (!live) return;
  const float s = (m == 0.0f) ? 1.0f : m / kE4M3Max;
  uint32_t lo = 0, hi = 0;
  #pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3(v[i] / s) << (8 * i);
    hi |= f32_to_e4m3(v[4 + i] / s) << (8 * i);
  }
  xq8[grp * kQuantLanes + sub] = make_uint2(lo, hi);
  if (sub == 0) scales[grp] = s;
}

hipError_t launch_quant_rows(const Resolved& r, const void* x, uint8_t* xq, float* scales,
                             hipStream_t s) {
  const int64_t groups = (int64_t)r.T * (r.H / kGroup);
  const int64_t blocks = (groups + kQuantGroupsPerBlock - 1) / kQuantGroupsPerBlock;
  hipLaunchKernelGGL(quant_rows_e4m3_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, s,
                     (const i32x4*)x, (uint2*)xq, scales, groups);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine ("factor_moe_fused_gemm.cu": index_add_ in the slow path and
// weighted_scatter_add_kernel, which there adds with float atomics).  Here each thread
// owns 16 bytes of one token's output row and adds that token's top_k slot rows in
// ascending j in fp32, then rounds once: no atomics, same bits on every run.
// ---------------------------------------------------------------------------------------------
constexpr int kCombineThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const i32x4* __restrict__ slot_out, const int32_t* __restrict__ slot_row,
    i32x4* __restrict__ out, int T, int top_k, int vec_per_row) {
  const int64_t idx = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (idx >= (int64_t)T * vec_per_row) return;
  const int t = (int)(idx / vec_per_row);
  const int c = (int)(idx - (int64_t)t * vec_per_row);
  constexpr int L = BF16 ? 8 : 4;
  float acc[L];
  #pragma unroll
  for (int i = 0; i < L; ++i) acc[i] = 0.0f;
  // slots in batches of 4: every row load of a batch is issued before the first add.  A slot
  // with an excluded id (another shard's expert) was never written and is not read: on an
  // expert-parallel shard most slots are such.
  constexpr int U = 4;
  for (int j0 = 0; j0 < top_k; j0 += U) {
    int ok[U];
    i32x4 v[U];
    #pragma unroll
    for (int u = 0; u < U; ++u)
      ok[u] = (j0 + u < top_k) ? slot_row[(int64_t)t * top_k + j0 + u] >= 0 : 0;
    #pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = (int64_t)t * top_k + j0 + u;
      v[u] = ok[u] ? slot_out[s * vec_per_row + c] : i32x4{0, 0, 0, 0};
    }
    #pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      if (BF16) {
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_bits_to_f32((uint32_t)v[u][i] & 0xFFFFu);
          acc[2 * i + 1] += bf16_bits_to_f32((uint32_t)v[u][i] >> 16);
        }
      } else {
        #pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += __int_as_float(v[u][i]);
      }
    }
  }
  i32x4 o;
  if (BF16) {
    #pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (int)pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  } else {
    #pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_int(acc[i]);
  }
  out[idx] = o;
}

hipError_t launch_combine(const Resolved& r, const void* slot_out, const int32_t* slot_row,
                          void* out, hipStream_t s) {
  const bool bf16 = (r.dtype == MOE_BF16);
  const int vec_per_row = r.H * (bf16 ? 2 : 4) / 16;
  const int64_t total = (int64_t)r.T * vec_per_row;
  const unsigned blocks = (unsigned)((total + kCombineThreads - 1) / kCombineThreads);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(kCombineThreads), 0, s,
                       (const i32x4*)slot_out, slot_row, (i32x4*)out, r.T, r.K, vec_per_row);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(kCombineThreads), 0, s,
                       (const i32x4*)slot_out, slot_row, (i32x4*)out, r.T, r.K, vec_per_row);
  return hipGetLastError();
}

}  // namespace moe
