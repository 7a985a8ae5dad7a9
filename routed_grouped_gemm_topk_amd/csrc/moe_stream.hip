// HBM-streaming kernels: the per-(row, 128-group) e4m3 quantisation of X and the
// deterministic per-token combine.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// X quantisation ("MOE Bmm1 Fused Gather", pack_e4m3x2: round to nearest even with
// saturation to the largest finite e4m3 value).  One wavefront per 128-column group:
// each lane owns two adjacent bf16 values, the group amax is a wavefront max
// reduction, s = amax/448 (IEEE division), codes = e4m3(x/s) (IEEE division).
// ---------------------------------------------------------------------------------------------
constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quant_rows_e4m3_kernel(
    const uint32_t* __restrict__ x_pairs, uint16_t* __restrict__ xq_pairs,
    float* __restrict__ scales, int64_t n_groups) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t grp = (int64_t)blockIdx.x * (kQuantThreads / kWave) + threadIdx.x / kWave;
  if (grp >= n_groups) return;
  const uint32_t v = x_pairs[grp * (kGroup / 2) + lane];
  const float a = bf16_bits_to_f32(v & 0xFFFFu);
  const float b = bf16_bits_to_f32(v >> 16);
  float m = fmaxf(fabsf(a), fabsf(b));
  #pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
  const float s = (m == 0.0f) ? 1.0f : m / kE4M3Max;
  const uint32_t qa = f32_to_e4m3(a / s);
  const uint32_t qb = f32_to_e4m3(b / s);
  xq_pairs[grp * (kGroup / 2) + lane] = (uint16_t)(qa | (qb << 8));
  if (lane == 0) scales[grp] = s;
}

hipError_t launch_quant_rows(const Resolved& r, const void* x, uint8_t* xq, float* scales,
                             hipStream_t s) {
  const int64_t groups = (int64_t)r.T * (r.H / kGroup);
  const int per_block = kQuantThreads / kWave;
  const int64_t blocks = (groups + per_block - 1) / per_block;
  hipLaunchKernelGGL(quant_rows_e4m3_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, s,
                     (const uint32_t*)x, (uint16_t*)xq, scales, groups);
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
  for (int j = 0; j < top_k; ++j) {
    const int64_t s = (int64_t)t * top_k + j;
    if (slot_row[s] < 0) continue;
    const i32x4 v = slot_out[s * vec_per_row + c];
    if (BF16) {
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_bits_to_f32((uint32_t)v[i] & 0xFFFFu);
        acc[2 * i + 1] += bf16_bits_to_f32((uint32_t)v[i] >> 16);
      }
    } else {
      #pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += __int_as_float(v[i]);
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
