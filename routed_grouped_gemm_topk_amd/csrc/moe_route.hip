// Router producer: logits [T, E] (fp32) -> topk_ids [T, K] (int32), topk_weights [T, K] (fp32).
// One wavefront per token (route_token in moe_route.h), four tokens per workgroup.
#include "moe_route.h"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouteTokensPerBlock = kRouteThreads / kWave;

template <int LPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ logits, int T, int E, int K, int renorm,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteTokensPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int id;
  float w;
  route_token<LPL>(logits + (size_t)t * E, E, K, renorm != 0, lane, id, w);
  if (lane < K) {
    topk_ids[(size_t)t * K + lane] = id;
    topk_w[(size_t)t * K + lane] = w;
  }
}

hipError_t launch_route(const Resolved& r, const float* logits, int renorm, int32_t* topk_ids,
                        float* topk_w, hipStream_t s) {
  const unsigned blocks = (unsigned)((r.T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock);
  switch (route_lpl(r.E)) {
#define MOE_ROUTE_CASE(L)                                                                     \
  case L:                                                                                    \
    hipLaunchKernelGGL(route_kernel<L>, dim3(blocks), dim3(kRouteThreads), 0, s, logits, r.T, \
                       r.E, r.K, renorm, topk_ids, topk_w);                                  \
    break;
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Routing, then alignment of its ids.  Up to kSmallN slots one launch does both
// (route_align_kernel in moe_align.hip: routing spread over the GPU, the last workgroup to
// finish aligns).  Above that the alignment itself needs several workgroups for its count and
// placement, which wait on one another; handing work between them inside one launch (each
// hand-over a device-scope counter that the waiting workgroups poll, then device-scope loads
// of what the others wrote) was measured slower than the kernel boundaries, so larger
// problems run the routing launch, then the alignment launches, on one stream.
hipError_t launch_route_align(const Resolved& r, const float* logits, int renorm, int32_t* topk_ids,
                              float* topk_w, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles,
                              int32_t* num_tiles, int32_t* n_invalid, hipStream_t s) {
  if (route_align_one_launch(r))
    return launch_route_align_one(r, logits, renorm, topk_ids, topk_w, counts, offsets,
                                  sorted_slots, slot_row, tiles, num_tiles, n_invalid, s);
  hipError_t e = launch_route(r, logits, renorm, topk_ids, topk_w, s);
  if (e != hipSuccess) return e;
  return launch_align(r, topk_ids, counts, offsets, sorted_slots, slot_row, tiles, num_tiles,
                      n_invalid, s);
}

}  // namespace moe
