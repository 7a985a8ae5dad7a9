// Router producer for one token, one wavefront: logits [E] -> the top_k experts and weights.
//
// Sources: "MOE Bmm1 Fused Gather" (bench setup: topk(logits, experts_per_token,
// apply_softmax=True), then the expert histogram col_sum) and "factor_moe_fused_gemm.cu"
// ("factor 0", topk_softmax, yielding topk_weights and topk_ids).  Reading: softmax over all E
// logits; the top_k experts in descending probability, ties to the lower expert id; their
// probabilities as weights, renormalised to sum 1 when asked.  Softmax is strictly increasing
// in the logit, so the selection compares the fp32 logits themselves (exactly).
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kRouteMaxK = 64;   // one selected expert per lane

// Lane l holds logits l, l+64, ..., l+64*(LPL-1) (E <= 64*LPL).  On return lane j < K holds
// the j-th choice (id, weight).  The max and the sum of exponentials are wavefront butterfly
// reductions; each of the K rounds is a wavefront argmax over (logit, lowest id).
template <int LPL>
__device__ __forceinline__ void route_token(const float* __restrict__ lg, int E, int K,
                                            bool renorm, int lane, int& my_id, float& my_w) {
  float v[LPL];
  #pragma unroll
  for (int i = 0; i < LPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? lg[e] : -INFINITY;
  }
  float m = -INFINITY;
  #pragma unroll
  for (int i = 0; i < LPL; ++i) m = fmaxf(m, v[i]);
  #pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
  float s = 0.0f;
  #pragma unroll
  for (int i = 0; i < LPL; ++i)
    if (lane + kWave * i < E) s += expf(v[i] - m);
  #pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);

  uint32_t taken = 0;          // bit i: v[i] already chosen
  float sel_sum = 0.0f;
  my_id = -1;
  my_w = 0.0f;
  for (int j = 0; j < K; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    #pragma unroll
    for (int i = 0; i < LPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
    #pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oi = __shfl_xor(bi, d, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << ((bi / kWave) & 31);
    const float p = expf(bv - m) / s;
    sel_sum += p;
    if (lane == j) {
      my_id = bi;
      my_w = p;
    }
  }
  if (renorm) my_w = my_w / sel_sum;
}

// Logits per lane for E experts (1, 2, 4, 8 or 16).
inline int route_lpl(int E) {
  int l = 1;
  while (l * kWave < E) l *= 2;
  return l;
}

}  // namespace moe
