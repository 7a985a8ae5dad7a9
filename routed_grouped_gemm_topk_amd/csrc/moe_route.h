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

// Wavefront all-reductions from short-latency lane exchanges (gfx950): inside each 16-lane
// row, the quad permutes [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors; across
// rows, v_permlane16_swap (rows 0<->1, 2<->3) and v_permlane32_swap (halves).  Each step
// combines a lane's value with one other lane's, the pairs covering the wave after six
// steps, so every lane ends with the combination of all 64.  The combine must be commutative
// (both lanes of a pair then compute the same value).
template <int CTRL>
__device__ __forceinline__ int dpp_xchg(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_xchg(float v) {
  return __builtin_bit_cast(float, dpp_xchg<CTRL>(__builtin_bit_cast(int, v)));
}
template <class T, class F>
__device__ __forceinline__ T wave_allreduce(T v, F combine) {
  v = combine(v, dpp_xchg<0xB1>(v));    // quad_perm 1,0,3,2
  v = combine(v, dpp_xchg<0x4E>(v));    // quad_perm 2,3,0,1
  v = combine(v, dpp_xchg<0x141>(v));   // row_half_mirror
  v = combine(v, dpp_xchg<0x140>(v));   // row_mirror
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = combine(__builtin_bit_cast(T, (uint32_t)r16[0]), __builtin_bit_cast(T, (uint32_t)r16[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return combine(__builtin_bit_cast(T, (uint32_t)r32[0]), __builtin_bit_cast(T, (uint32_t)r32[1]));
}

// Wavefront argmax of (value, id), larger value first, ties to the lower id (a total order,
// so the pairwise choice is commutative).
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  auto better = [](float av, int ai, float ov, int oi) {
    return ov > av || (ov == av && oi < ai);
  };
  auto step_dpp = [&](float ov, int oi) {
    if (better(bv, bi, ov, oi)) { bv = ov; bi = oi; }
  };
  step_dpp(dpp_xchg<0xB1>(bv), dpp_xchg<0xB1>(bi));
  step_dpp(dpp_xchg<0x4E>(bv), dpp_xchg<0x4E>(bi));
  step_dpp(dpp_xchg<0x141>(bv), dpp_xchg<0x141>(bi));
  step_dpp(dpp_xchg<0x140>(bv), dpp_xchg<0x140>(bi));
  auto step_swap = [&](auto swap) {
    const auto v2 = swap(__builtin_bit_cast(uint32_t, bv));
    const auto i2 = swap((uint32_t)bi);
    float av = __builtin_bit_cast(float, (uint32_t)v2[0]);
    int ai = (int)i2[0];
    const float ov = __builtin_bit_cast(float, (uint32_t)v2[1]);
    const int oi = (int)i2[1];
    if (better(av, ai, ov, oi)) { av = ov; ai = oi; }
    bv = av;
    bi = ai;
  };
  step_swap([](uint32_t x) { return __builtin_amdgcn_permlane16_swap(x, x, false, false); });
  step_swap([](uint32_t x) { return __builtin_amdgcn_permlane32_swap(x, x, false, false); });
}

// Lane l holds logits l, l+64, ..., l+64*(LPL-1) (E <= 64*LPL).  On return lane j < K holds
// the j-th choice (id, weight).  The max and the sum of exponentials are wavefront
// all-reductions; each of the K rounds is a wavefront argmax over (logit, lowest id).  Every
// lane of the wave must be active.
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
  m = wave_allreduce(m, [](float a, float b) { return fmaxf(a, b); });
  float s = 0.0f;
  #pragma unroll
  for (int i = 0; i < LPL; ++i)
    if (lane + kWave * i < E) s += expf(v[i] - m);
  s = wave_allreduce(s, [](float a, float b) { return a + b; });

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
    wave_argmax(bv, bi);
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
