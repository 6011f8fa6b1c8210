// route_topk.h -- the router's per-token selection, shared by the top-k
// kernel of moe_route and the one-workgroup route-and-dispatch kernel of
// small batches (the same instructions either way, so the same bits).
//
// The layer definition fixes the router as softmax over all experts, top-k,
// and renormalisation of the k weights; softmax followed by renormalisation
// over the picks equals exp(l_j - l_max) / sum_{picks} exp(l_j' - l_max),
// and softmax is monotone, so the selection runs on the fp32 logits and only
// the k picks are exponentiated.
#pragma once

#include "moe_common.h"

namespace moe {

// Order used by the selection: higher score first, lower expert id on ties.
__device__ __forceinline__ bool topk_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One wavefront selects for token t (wave-uniform); lane l holds experts l,
// l+64, l+128, l+192 (E <= 256).  The logit of expert e is the sum of the
// `splits` partial logits in ascending split order, plus the bias; it is
// written to `logits` when that is given.  Then k rounds of a butterfly
// arg-max; round j's winner is recorded by lane j.
__device__ __forceinline__ void topk_token(const float* __restrict__ partial, int splits,
                                           const float* __restrict__ bias, int T, int E, int k, int t,
                                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                           float* __restrict__ logits) {
  const int lane = lane_id();
  float v[4];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    live[q] = e < E;
    float acc = 0.f;
    if (live[q]) {
      acc = partial[static_cast<size_t>(t) * E + e];
      for (int sp = 1; sp < splits; ++sp) acc += partial[(static_cast<size_t>(sp) * T + t) * E + e];
      if (bias) acc += bias[e];
      if (logits) logits[static_cast<size_t>(t) * E + e] = acc;
    }
    v[q] = acc;
  }
  float my_v = 0.f;
  int my_i = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (live[q] && topk_better(v[q], lane + 64 * q, bv, bi)) {
        bv = v[q];
        bi = lane + 64 * q;
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      if (topk_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the same winner (the order is a total order)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q == bi) live[q] = false;
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
  }
  const float vmax = __shfl(my_v, 0, kWave);
  const float ex = (lane < k) ? expf(my_v - vmax) : 0.f;
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, j, kWave);  // ascending rank order
  if (lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = my_i;
    topk_w[static_cast<size_t>(t) * k + lane] = ex / sum;
  }
}

}  // namespace moe
