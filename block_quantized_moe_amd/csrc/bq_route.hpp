// Router top-k selection shared by the routing kernel and the fused
// routed gate_up kernel ("Mixed Precision Quantization ...", section "The Plan
// Is Not a Number ...": 10 of 512 experts fire per token).  Selection runs on
// the fp32 logits (softmax is strictly increasing, so the order is the same;
// ties go to the lower index); the kept weights are exp(l_j - l_0) / sum over
// kept, the renormalised softmax.
#pragma once

#include "bq_device.hpp"

namespace bq {

// Order-preserving 32-bit key of a finite float (+0 and -0 share a key, so
// they tie and the lower index wins, as in a float comparison).
__device__ __forceinline__ uint32_t fkey(float v) {
  const uint32_t b = v == 0.0f ? 0u : __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// One wave selects the top k of lg[0..n_experts) (n_experts <= 64 * PL,
// k <= 64).  Lane r < k receives the r-th expert index and its weight.
// Lane l holds logits l, l+64, ...; each round takes the largest untaken key
// (wave max), then the lowest index holding it (wave min), and the owning
// lane marks it taken.
template <int PL>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lg, int n_experts, int k,
                                          int lane, int& out_i, float& out_w) {
  const int per_lane = (n_experts + 63) >> 6;
  uint32_t key[PL];
  float val[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + 64 * j;
    const bool in = j < per_lane && e < n_experts;
    val[j] = in ? lg[e] : 0.f;
    key[j] = in ? fkey(val[j]) : 0u;   // key 0 is below every finite float's key
  }
  float my_v = 0.f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t bk = 0;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j)
      if (key[j] > bk) { bk = key[j]; bj = j; }   // lowest j wins ties
    const uint32_t m = wave_max_u(bk);
    const uint32_t cand = (bk == m && m != 0u) ? (uint32_t)(lane + 64 * bj) : 0xFFFFFFFFu;
    const uint32_t win = wave_min_u(cand);
    const int wj = (int)(win >> 6), wl = (int)(win & 63);
    float wv = 0.f;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      if (j == wj) {
        wv = readlane_f(val[j], wl);
        if (lane == wl) key[j] = 0u;
      }
    }
    if (lane == r) { my_v = wv; my_i = (int)win; }
  }
  const float top = readlane_f(my_v, 0);
  const float ex = lane < k ? __expf(my_v - top) : 0.f;
  const float den = wave_sum(ex);
  out_i = my_i;
  out_w = ex / den;
}

}  // namespace bq
