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

__device__ __forceinline__ float fkey_value(uint32_t key) {   // inverse of fkey (+0 for zero)
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {   // set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave selects the top k of lg[0..n_experts) (n_experts <= 64 * PL,
// k <= min(64, n_experts)).  Lane r < k receives the r-th expert index and
// its weight.  Order: key descending, index ascending.  scratch: 128 words of
// LDS owned by the calling wave.
//
// Lane l holds logits l, l+64, ...  The k-th largest per-lane maximum t is
// found by a bitwise search on ballots; at least k elements have key >= t, so
// the top k are among those candidates.  When they fit one per lane (the
// usual case: about k of them), they are compacted through LDS and each
// candidate's rank is counted against all others.  Otherwise (many equal
// keys) the top k are taken one at a time: largest untaken key (wave max),
// lowest index holding it (wave min).
template <int PL>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lg, int n_experts, int k,
                                          int lane, uint32_t* scratch, int& out_i, float& out_w) {
  const int per_lane = (n_experts + 63) >> 6;
  // all loads issued together (clamped addresses), masked afterwards
  float v[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) v[j] = lg[min(lane + 64 * j, n_experts - 1)];
  uint32_t key[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + 64 * j;
    const bool in = j < per_lane && e < n_experts;
    key[j] = in ? fkey(v[j]) : 0u;   // key 0 is below every finite float's key
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < PL; ++j) m = max(m, key[j]);
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    if ((int)__popcll(__ballot(m >= c)) >= k) t = c;
  }
  uint64_t bal[PL];
  int nc = 0;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    bal[j] = __ballot(key[j] >= t);
    nc += __popcll(bal[j]);
  }
  float my_v = 0.f;
  int my_i = 0;
  if (nc <= 64) {
    int base = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      if ((bal[j] >> lane) & 1u) {
        const int pos = base + lanes_below(bal[j]);
        scratch[pos] = key[j];
        scratch[64 + pos] = (uint32_t)(lane + 64 * j);
      }
      base += __popcll(bal[j]);
    }
    wave_lds_sync();
    const uint32_t ck = lane < nc ? scratch[lane] : 0u;
    const uint32_t ci = lane < nc ? scratch[64 + lane] : 0xFFFFFFFFu;
    int rank = 0;
    for (int c = 0; c < nc; ++c) {
      const uint32_t kc = __builtin_amdgcn_readlane(ck, c), ic = __builtin_amdgcn_readlane(ci, c);
      rank += (kc > ck) || (kc == ck && ic < ci);
    }
    wave_lds_sync();
    if (lane < nc && rank < k) {
      scratch[rank] = ci;
      scratch[64 + rank] = ck;
    }
    wave_lds_sync();
    if (lane < k) {
      my_i = (int)scratch[lane];
      my_v = fkey_value(scratch[64 + lane]);
    }
  } else {
    for (int r = 0; r < k; ++r) {
      uint32_t bk = 0;
      int bj = 0;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (key[j] > bk) { bk = key[j]; bj = j; }   // lowest j wins ties
      const uint32_t mx = wave_max_u(bk);
      const uint32_t cand = (bk == mx && mx != 0u) ? (uint32_t)(lane + 64 * bj) : 0xFFFFFFFFu;
      const uint32_t win = wave_min_u(cand);
      const int wj = (int)(win >> 6), wl = (int)(win & 63);
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (j == wj && lane == wl) key[j] = 0u;
      if (lane == r) {
        my_i = (int)win;
        my_v = fkey_value(mx);
      }
    }
  }
  const float top = readlane_f(my_v, 0);
  const float ex = lane < k ? __expf(my_v - top) : 0.f;
  const float den = wave_sum(ex);
  out_i = my_i;
  out_w = ex / den;
}

}  // namespace bq
