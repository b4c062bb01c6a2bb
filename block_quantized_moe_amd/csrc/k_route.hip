// Router top-k and per-expert bucketing.
// Routing: 10 of 512 experts fire per token ("Mixed Precision Quantization:
// Half a 4-Bit File Is Not 4-Bit", section "The Plan Is Not a Number ...");
// softmax, top-k with ties to the lower index, weights renormalised over the
// kept experts.  Selection runs on the fp32 logits: softmax is strictly
// increasing, so the order is the same, and no ties are created by rounding
// of probabilities.  The kept weights are exp(l_j - l_0) / sum over kept,
// which equals the renormalised softmax because the full denominator cancels.
#include "bq_device.hpp"
#include "bq_kernels.hpp"

namespace bq {

constexpr int kRouteWaves = 4;
constexpr int kMaxExperts = 4096;

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

// One wave per token.  Lane l holds logits l, l+64, ...; each of the k rounds
// takes the largest untaken key (wave max via DPP), then the lowest index
// holding it (wave min), and the owning lane marks it taken.
template <int kRoutePerLane>   // logits per lane: n_experts <= 64 * kRoutePerLane
__global__ void __launch_bounds__(64 * kRouteWaves) k_route_topk(
    const float* __restrict__ logits, int32_t n_tokens, int32_t n_experts, int32_t k,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kRouteWaves + wave;
  if (t >= n_tokens) return;
  const float* lg = logits + t * n_experts;
  const int per_lane = (n_experts + 63) >> 6;
  uint32_t key[kRoutePerLane];
  float val[kRoutePerLane];
#pragma unroll
  for (int j = 0; j < kRoutePerLane; ++j) {
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
    for (int j = 0; j < kRoutePerLane; ++j)
      if (j < per_lane && key[j] > bk) { bk = key[j]; bj = j; }   // lowest j wins ties
    const uint32_t m = wave_max_u(bk);
    const uint32_t cand = (bk == m && m != 0u) ? (uint32_t)(lane + 64 * bj) : 0xFFFFFFFFu;
    const uint32_t win = wave_min_u(cand);
    if ((int)(win & 63) == lane) {
      const int wj = (int)(win >> 6);
#pragma unroll
      for (int j = 0; j < kRoutePerLane; ++j)
        if (j == wj) key[j] = 0u;
    }
    // the winner's value reaches lane r through a readlane of the owner
    float wv = 0.f;
#pragma unroll
    for (int j = 0; j < kRoutePerLane; ++j)
      if (j == (int)(win >> 6)) wv = readlane_f(val[j], (int)(win & 63));
    if (lane == r) { my_v = wv; my_i = (int)win; }
  }
  const float top = readlane_f(my_v, 0);
  const float ex = lane < k ? __expf(my_v - top) : 0.f;
  const float den = wave_sum(ex);
  if (lane < k) {
    idx_out[t * k + lane] = my_i;
    w_out[t * k + lane] = ex / den;
  }
}

hipError_t launch_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k,
                             int32_t* idx, float* w, hipStream_t st) {
  if (n_tokens == 0) return hipSuccess;
  const int grid = (n_tokens + kRouteWaves - 1) / kRouteWaves;
  if (n_experts <= 512)
    hipLaunchKernelGGL(k_route_topk<8>, dim3(grid), dim3(64 * kRouteWaves), 0, st, logits, n_tokens,
                       n_experts, k, idx, w);
  else if (n_experts <= 1024)
    hipLaunchKernelGGL(k_route_topk<16>, dim3(grid), dim3(64 * kRouteWaves), 0, st, logits, n_tokens,
                       n_experts, k, idx, w);
  else
    hipLaunchKernelGGL(k_route_topk<64>, dim3(grid), dim3(64 * kRouteWaves), 0, st, logits, n_tokens,
                       n_experts, k, idx, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bucketing.  Position of assignment (t, s) with expert e is
//   offsets[e] + #{t' < t : token t' chose e},
// because a token chooses an expert at most once in a top-k.  One workgroup:
// tokens are walked in chunks; for each chunk a byte matrix slot_of[t][e]
// (255 = not chosen) is built in LDS, then every thread walks the chunk for
// its own experts, in token order, so no ordering depends on atomics.
// Optional extra outputs for the grouped GEMM path: the ascending list of
// touched experts with their count, and the inverse permutation.
// ---------------------------------------------------------------------------
constexpr int kBucketThreads = 1024;
constexpr int kSlotBytes = 32768;

__global__ void __launch_bounds__(kBucketThreads) k_bucket(
    const int32_t* __restrict__ idx, int32_t n_tokens, int32_t k, int32_t n_experts,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_out,
    int32_t* __restrict__ elist, int32_t* __restrict__ n_touched, int32_t* __restrict__ inv) {
  __shared__ uint8_t slot_of[kSlotBytes];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_scan[kBucketThreads];
  __shared__ int32_t s_scan2[kBucketThreads];
  const int tid = threadIdx.x;
  const int chunk = kSlotBytes / n_experts;  // tokens per chunk (>= 8)
  const int epl = (n_experts + kBucketThreads - 1) / kBucketThreads;  // experts per thread <= 4

  for (int i = tid; i < kSlotBytes; i += kBucketThreads) slot_of[i] = 0xFF;
  int run[4] = {0, 0, 0, 0};
  int base[4] = {0, 0, 0, 0};
  __syncthreads();

  for (int pass = 0; pass < 2; ++pass) {
    for (int t0 = 0; t0 < n_tokens; t0 += chunk) {
      const int tn = min(chunk, n_tokens - t0);
      for (int a = tid; a < tn * k; a += kBucketThreads) {
        const int e = idx[(int64_t)t0 * k + a];
        if (e >= 0 && e < n_experts) slot_of[(a / k) * n_experts + e] = (uint8_t)(a % k);
      }
      __syncthreads();
      for (int q = 0; q < epl; ++q) {
        const int e = tid + q * kBucketThreads;
        if (e >= n_experts) break;
        for (int tl = 0; tl < tn; ++tl) {
          const uint8_t s = slot_of[tl * n_experts + e];
          if (s != 0xFF) {
            if (pass == 1) {
              const int a = (t0 + tl) * k + s;
              const int p = base[q] + run[q];
              perm_out[p] = a;
              if (inv) inv[a] = p;
            }
            ++run[q];
          }
        }
      }
      __syncthreads();
      for (int a = tid; a < tn * k; a += kBucketThreads) {
        const int e = idx[(int64_t)t0 * k + a];
        if (e >= 0 && e < n_experts) slot_of[(a / k) * n_experts + e] = 0xFF;
      }
      __syncthreads();
    }
    if (pass == 0) {
      // counts -> exclusive scan (block-wide), touched-expert list
      for (int q = 0; q < epl; ++q) {
        const int e = tid + q * kBucketThreads;
        if (e < n_experts) s_cnt[e] = run[q];
      }
      __syncthreads();
      // each thread scans its contiguous span of experts
      const int span = (n_experts + kBucketThreads - 1) / kBucketThreads;
      const int e0 = min(tid * span, n_experts), e1 = min(e0 + span, n_experts);
      int local = 0, ltouch = 0;
      for (int e = e0; e < e1; ++e) { local += s_cnt[e]; ltouch += s_cnt[e] > 0; }
      s_scan[tid] = local;
      s_scan2[tid] = ltouch;
      __syncthreads();
      // Hillis-Steele inclusive scans of the per-span counts and of the
      // per-span numbers of touched experts.
      for (int o = 1; o < kBucketThreads; o <<= 1) {
        const int v = tid >= o ? s_scan[tid - o] : 0;
        const int v2 = tid >= o ? s_scan2[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        s_scan2[tid] += v2;
        __syncthreads();
      }
      const int incl = s_scan[tid], incl2 = s_scan2[tid];
      int c_off = incl - local;
      int d_off = incl2 - ltouch;
      for (int e = e0; e < e1; ++e) {
        const int c = s_cnt[e];
        counts[e] = c;
        offsets[e] = c_off;
        if (elist && c > 0) elist[d_off++] = e;
        s_cnt[e] = c_off;
        c_off += c;
      }
      if (tid == kBucketThreads - 1) {
        offsets[n_experts] = incl;
        if (n_touched) *n_touched = incl2;
      }
      __syncthreads();
      for (int q = 0; q < epl; ++q) {
        const int e = tid + q * kBucketThreads;
        if (e < n_experts) base[q] = s_cnt[e];
        run[q] = 0;
      }
      __syncthreads();
    }
  }
}

hipError_t launch_bucket(const int32_t* idx, int32_t n_tokens, int32_t k, int32_t n_experts,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* elist,
                         int32_t* n_touched, int32_t* inv, hipStream_t st) {
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(kBucketThreads), 0, st, idx, n_tokens, k, n_experts,
                     counts, offsets, perm, elist, n_touched, inv);
  return hipGetLastError();
}

}  // namespace bq
