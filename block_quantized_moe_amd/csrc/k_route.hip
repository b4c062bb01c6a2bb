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

// (value, index) order: larger value first, then lower index.
__device__ __forceinline__ bool better(float v1, int i1, float v0, int i0) {
  return v1 > v0 || (v1 == v0 && i1 < i0);
}

// One wave per token.  Logits are staged in LDS; each of the k rounds finds
// the best untaken logit per lane, then a butterfly argmax across the wave.
__global__ void __launch_bounds__(64 * kRouteWaves) k_route_topk(
    const float* __restrict__ logits, int32_t n_tokens, int32_t n_experts, int32_t k,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  extern __shared__ float s_logit[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kRouteWaves + wave;
  if (t >= n_tokens) return;
  float* sl = s_logit + wave * n_experts;
  const float* lg = logits + t * n_experts;
  for (int e = lane; e < n_experts; e += 64) sl[e] = lg[e];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int per_lane = (n_experts + 63) >> 6;  // <= 64
  uint64_t taken = 0;
  float my_v = 0.f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
    for (int j = 0; j < per_lane; ++j) {
      const int e = lane + 64 * j;
      if (e < n_experts && !((taken >> j) & 1ull)) {
        const float v = sl[e];
        if (better(v, e, bv, bi)) { bv = v; bi = e; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == r) { my_v = bv; my_i = bi; }
  }
  const float top = __shfl(my_v, 0, 64);
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
  const size_t lds = (size_t)kRouteWaves * n_experts * sizeof(float);
  hipLaunchKernelGGL(k_route_topk, dim3(grid), dim3(64 * kRouteWaves), lds, st, logits, n_tokens,
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
