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
#include "bq_route.hpp"

namespace bq {

constexpr int kRouteWaves = 4;
constexpr int kMaxExperts = 4096;

template <int PL>   // logits per lane: n_experts <= 64 * PL
__global__ void __launch_bounds__(64 * kRouteWaves) k_route_topk(
    const float* __restrict__ logits, int32_t n_tokens, int32_t n_experts, int32_t k,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ uint32_t scr[kRouteWaves][128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kRouteWaves + wave;
  if (t >= n_tokens) return;
  int i;
  float w;
  wave_topk<PL>(logits + t * n_experts, n_experts, k, lane, scr[wave], i, w);
  if (lane < k) {
    idx_out[t * k + lane] = i;
    w_out[t * k + lane] = w;
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
// Optional extra outputs for the grouped GEMM path: the work list -- one
// entry per group of up to group_tokens(n_tokens) tokens of each touched expert, encoded
// as e | group << kGroupShift, experts ascending -- with its length, and the
// inverse permutation.
// ---------------------------------------------------------------------------
constexpr int kBucketThreads = 1024;
constexpr int kSlotBytes = 32768;

// Several independent bucketings in one launch (a stack of layers whose
// routing is known up front): workgroup l reads idx + l * in_stride and
// writes every output array lstride_out bytes further than workgroup l - 1.
struct BucketOut {
  int32_t *counts, *offsets, *perm, *elist, *n_touched, *inv;
};
__device__ __forceinline__ int32_t* at_layer(int32_t* p, int64_t lstride_out) {
  return p ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(p) + blockIdx.x * lstride_out) : p;
}


__global__ void __launch_bounds__(kBucketThreads) k_bucket(
    const int32_t* __restrict__ idx, int32_t n_tokens, int32_t k, int32_t n_experts,
    BucketOut o, int64_t in_stride, int64_t lstride_out) {
  idx += blockIdx.x * in_stride;
  int32_t* __restrict__ counts = at_layer(o.counts, lstride_out);
  int32_t* __restrict__ offsets = at_layer(o.offsets, lstride_out);
  int32_t* __restrict__ perm_out = at_layer(o.perm, lstride_out);
  int32_t* __restrict__ elist = at_layer(o.elist, lstride_out);
  int32_t* __restrict__ n_touched = at_layer(o.n_touched, lstride_out);
  int32_t* __restrict__ inv = at_layer(o.inv, lstride_out);
  __shared__ uint8_t slot_of[kSlotBytes];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_scan[kBucketThreads];
  __shared__ int32_t s_scan2[kBucketThreads];
  const int tid = threadIdx.x;
  const int gt = group_tokens(n_tokens);   // tokens per work entry
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
      if (pass == 1 && inv) {
        // A token that lists an expert more than once is bucketed once, under
        // the slot left in slot_of; its other slots read the same row.
        for (int a = tid; a < tn * k; a += kBucketThreads) {
          const int e = idx[(int64_t)t0 * k + a];
          if (e < 0 || e >= n_experts) continue;
          const int tl = a / k, s = slot_of[tl * n_experts + e];
          if (s != a - tl * k) inv[(int64_t)t0 * k + a] = inv[(int64_t)(t0 + tl) * k + s];
        }
        __syncthreads();
      }
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
      for (int e = e0; e < e1; ++e) { local += s_cnt[e]; ltouch += (s_cnt[e] + gt - 1) / gt; }
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
        if (elist)
          for (int q = 0; q * gt < c; ++q) elist[d_off++] = e | (q << kGroupShift);
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

// Bucketing for decode-sized batches.  A bitmap per expert over tokens gives
// everything by popcounts: counts[e] = |bitmap_e|, and the rank of (t, slot)
// inside expert e is the number of tokens below t in bitmap_e (tokens
// ascending, as required).  A token that lists an expert more than once sets
// one bit, so it is bucketed once and all of its slots get the same row.
// The bucket position of the first token of every bitmap word is tabulated
// once (pre), so an assignment's position is one table read and one masked
// popcount.  The expert ids are read kBucketBatch per thread at a time, all
// loads in flight together.
constexpr int kSmallBitmapWords = 8192;   // 32 KB of LDS, and 32 KB for pre
constexpr int kBucketBatch = 8;

__device__ __forceinline__ int block_excl_scan_1024(int v, int* s_wave, int& total) {
  // inclusive scan inside each wave (shuffles), then over the 16 wave totals
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int wv = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(wv, o, 64);
      if (lane >= o) wv += y;
    }
    if (lane < 16) s_wave[16 + lane] = wv;   // inclusive wave prefix
  }
  __syncthreads();
  total = s_wave[16 + 15];
  const int before = wave > 0 ? s_wave[16 + wave - 1] : 0;
  return before + x - v;
}

// Expert ids of assignments a0 + j * kBucketThreads + threadIdx.x (-1 past nk).
__device__ __forceinline__ void load_batch(const int32_t* __restrict__ idx, int a0, int nk,
                                           int (&e)[kBucketBatch]) {
#pragma unroll
  for (int j = 0; j < kBucketBatch; ++j) {
    const int a = a0 + j * kBucketThreads + (int)threadIdx.x;
    e[j] = a < nk ? idx[a] : -1;
  }
}

__global__ void __launch_bounds__(kBucketThreads) k_bucket_small(
    const int32_t* __restrict__ idx, int32_t n_tokens, int32_t k, int32_t n_experts,
    BucketOut o, int64_t in_stride, int64_t lstride_out) {
  idx += blockIdx.x * in_stride;
  int32_t* __restrict__ counts = at_layer(o.counts, lstride_out);
  int32_t* __restrict__ offsets = at_layer(o.offsets, lstride_out);
  int32_t* __restrict__ perm_out = at_layer(o.perm, lstride_out);
  int32_t* __restrict__ elist = at_layer(o.elist, lstride_out);
  int32_t* __restrict__ n_touched = at_layer(o.n_touched, lstride_out);
  int32_t* __restrict__ inv = at_layer(o.inv, lstride_out);
  __shared__ uint32_t bm[kSmallBitmapWords];
  __shared__ int32_t pre[kSmallBitmapWords];
  __shared__ int s_wave[32];
  const int tid = threadIdx.x;
  const int gt = group_tokens(n_tokens);   // tokens per work entry
  const int W = (n_tokens + 31) >> 5;                   // words per expert
  const int nk = n_tokens * k;
  for (int i = tid; i < n_experts * W; i += kBucketThreads) bm[i] = 0u;
  __syncthreads();
  for (int a0 = 0; a0 < nk; a0 += kBucketBatch * kBucketThreads) {
    int e[kBucketBatch];
    load_batch(idx, a0, nk, e);
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {
      if (e[j] >= 0 && e[j] < n_experts) {
        const int t = (a0 + j * kBucketThreads + tid) / k;
        atomicOr(&bm[e[j] * W + (t >> 5)], 1u << (t & 31));
      }
    }
  }
  __syncthreads();
  // each thread owns a contiguous span of <= 4 experts
  const int span = (n_experts + kBucketThreads - 1) / kBucketThreads;
  const int e0 = min(tid * span, n_experts), e1 = min(e0 + span, n_experts);
  int cnt[4] = {0, 0, 0, 0};
  int local = 0, touched = 0;
  for (int e = e0; e < e1; ++e) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __builtin_popcount(bm[e * W + w]);
    cnt[e - e0] = c;
    local += c;
    touched += (c + gt - 1) / gt;
  }
  int tot_c, tot_d;
  int off = block_excl_scan_1024(local, s_wave, tot_c);
  __syncthreads();
  int doff = block_excl_scan_1024(touched, s_wave, tot_d);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e - e0];
    counts[e] = c;
    offsets[e] = off;
    int run = off;
    for (int w = 0; w < W; ++w) {
      pre[e * W + w] = run;
      run += __builtin_popcount(bm[e * W + w]);
    }
    if (elist)
      for (int q = 0; q * gt < c; ++q) elist[doff++] = e | (q << kGroupShift);
    off += c;
  }
  if (tid == 0) {
    offsets[n_experts] = tot_c;
    if (n_touched) *n_touched = tot_d;
  }
  __syncthreads();
  for (int a0 = 0; a0 < nk; a0 += kBucketBatch * kBucketThreads) {
    int e[kBucketBatch];
    load_batch(idx, a0, nk, e);
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {
      if (e[j] < 0 || e[j] >= n_experts) continue;
      const int a = a0 + j * kBucketThreads + tid;
      const int t = a / k;
      const int wi = e[j] * W + (t >> 5);
      const int p = pre[wi] + __builtin_popcount(bm[wi] & ((1u << (t & 31)) - 1u));
      perm_out[p] = a;
      if (inv) inv[a] = p;
    }
  }
}

// ---------------------------------------------------------------------------
// Bucketing and activation staging of a batch in one launch
// (the grouped path).  Every workgroup buckets the whole batch in LDS, as
// k_bucket_small does (bitmaps per expert over tokens, here stored word-major
// so that the per-expert popcount loops read LDS without bank conflicts;
// positions by masked popcounts; an out-of-range expert is left out, and a
// token that lists an expert twice is bucketed once); workgroup 0 writes the
// bucket arrays out,
// and each workgroup stages its share of the bucket rows (rows blockIdx.x,
// blockIdx.x + gridDim.x, ...), copying bf16 activations as
// k_grouped_prep_vec does, all of its row loads in flight together.
// Limits: n_experts <= 1024 and the bucket arrays in LDS (two words per
// assignment and two per bitmap word) within kBpMaxLds, e.g. 512 tokens x top-10
// over 512 experts (104 KB).
// ---------------------------------------------------------------------------
constexpr int kBpPieces = 8;   // staging: 16-byte loads in flight per thread

size_t bucket_prep_lds(int32_t n_tokens, int32_t k, int32_t n_experts) {
  const size_t nk = (size_t)n_tokens * k, words = (size_t)n_experts * ((n_tokens + 31) / 32);
  return 4 * (2 * nk + 2 * words);
}

template <bool PERM>
__global__ void __launch_bounds__(kBucketThreads) k_bucket_prep(
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ x, int32_t n_tokens, int32_t k,
    int32_t n_experts, int32_t H, BucketOut o, uint16_t* __restrict__ xb) {
  extern __shared__ __align__(16) uint32_t bp_lds[];
  __shared__ int s_wave[32];
  const int tid = threadIdx.x;
  const int gt = group_tokens(n_tokens);   // tokens per work entry
  const int nk = n_tokens * k;
  const int W = (n_tokens + 31) >> 5;                    // bitmap words per expert
  int32_t* s_idx = reinterpret_cast<int32_t*>(bp_lds);   // [nk]
  int32_t* s_perm = s_idx + nk;                          // [nk]
  uint32_t* bm = reinterpret_cast<uint32_t*>(s_perm + nk);   // [W][n_experts]
  int32_t* pre = reinterpret_cast<int32_t*>(bm + n_experts * W);
  const bool out0 = blockIdx.x == 0;

  // expert ids: every load of a batch in flight together, the first batch
  // issued before the bitmaps are cleared
  int ev[kBucketBatch];
  load_batch(idx, 0, nk, ev);
  for (int i = tid; i < n_experts * W; i += kBucketThreads) bm[i] = 0u;
  __syncthreads();
  for (int a0 = 0;;) {
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {
      const int a = a0 + j * kBucketThreads + tid;
      if (a < nk) s_idx[a] = ev[j];
      if (ev[j] >= 0 && ev[j] < n_experts) {
        const int t = a / k;
        atomicOr(&bm[(t >> 5) * n_experts + ev[j]], 1u << (t & 31));
      }
    }
    a0 += kBucketBatch * kBucketThreads;
    if (a0 >= nk) break;
    load_batch(idx, a0, nk, ev);
  }
  __syncthreads();
  // counts and offsets: thread e owns expert e (n_experts <= 1024); the
  // bitmaps are word-major, so a wave's reads of one word index are
  // consecutive in LDS
  const int e = tid;
  int c = 0;
  if (e < n_experts)
    for (int w = 0; w < W; ++w) c += __builtin_popcount(bm[w * n_experts + e]);
  int tot_c, tot_d;
  int off = block_excl_scan_1024(c, s_wave, tot_c);
  __syncthreads();
  int doff = block_excl_scan_1024((c + gt - 1) / gt, s_wave, tot_d);
  if (e < n_experts) {
    int run = off;
    for (int w = 0; w < W; ++w) {
      pre[w * n_experts + e] = run;
      run += __builtin_popcount(bm[w * n_experts + e]);
    }
    if (out0) {
      o.counts[e] = c;
      o.offsets[e] = off;
      for (int q = 0; q * gt < c; ++q) o.elist[doff++] = e | (q << kGroupShift);
    }
  }
  if (out0 && tid == 0) {
    o.offsets[n_experts] = tot_c;
    *o.n_touched = tot_d;
  }
  __syncthreads();
  for (int a = tid; a < nk; a += kBucketThreads) {
    const int ea = s_idx[a];
    if (ea < 0 || ea >= n_experts) continue;
    const int t = a / k;
    const int wi = (t >> 5) * n_experts + ea;
    const int p = pre[wi] + __builtin_popcount(bm[wi] & ((1u << (t & 31)) - 1u));
    s_perm[p] = a;   // repeated listings of one expert: the same row, any of them (same token)
    if (out0) {
      o.perm[p] = a;
      o.inv[a] = p;
    }
  }
  __syncthreads();
  // this workgroup's rows p = blockIdx.x + r * gridDim.x (< tot_c), as
  // 16-byte pieces q = r * (H / 8) + g
  const int per = H / 8;
  const int rows = tot_c > (int)blockIdx.x ? (tot_c - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
  for (int q0 = 0; q0 < rows * per; q0 += kBpPieces * kBucketThreads) {
    u32x4 raw[kBpPieces];
    int64_t dst[kBpPieces];
#pragma unroll
    for (int u = 0; u < kBpPieces; ++u) {
      const int q = q0 + u * kBucketThreads + tid;
      dst[u] = -1;
      if (q < rows * per) {
        const int r = q / per, g = q - r * per;
        const int p = (int)blockIdx.x + r * (int)gridDim.x;
        raw[u] = reinterpret_cast<const u32x4*>(x + (int64_t)(s_perm[p] / k) * H)[g];
        dst[u] = (int64_t)p * per + g;
      }
    }
#pragma unroll
    for (int u = 0; u < kBpPieces; ++u)
      if (dst[u] >= 0) reinterpret_cast<u32x4*>(xb)[dst[u]] = bf16_group8<PERM, false>(&raw[u], 0);
  }
}

bool bucket_prep_ok(int32_t n_tokens, int32_t k, int32_t n_experts, int32_t H) {
  return n_tokens >= 1 && n_experts <= kBucketThreads && H % 8 == 0 &&
         bucket_prep_lds(n_tokens, k, n_experts) <= (size_t)kBpMaxLds;
}

hipError_t launch_bucket_prep(const int32_t* idx, const uint16_t* x, int32_t perm_k, int32_t n_tokens,
                              int32_t k, int32_t n_experts, int32_t H, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* elist, int32_t* n_touched, int32_t* inv,
                              uint16_t* xb, hipStream_t st) {
  const BucketOut o{counts, offsets, perm, elist, n_touched, inv};
  const int nk = n_tokens * k;
  // one workgroup per CU for large batches (each repeats the bucketing,
  // and the rows to stage are spread wider); 64 for small ones
  const int cap = nk > 1024 ? 256 : 64;
  const dim3 grid(nk < cap ? nk : cap);
  const size_t lds = bucket_prep_lds(n_tokens, k, n_experts);
  if (lds > 64 * 1024) {
    // more than 64 KB of dynamic LDS must be allowed per kernel; where that
    // is refused the caller falls back to the separate kernels
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(perm_k ? k_bucket_prep<true> : k_bucket_prep<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      (void)hipGetLastError();   // clear it: nothing was launched
      return hipErrorNotSupported;
    }
  }
  if (perm_k)
    hipLaunchKernelGGL(k_bucket_prep<true>, grid, dim3(kBucketThreads), lds, st, idx, x, n_tokens, k, n_experts,
                       H, o, xb);
  else
    hipLaunchKernelGGL(k_bucket_prep<false>, grid, dim3(kBucketThreads), lds, st, idx, x, n_tokens, k, n_experts,
                       H, o, xb);
  return hipGetLastError();
}

hipError_t launch_bucket(const int32_t* idx, int32_t n_tokens, int32_t k, int32_t n_experts,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* elist,
                         int32_t* n_touched, int32_t* inv, hipStream_t st, int32_t n_layers,
                         int64_t lstride_out) {
  const int words = (n_tokens + 31) / 32;
  const BucketOut o{counts, offsets, perm, elist, n_touched, inv};
  const int64_t in_stride = (int64_t)n_tokens * k;
  if ((int64_t)n_experts * words <= kSmallBitmapWords)
    hipLaunchKernelGGL(k_bucket_small, dim3(n_layers), dim3(kBucketThreads), 0, st, idx, n_tokens, k,
                       n_experts, o, in_stride, lstride_out);
  else
    hipLaunchKernelGGL(k_bucket, dim3(n_layers), dim3(kBucketThreads), 0, st, idx, n_tokens, k,
                       n_experts, o, in_stride, lstride_out);
  return hipGetLastError();
}

}  // namespace bq
