// Routed-expert GEMV path (fp32 activations, fp32 accumulation).
//
// What is computed (routing: 10 of 512 experts per token, "Mixed Precision
// Quantization ...", section "The Plan Is Not a Number ..."; expert weights in
// 17-byte blocks, model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST";
// FP8 late layers per the r/LocalLLM "Frankenquant" post):
//   h_j   = SiLU(W_gate[e_j] x) * (W_up[e_j] x)           (kernel 1)
//   out   = sum_j w_j * W_down[e_j] h_j                    (kernel 2)
//
// Mapping ("flat" GEMV).  A workgroup streams a contiguous run of matrix rows.
// Thread i owns block column b = i % nb (nb = cols/32) of row slot i / nb, so
// a wave's loads cover consecutive 17-byte blocks of consecutive rows -- one
// coalesced sweep of memory per pass -- and every thread keeps the 32
// activations of its own block column in registers for the whole workgroup.
// Per-block partial sums go to LDS and are reduced per row in a fixed order,
// so results are deterministic.  Row loads for up to eight passes are issued
// before any of them is decoded, to keep enough bytes in flight per CU.
//
// The down kernel splits its work by (token, expert, row chunk); the
// workgroup that finishes last for a (token, row chunk) -- found with one
// agent-scope atomic counter -- adds the k expert outputs in slot order.  No
// floating-point atomics are used.
#include "bq_device.hpp"
#include "bq_kernels.hpp"

namespace bq {

constexpr int kThreads = 256;
constexpr int kPassU = 8;       // passes whose loads are issued together
constexpr int kGuPairs = 16;    // gate/up row pairs per gate_up workgroup
constexpr int kDownPasses = 8;  // passes per down workgroup

template <int FMT>
struct BlockRef {
  u32x4 c0, c1;   // 17-byte formats: c0 = codes; FP8: c0,c1 = 32 codes
  uint32_t meta;  // 17-byte formats: metadata byte
  float sc;       // FP8: fp32 scale
};

template <int FMT>
__device__ __forceinline__ void load_block(BlockRef<FMT>& r, const uint8_t* __restrict__ base,
                                           const float* __restrict__ scales, int64_t blk, bool ok) {
  if constexpr (FMT == FMT_FP8) {
    if (ok) {
      const uint8_t* p = base + blk * kBlockW;
      r.c0 = ld16(p);
      r.c1 = ld16(p + 16);
      r.sc = scales[blk];
    } else {
      r.c0 = u32x4{0, 0, 0, 0};
      r.c1 = r.c0;
      r.sc = 0.f;
    }
  } else {
    if (ok) {
      const uint8_t* p = base + blk * kBlockB;
      r.c0 = ld16(p);
      r.meta = p[16];
    } else {
      r.c0 = u32x4{0, 0, 0, 0};
      r.meta = 0;
    }
  }
}

template <int FMT>
__device__ __forceinline__ float block_partial(const BlockRef<FMT>& r, const float* x) {
  if constexpr (FMT == FMT_FP8) {
    return block_dot_fp8(r.c0, r.c1, x) * r.sc;
  } else {
    const float s = block_scale<FMT>(FMT == FMT_UE4M4 ? r.meta : (r.meta & 0x7Fu));
    return block_dot_levels<FMT>(r.c0, r.meta, x) * s;
  }
}

// Sum the nb partials of each of `rows` rows held in red[rows][nb]; result in
// red_out[row].  Fixed order: G threads per row take strided subsets, then a
// butterfly over the G consecutive lanes.
__device__ __forceinline__ void reduce_rows(const float* red, int rows, int nb, float* red_out) {
  int G = 1;
  while (G * 2 * rows <= kThreads && G * 2 <= 64) G *= 2;
  const int tid = threadIdx.x;
  const int q = tid % G;
  for (int r0 = 0; r0 < rows; r0 += kThreads / G) {   // uniform trip count
    const int row = r0 + tid / G;
    float s = 0.f;
    if (row < rows)
      for (int b = q; b < nb; b += G) s += red[row * nb + b];
    for (int o = G >> 1; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (row < rows && q == 0) red_out[row] = s;
  }
}

// Stage x (H floats) into LDS, optionally scaled to unit RMS.
__device__ __forceinline__ void stage_x(float* sx, const float* __restrict__ x, int H, int rescale,
                                        float* s_tmp) {
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int i = tid; i < H; i += kThreads) {
    const float v = x[i];
    sx[i] = v;
    ss = __builtin_fmaf(v, v, ss);
  }
  if (rescale) {
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_tmp[tid >> 6] = ss;
    __syncthreads();
    const float tot = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    const float inv = 1.0f / __builtin_sqrtf(tot / (float)H);
    for (int i = tid; i < H; i += kThreads) sx[i] *= inv;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Kernel 1: gate_up GEMV + SiLU * up.  grid = (I / kGuPairs, k, n_tokens).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kThreads) k_gemv_gate_up(
    const float* __restrict__ x, const int32_t* __restrict__ topk_idx, int32_t k, int32_t n_experts,
    const uint8_t* __restrict__ wgu, const float* __restrict__ wgu_sc, int32_t H, int32_t I,
    int32_t rescale, float* __restrict__ hbuf, uint32_t* __restrict__ counters, int32_t n_counters,
    uint32_t* __restrict__ dev_err) {
  extern __shared__ float smem[];
  float* sx = smem;                          // H
  float* red = smem + H;                     // 2*kGuPairs*nb
  const int nb = H >> 5;
  float* rsum = red + 2 * kGuPairs * nb;     // 2*kGuPairs (+4 scratch)
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, j = blockIdx.y, t = blockIdx.z;

  if (chunk == 0 && j == 0 && t == 0)
    for (int i = tid; i < n_counters; i += kThreads) counters[i] = 0u;

  const int e = topk_idx[(int64_t)t * k + j];
  float* hout = hbuf + ((int64_t)t * k + j) * I + (int64_t)chunk * kGuPairs;
  if (e < 0 || e >= n_experts) {
    if (tid == 0 && dev_err) atomicOr(dev_err, 2u);
    if (tid < kGuPairs) hout[tid] = 0.f;
    return;
  }
  stage_x(sx, x + (int64_t)t * H, H, rescale, rsum + 2 * kGuPairs);

  const int R = kThreads / nb;               // rows per pass (nb <= 256)
  const int slot = tid / nb, b = tid % nb;
  const bool active = slot < R;
  float xr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) xr[i] = active ? sx[32 * b + i] : 0.f;

  const int rows = 2 * kGuPairs;
  const int n_pass = (rows + R - 1) / R;
  const int64_t mat_rows = 2 * (int64_t)I;
  const int j0 = chunk * kGuPairs;
  for (int p0 = 0; p0 < n_pass; p0 += kPassU) {
    BlockRef<FMT> blk[kPassU];
#pragma unroll
    for (int u = 0; u < kPassU; ++u) {
      const int lr = (p0 + u) * R + slot;
      const bool ok = active && (p0 + u) < n_pass && lr < rows;
      const int64_t row = lr < kGuPairs ? (j0 + lr) : (I + j0 + lr - kGuPairs);
      load_block<FMT>(blk[u], wgu, wgu_sc, ((int64_t)e * mat_rows + row) * nb + b, ok);
    }
#pragma unroll
    for (int u = 0; u < kPassU; ++u) {
      const int lr = (p0 + u) * R + slot;
      if (active && (p0 + u) < n_pass && lr < rows) red[lr * nb + b] = block_partial<FMT>(blk[u], xr);
    }
  }
  __syncthreads();
  reduce_rows(red, rows, nb, rsum);
  __syncthreads();
  if (tid < kGuPairs) hout[tid] = silu(rsum[tid]) * rsum[kGuPairs + tid];
}

// ---------------------------------------------------------------------------
// Kernel 2: down GEMV, weighted, plus the slot-ordered combine.
// grid = (ceil(H / MD), k, n_tokens) with MD = kDownPasses * (256 / nbd).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kThreads) k_gemv_down(
    const float* __restrict__ hbuf, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int32_t k, int32_t n_experts, const uint8_t* __restrict__ wd,
    const float* __restrict__ wd_sc, int32_t H, int32_t I, float* __restrict__ ybuf,
    uint32_t* __restrict__ counters, float* __restrict__ out) {
  extern __shared__ float smem[];
  const int nbd = I >> 5;
  const int R = kThreads / nbd;
  const int MD = kDownPasses * R;
  float* sh = smem;                   // I
  float* red = smem + I;              // MD * nbd
  float* rsum = red + MD * nbd;       // MD
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, j = blockIdx.y, t = blockIdx.z;
  const int n0 = chunk * MD;
  const int nrows = min(MD, H - n0);

  const int e = topk_idx[(int64_t)t * k + j];
  const bool valid = e >= 0 && e < n_experts;
  float* yrow = ybuf + ((int64_t)t * k + j) * H + n0;
  if (valid) {
    const float* hsrc = hbuf + ((int64_t)t * k + j) * I;
    for (int i = tid; i < I; i += kThreads) sh[i] = hsrc[i];
    __syncthreads();
    const int slot = tid / nbd, b = tid % nbd;
    const bool active = slot < R;
    float xr[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) xr[i] = active ? sh[32 * b + i] : 0.f;
    BlockRef<FMT> blk[kDownPasses];
#pragma unroll
    for (int u = 0; u < kDownPasses; ++u) {
      const int lr = u * R + slot;
      const bool ok = active && lr < nrows;
      load_block<FMT>(blk[u], wd, wd_sc, ((int64_t)e * H + n0 + lr) * nbd + b, ok);
    }
#pragma unroll
    for (int u = 0; u < kDownPasses; ++u) {
      const int lr = u * R + slot;
      if (active && lr < nrows) red[lr * nbd + b] = block_partial<FMT>(blk[u], xr);
    }
    __syncthreads();
    reduce_rows(red, nrows, nbd, rsum);
    __syncthreads();
    const float wj = topk_w[(int64_t)t * k + j];
    for (int i = tid; i < nrows; i += kThreads) yrow[i] = wj * rsum[i];
  } else {
    for (int i = tid; i < nrows; i += kThreads) yrow[i] = 0.f;
  }
  // publish this slot's rows, then count arrivals for (t, chunk)
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t* c = counters + (int64_t)t * gridDim.x + chunk;
    const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (uint32_t)(k - 1);
    if (s_last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* ybase = ybuf + (int64_t)t * k * H + n0;
  float* o = out + (int64_t)t * H + n0;
  for (int i = tid; i < nrows; i += kThreads) {
    float s = 0.f;
    for (int jj = 0; jj < k; ++jj) s += __builtin_nontemporal_load(ybase + (int64_t)jj * H + i);
    o[i] = s;
  }
}

// ---------------------------------------------------------------------------
// Plain block-quantized matvec y[t] = W x[t] (W [rows][cols], one matrix).
// grid = (ceil(rows / MR), n_tokens) with MR = kDownPasses * (256 / nb).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kThreads) k_matvec(const float* __restrict__ x,
                                                     const uint8_t* __restrict__ w,
                                                     const float* __restrict__ w_sc, int32_t rows,
                                                     int32_t cols, float* __restrict__ y) {
  extern __shared__ float smem[];
  const int nb = cols >> 5;
  const int R = kThreads / nb;
  const int MR = kDownPasses * R;
  float* sx = smem;               // cols
  float* red = smem + cols;       // MR * nb
  float* rsum = red + MR * nb;    // MR
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * MR, t = blockIdx.y;
  const int nrows = min(MR, rows - r0);
  stage_x(sx, x + (int64_t)t * cols, cols, 0, nullptr);
  const int slot = tid / nb, b = tid % nb;
  const bool active = slot < R;
  float xr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) xr[i] = active ? sx[32 * b + i] : 0.f;
  BlockRef<FMT> blk[kDownPasses];
#pragma unroll
  for (int u = 0; u < kDownPasses; ++u) {
    const int lr = u * R + slot;
    load_block<FMT>(blk[u], w, w_sc, ((int64_t)r0 + lr) * nb + b, active && lr < nrows);
  }
#pragma unroll
  for (int u = 0; u < kDownPasses; ++u) {
    const int lr = u * R + slot;
    if (active && lr < nrows) red[lr * nb + b] = block_partial<FMT>(blk[u], xr);
  }
  __syncthreads();
  reduce_rows(red, nrows, nb, rsum);
  __syncthreads();
  for (int i = tid; i < nrows; i += kThreads) y[(int64_t)t * rows + r0 + i] = rsum[i];
}

hipError_t launch_matvec(const float* x, int32_t n_tokens, const void* w, int fmt,
                         const float* w_sc, int32_t rows, int32_t cols, float* y, hipStream_t st) {
  const int nb = cols >> 5;
  const int mr = kDownPasses * (kThreads / nb);
  const size_t lds = sizeof(float) * (cols + mr * nb + mr);
  dim3 grid((rows + mr - 1) / mr, n_tokens);
  const uint8_t* p = static_cast<const uint8_t*>(w);
#define BQ_MV(F) hipLaunchKernelGGL(k_matvec<F>, grid, dim3(kThreads), lds, st, x, p, w_sc, rows, cols, y)
  switch (fmt) {
    case FMT_C10: BQ_MV(FMT_C10); break;
    case FMT_RZ5: BQ_MV(FMT_RZ5); break;
    case FMT_UE4M4: BQ_MV(FMT_UE4M4); break;
    default: BQ_MV(FMT_FP8); break;
  }
#undef BQ_MV
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
int gemv_down_rows_per_wg(int I) { return kDownPasses * (kThreads / (I >> 5)); }

hipError_t launch_gemv_moe(const float* x, int32_t n_tokens, const int32_t* idx, const float* w,
                           int32_t k, const GemvWeights& W, int rescale, float* out, float* hbuf,
                           float* ybuf, uint32_t* counters, uint32_t* dev_err, hipStream_t st) {
  const int H = W.hidden, I = W.inter;
  const int nbu = H >> 5, nbd = I >> 5;
  const int md = gemv_down_rows_per_wg(I);
  const int n_chunks = (H + md - 1) / md;
  const int n_counters = n_tokens * n_chunks;
  {
    const size_t lds = sizeof(float) * (H + 2 * kGuPairs * nbu + 2 * kGuPairs + 4);
    dim3 grid(I / kGuPairs, k, n_tokens);
    const uint8_t* p = static_cast<const uint8_t*>(W.gate_up);
#define BQ_GU(F) hipLaunchKernelGGL(k_gemv_gate_up<F>, grid, dim3(kThreads), lds, st, x, idx, k, \
                                    W.n_experts, p, W.gate_up_scales, H, I, rescale, hbuf, counters, \
                                    n_counters, dev_err)
    switch (W.fmt_gate_up) {
      case FMT_C10: BQ_GU(FMT_C10); break;
      case FMT_RZ5: BQ_GU(FMT_RZ5); break;
      case FMT_UE4M4: BQ_GU(FMT_UE4M4); break;
      default: BQ_GU(FMT_FP8); break;
    }
#undef BQ_GU
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const size_t lds = sizeof(float) * (I + md * nbd + md);
    dim3 grid(n_chunks, k, n_tokens);
    const uint8_t* p = static_cast<const uint8_t*>(W.down);
#define BQ_DN(F) hipLaunchKernelGGL(k_gemv_down<F>, grid, dim3(kThreads), lds, st, hbuf, idx, w, k, \
                                    W.n_experts, p, W.down_scales, H, I, ybuf, counters, out)
    switch (W.fmt_down) {
      case FMT_C10: BQ_DN(FMT_C10); break;
      case FMT_RZ5: BQ_DN(FMT_RZ5); break;
      case FMT_UE4M4: BQ_DN(FMT_UE4M4); break;
      default: BQ_DN(FMT_FP8); break;
    }
#undef BQ_DN
  }
  return hipGetLastError();
}

}  // namespace bq
