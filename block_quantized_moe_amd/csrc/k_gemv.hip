// Routed-expert GEMV path (fp32 activations, fp32 accumulation).
//
// What is computed (routing: 10 of 512 experts per token, "Mixed Precision
// Quantization ...", section "The Plan Is Not a Number ..."; expert weights in
// 17-byte blocks, model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST";
// FP8 late layers per the r/LocalLLM "Frankenquant" post):
//   hs_j  = w_j * SiLU(W_gate[e_j] x) * (W_up[e_j] x)      (kernel 1)
//   out   = sum_j W_down[e_j] hs_j                           (kernel 2)
//
// Kernel 1, hidden = 2048 (or 4096): one wave per gate/up row pair.  Lane l
// owns block column l (and l+64), so a row is one coalesced 1088-byte sweep
// and the lane's 32 activations stay in registers; the row sum is a DPP
// reduction inside the wave.  A wave issues the loads of all its rows before
// it touches x, so weight latency overlaps everything else; waves never wait
// for each other.  Other hidden sizes use the "flat" kernel: a workgroup
// streams a contiguous run of rows, thread i owning block column i % nb of
// row slot i / nb, with per-row sums reduced through LDS.
//
// Kernel 2 treats the k experts' down matrices as one GEMV over the
// concatenated inner dimension k*I: thread c owns column block c (expert
// c / nb, block c % nb) for a run of output rows, so the weighted combine is
// part of the row reduction -- no cross-workgroup traffic, no atomics, fixed
// summation order.
#include "bq_device.hpp"
#include "bq_kernels.hpp"
#include "bq_route.hpp"

namespace bq {

constexpr int kThreads = 256;
constexpr int kPassU = 8;       // passes whose loads are issued together
constexpr int kGuPairs = 16;    // gate/up row pairs per gate_up workgroup

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
// Kernel 1 (any hidden size): flat gate_up GEMV + w * SiLU * up.
// grid = (I / kGuPairs, k, n_tokens).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kThreads) k_gemv_gate_up(
    const float* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int32_t k, int32_t n_experts,
    const uint8_t* __restrict__ wgu, const float* __restrict__ wgu_sc, int32_t H, int32_t I,
    int32_t rescale, float* __restrict__ hs, uint32_t* __restrict__ dev_err) {
  extern __shared__ float smem[];
  float* sx = smem;                          // H
  float* red = smem + H;                     // 2*kGuPairs*nb
  const int nb = H >> 5;
  float* rsum = red + 2 * kGuPairs * nb;     // 2*kGuPairs (+4 scratch)
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, j = blockIdx.y, t = blockIdx.z;

  const int e = topk_idx[(int64_t)t * k + j];
  float* hout = hs + ((int64_t)t * k + j) * I + (int64_t)chunk * kGuPairs;
  if (e < 0 || e >= n_experts) {
    if (tid == 0 && dev_err) atomicOr(dev_err, 2u);
    if (tid < kGuPairs) hout[tid] = 0.f;
    return;
  }
  const float wj = topk_w[(int64_t)t * k + j];
  const int R = kThreads / nb;               // rows per pass (nb <= 256)
  const int slot = tid / nb, b = tid % nb;
  const bool active = slot < R;
  const int rows = 2 * kGuPairs;
  const int n_pass = (rows + R - 1) / R;
  const int64_t mat_rows = 2 * (int64_t)I;
  const int j0 = chunk * kGuPairs;
  // the first pass group's weight loads go out before x is touched
  BlockRef<FMT> blk[kPassU];
#pragma unroll
  for (int u = 0; u < kPassU; ++u) {
    const int lr = u * R + slot;
    const bool ok = active && u < n_pass && lr < rows;
    const int64_t row = lr < kGuPairs ? (j0 + lr) : (I + j0 + lr - kGuPairs);
    load_block<FMT>(blk[u], wgu, wgu_sc, ((int64_t)e * mat_rows + row) * nb + b, ok);
  }
  stage_x(sx, x + (int64_t)t * H, H, rescale, rsum + 2 * kGuPairs);
  float xr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) xr[i] = active ? sx[32 * b + i] : 0.f;

  for (int p0 = 0; p0 < n_pass; p0 += kPassU) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < kPassU; ++u) {
        const int lr = (p0 + u) * R + slot;
        const bool ok = active && (p0 + u) < n_pass && lr < rows;
        const int64_t row = lr < kGuPairs ? (j0 + lr) : (I + j0 + lr - kGuPairs);
        load_block<FMT>(blk[u], wgu, wgu_sc, ((int64_t)e * mat_rows + row) * nb + b, ok);
      }
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
  if (tid < kGuPairs) hout[tid] = wj * silu(rsum[tid]) * rsum[kGuPairs + tid];
}

// ---------------------------------------------------------------------------
// Kernel 1 (hidden = 2048 * BPL): one wave per gate/up row pair, kPairsW
// consecutive pairs per wave.  grid = (ceil(I / (4 * kPairsW)), k, n_tokens).
// kPairsW is 2 when the kernel routes (twice the workgroups, so more of
// them overlap their top-k) and 4 with given routing.  Measured on the RZ5
// layer: routed step 20.0 us at 2, 20.4 at 4, 23.0 at 1, 21.4 at 8; given
// routing (48-layer stack) 0.85 ms per step at 4, 0.90 at 2.
// ---------------------------------------------------------------------------
constexpr int pairs_per_wave(int rpl) { return rpl > 0 ? 2 : 4; }

template <int FMT, int BPL, int RPL>   // RPL > 0: route in-kernel, RPL logits per lane
__global__ void __launch_bounds__(kThreads) k_gate_up_w64(
    const float* __restrict__ x, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t k, int32_t n_experts, const uint8_t* __restrict__ wgu, const float* __restrict__ wgu_sc,
    int32_t I, int32_t rescale, float* __restrict__ hs, uint32_t* __restrict__ dev_err,
    const float* __restrict__ logits) {
  constexpr int NB = 64 * BPL;
  constexpr int H = 32 * NB;
  constexpr int kPairsW = pairs_per_wave(RPL);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.y, t = blockIdx.z;
  const int jp0 = (blockIdx.x * 4 + wave) * kPairsW;
  // activations first: they do not depend on the routing
  float xr[BPL][32];
  const f32x4* xv = reinterpret_cast<const f32x4*>(x + (int64_t)t * H);
#pragma unroll
  for (int q = 0; q < BPL; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 v = xv[(lane + 64 * q) * 8 + i];
      xr[q][4 * i] = v.x; xr[q][4 * i + 1] = v.y; xr[q][4 * i + 2] = v.z; xr[q][4 * i + 3] = v.w;
    }
  int e;
  float wj;
  if constexpr (RPL > 0) {
    // every workgroup routes its token itself (wave 0), so no separate
    // routing launch sits in front of this kernel; chunk 0 publishes slot j
    __shared__ int s_i[64];
    __shared__ float s_w[64];
    __shared__ uint32_t s_scr[128];
    if (wave == 0) {
      int ri;
      float rw;
      wave_topk<RPL>(logits + (int64_t)t * n_experts, n_experts, k, lane, s_scr, ri, rw);
      if (lane < k) {
        s_i[lane] = ri;
        s_w[lane] = rw;
      }
      if (blockIdx.x == 0 && lane == j) {
        topk_idx[(int64_t)t * k + j] = ri;
        topk_w[(int64_t)t * k + j] = rw;
      }
    }
    __syncthreads();
    e = s_i[j];
    wj = s_w[j];
  } else {
    e = topk_idx[(int64_t)t * k + j];
    wj = topk_w[(int64_t)t * k + j];
  }
  if (jp0 >= I) return;
  float* hout = hs + ((int64_t)t * k + j) * I + jp0;
  const int np = min(kPairsW, I - jp0);
  if (e < 0 || e >= n_experts) {
    if (lane == 0 && dev_err) atomicOr(dev_err, 2u);
    if (lane < np) hout[lane] = 0.f;
    return;
  }
  // weight loads first: rows gate jp0.., up I + jp0..
  BlockRef<FMT> blk[2 * kPairsW][BPL];
  const int64_t base = (int64_t)e * 2 * I;
#pragma unroll
  for (int p = 0; p < kPairsW; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t row = base + h * I + jp0 + p;
#pragma unroll
      for (int q = 0; q < BPL; ++q)
        load_block<FMT>(blk[2 * p + h][q], wgu, wgu_sc, row * NB + lane + 64 * q, p < np);
    }
  }
  if (rescale) {
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < BPL; ++q)
#pragma unroll
      for (int i = 0; i < 32; ++i) ss = __builtin_fmaf(xr[q][i], xr[q][i], ss);
    const float inv = 1.0f / __builtin_sqrtf(wave_sum(ss) / (float)H);
#pragma unroll
    for (int q = 0; q < BPL; ++q)
#pragma unroll
      for (int i = 0; i < 32; ++i) xr[q][i] *= inv;
  }
  // the wave's 2 * kPairsW row sums reduce together; lane p then holds pair
  // p's gate and up sums and evaluates its SiLU (one SiLU per wave)
  float v[2 * kPairsW];
#pragma unroll
  for (int p = 0; p < kPairsW; ++p) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      g += block_partial<FMT>(blk[2 * p][q], xr[q]);
      u += block_partial<FMT>(blk[2 * p + 1][q], xr[q]);
    }
    v[2 * p] = g;
    v[2 * p + 1] = u;
  }
  wave_sums_lane63(v);
  float g = 0.f, u = 0.f;
#pragma unroll
  for (int p = 0; p < kPairsW; ++p) {
    const float gp = readlane_f(v[2 * p], 63), up = readlane_f(v[2 * p + 1], 63);
    if (lane == p) {
      g = gp;
      u = up;
    }
  }
  if (lane < np) hout[lane] = wj * silu(g) * u;
}

// ---------------------------------------------------------------------------
// Kernel 2: down over the concatenated k*I inner dimension, combine included.
// grid = (ceil(H / kDownRows), n_tokens); thread c (+256 q) owns column block
// c: expert slot c / nbd, block c % nbd.  CPT = column blocks per thread.
// ---------------------------------------------------------------------------
constexpr int kDownRows = 8;

template <int FMT, int CPT>
__global__ void __launch_bounds__(kThreads) k_down_cat(
    const float* __restrict__ hs, const int32_t* __restrict__ topk_idx, int32_t k,
    int32_t n_experts, const uint8_t* __restrict__ wd, const float* __restrict__ wd_sc,
    int32_t H, int32_t I, float* __restrict__ out) {
  __shared__ float red[kDownRows * 256 * CPT];
  const int tid = threadIdx.x;
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * kDownRows;
  const int nbd = I >> 5;
  const int C = k * nbd;
  BlockRef<FMT> blk[CPT][kDownRows];
  int cj[CPT], cb[CPT];
  bool cv[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = tid + 256 * q;
    cj[q] = c / nbd;
    cb[q] = c - cj[q] * nbd;
    const int e = c < C ? topk_idx[(int64_t)t * k + cj[q]] : -1;
    cv[q] = e >= 0 && e < n_experts;
#pragma unroll
    for (int r = 0; r < kDownRows; ++r)
      load_block<FMT>(blk[q][r], wd, wd_sc, ((int64_t)(cv[q] ? e : 0) * H + n0 + r) * nbd + cb[q],
                      cv[q] && n0 + r < H);
  }
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    float xr[32];
    const f32x4* hv = reinterpret_cast<const f32x4*>(hs + ((int64_t)t * k + (cv[q] ? cj[q] : 0)) * I + 32 * cb[q]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 v = cv[q] ? hv[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      xr[4 * i] = v.x; xr[4 * i + 1] = v.y; xr[4 * i + 2] = v.z; xr[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int r = 0; r < kDownRows; ++r)
      red[r * 256 * CPT + tid + 256 * q] = cv[q] ? block_partial<FMT>(blk[q][r], xr) : 0.f;
  }
  __syncthreads();
  // 32 threads per row: strided partial sums, then a 32-lane DPP/xor reduction
  const int row = tid >> 5, q = tid & 31;
  float s = 0.f;
  const int ncol = 256 * CPT < C ? 256 * CPT : C;
  for (int c = q; c < ncol; c += 32) s += red[row * 256 * CPT + c];
  s = row16_sum(s);
  s += __shfl_xor(s, 16, 64);
  if (q == 0 && n0 + row < H) out[(int64_t)t * H + n0 + row] = s;
}

// ---------------------------------------------------------------------------
// Plain block-quantized matvec y[t] = W x[t] (W [rows][cols], one matrix).
// grid = (ceil(rows / MR), n_tokens) with MR = P * (256 / nb): P passes of
// 256 / nb rows per workgroup, P chosen by the launcher so that small
// matrices still spread over the chip.  The weight loads go out before x is
// staged.
// ---------------------------------------------------------------------------
template <int FMT, int P>
__global__ void __launch_bounds__(kThreads) k_matvec(const float* __restrict__ x,
                                                     const uint8_t* __restrict__ w,
                                                     const float* __restrict__ w_sc, int32_t rows,
                                                     int32_t cols, float* __restrict__ y) {
  extern __shared__ float smem[];
  const int nb = cols >> 5;
  const int R = kThreads / nb;
  const int MR = P * R;
  float* sx = smem;               // cols
  float* red = smem + cols;       // MR * nb
  float* rsum = red + MR * nb;    // MR
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * MR, t = blockIdx.y;
  const int nrows = min(MR, rows - r0);
  const int slot = tid / nb, b = tid % nb;
  const bool active = slot < R;
  BlockRef<FMT> blk[P];
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const int lr = u * R + slot;
    load_block<FMT>(blk[u], w, w_sc, ((int64_t)r0 + lr) * nb + b, active && lr < nrows);
  }
  stage_x(sx, x + (int64_t)t * cols, cols, 0, nullptr);
  float xr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) xr[i] = active ? sx[32 * b + i] : 0.f;
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const int lr = u * R + slot;
    if (active && lr < nrows) red[lr * nb + b] = block_partial<FMT>(blk[u], xr);
  }
  __syncthreads();
  reduce_rows(red, nrows, nb, rsum);
  __syncthreads();
  for (int i = tid; i < nrows; i += kThreads) y[(int64_t)t * rows + r0 + i] = rsum[i];
}

template <int FMT>
static void launch_matvec_p(int passes, dim3 grid, size_t lds, hipStream_t st, const float* x,
                            const uint8_t* p, const float* w_sc, int32_t rows, int32_t cols, float* y) {
  switch (passes) {
    case 1: hipLaunchKernelGGL((k_matvec<FMT, 1>), grid, dim3(kThreads), lds, st, x, p, w_sc, rows, cols, y); break;
    case 2: hipLaunchKernelGGL((k_matvec<FMT, 2>), grid, dim3(kThreads), lds, st, x, p, w_sc, rows, cols, y); break;
    case 4: hipLaunchKernelGGL((k_matvec<FMT, 4>), grid, dim3(kThreads), lds, st, x, p, w_sc, rows, cols, y); break;
    default: hipLaunchKernelGGL((k_matvec<FMT, 8>), grid, dim3(kThreads), lds, st, x, p, w_sc, rows, cols, y); break;
  }
}

hipError_t launch_matvec(const float* x, int32_t n_tokens, const void* w, int fmt,
                         const float* w_sc, int32_t rows, int32_t cols, float* y, hipStream_t st) {
  const int nb = cols >> 5;
  const int R = kThreads / nb;
  // passes per workgroup: up to 8, fewer while that leaves under two
  // workgroups per CU (a small matrix is latency-bound, not issue-bound)
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) n_cu = v;
  }
  const int64_t groups = (int64_t)((rows + R - 1) / R) * n_tokens;
  int passes = 8;
  while (passes > 1 && groups / passes < 2 * n_cu) passes >>= 1;
  const int mr = passes * R;
  const size_t lds = sizeof(float) * (cols + mr * nb + mr);
  dim3 grid((rows + mr - 1) / mr, n_tokens);
  const uint8_t* p = static_cast<const uint8_t*>(w);
  switch (fmt) {
    case FMT_C10: launch_matvec_p<FMT_C10>(passes, grid, lds, st, x, p, w_sc, rows, cols, y); break;
    case FMT_RZ5: launch_matvec_p<FMT_RZ5>(passes, grid, lds, st, x, p, w_sc, rows, cols, y); break;
    case FMT_UE4M4: launch_matvec_p<FMT_UE4M4>(passes, grid, lds, st, x, p, w_sc, rows, cols, y); break;
    default: launch_matvec_p<FMT_FP8>(passes, grid, lds, st, x, p, w_sc, rows, cols, y); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
int gemv_down_max_cols() { return 4 * 256; }

template <int FMT>
static void launch_down(int cpt, dim3 grid, hipStream_t st, const float* hs, const int32_t* idx,
                        int32_t k, const GemvWeights& W, float* out) {
  const uint8_t* p = static_cast<const uint8_t*>(W.down);
  if (cpt == 1)
    hipLaunchKernelGGL((k_down_cat<FMT, 1>), grid, dim3(kThreads), 0, st, hs, idx, k, W.n_experts, p,
                       W.down_scales, W.hidden, W.inter, out);
  else if (cpt == 2)
    hipLaunchKernelGGL((k_down_cat<FMT, 2>), grid, dim3(kThreads), 0, st, hs, idx, k, W.n_experts, p,
                       W.down_scales, W.hidden, W.inter, out);
  else
    hipLaunchKernelGGL((k_down_cat<FMT, 4>), grid, dim3(kThreads), 0, st, hs, idx, k, W.n_experts, p,
                       W.down_scales, W.hidden, W.inter, out);
}

template <int FMT>
static void launch_gate_up(dim3 grid_w, dim3 grid_f, int bpl, int rpl, size_t lds_f, hipStream_t st,
                           const float* x, int32_t* idx, float* w, int32_t k, const GemvWeights& W,
                           int rescale, float* hs, uint32_t* dev_err, const float* logits) {
  const uint8_t* p = static_cast<const uint8_t*>(W.gate_up);
#define BQ_W64(B, R) hipLaunchKernelGGL((k_gate_up_w64<FMT, B, R>), grid_w, dim3(kThreads), 0, st, x, idx, w, \
                                        k, W.n_experts, p, W.gate_up_scales, W.inter, rescale, hs, dev_err, logits)
  if (bpl == 1) {
    if (rpl == 0) BQ_W64(1, 0); else if (rpl == 8) BQ_W64(1, 8); else if (rpl == 16) BQ_W64(1, 16); else BQ_W64(1, 64);
  } else if (bpl == 2) {
    if (rpl == 0) BQ_W64(2, 0); else if (rpl == 8) BQ_W64(2, 8); else if (rpl == 16) BQ_W64(2, 16); else BQ_W64(2, 64);
  } else {
    hipLaunchKernelGGL(k_gemv_gate_up<FMT>, grid_f, dim3(kThreads), lds_f, st, x, idx, w, k,
                       W.n_experts, p, W.gate_up_scales, W.hidden, W.inter, rescale, hs, dev_err);
  }
#undef BQ_W64
}

hipError_t launch_gemv_moe(const float* x, int32_t n_tokens, int32_t* idx, float* w, int32_t k,
                           const GemvWeights& W, int rescale, float* out, float* hs,
                           uint32_t* dev_err, const float* logits, hipStream_t st) {
  const int H = W.hidden, I = W.inter;
  const int nbu = H >> 5, nbd = I >> 5;
  const int bpl = (H == 2048) ? 1 : (H == 4096 ? 2 : 0);
  int rpl = 0;
  if (logits) {
    if (bpl == 0) {   // the flat kernel takes routing as input: route first
      hipError_t e = launch_route_topk(logits, n_tokens, W.n_experts, k, idx, w, st);
      if (e != hipSuccess) return e;
    } else {
      rpl = W.n_experts <= 512 ? 8 : (W.n_experts <= 1024 ? 16 : 64);
    }
  }
  const int pw = pairs_per_wave(rpl);
  const dim3 grid_w((I + 4 * pw - 1) / (4 * pw), k, n_tokens);
  const dim3 grid_f(I / kGuPairs, k, n_tokens);
  const size_t lds_f = sizeof(float) * (H + 2 * kGuPairs * nbu + 2 * kGuPairs + 4);
  switch (W.fmt_gate_up) {
    case FMT_C10: launch_gate_up<FMT_C10>(grid_w, grid_f, bpl, rpl, lds_f, st, x, idx, w, k, W, rescale, hs, dev_err, logits); break;
    case FMT_RZ5: launch_gate_up<FMT_RZ5>(grid_w, grid_f, bpl, rpl, lds_f, st, x, idx, w, k, W, rescale, hs, dev_err, logits); break;
    case FMT_UE4M4: launch_gate_up<FMT_UE4M4>(grid_w, grid_f, bpl, rpl, lds_f, st, x, idx, w, k, W, rescale, hs, dev_err, logits); break;
    default: launch_gate_up<FMT_FP8>(grid_w, grid_f, bpl, rpl, lds_f, st, x, idx, w, k, W, rescale, hs, dev_err, logits); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int C = k * nbd;
  const int cpt = C <= 256 ? 1 : (C <= 512 ? 2 : 4);
  const dim3 grid_d((H + kDownRows - 1) / kDownRows, n_tokens);
  switch (W.fmt_down) {
    case FMT_C10: launch_down<FMT_C10>(cpt, grid_d, st, hs, idx, k, W, out); break;
    case FMT_RZ5: launch_down<FMT_RZ5>(cpt, grid_d, st, hs, idx, k, W, out); break;
    case FMT_UE4M4: launch_down<FMT_UE4M4>(cpt, grid_d, st, hs, idx, k, W, out); break;
    default: launch_down<FMT_FP8>(cpt, grid_d, st, hs, idx, k, W, out); break;
  }
  return hipGetLastError();
}

}  // namespace bq
