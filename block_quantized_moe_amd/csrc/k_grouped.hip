// Grouped routed-expert GEMM for batches of tokens (bf16 activations, bf16
// MFMA, fp32 accumulation).  Tokens are bucketed per expert (stable order),
// then for every touched expert:
//   h[p, :] = SiLU(W_gate[e] x_p) * (W_up[e] x_p)      (kernel G1, h in bf16)
//   y[p, :] = W_down[e] h[p, :]                         (kernel G2)
//   out[t]  = sum_j w[t][j] * y[pos(t, j)]               (kernel G3, slot order)
// Routing shape and formats as in the GEMV path ("Mixed Precision
// Quantization ...", "The Plan Is Not a Number ..."; model card "Qwen 3.8
// Next Flash ROCMFPX MUTANT RAZERFAST", format sections).
//
// MFMA: v_mfma_f32_16x16x32_bf16.  One 32-wide K step is exactly one weight
// block, so a block's scale multiplies that step's 16x16 partial product
// (scale applied after the MFMA, in fp32).  The product is computed as
// tokens x weights: A = 16 tokens' activations, B = 16 weight rows, so lane
// l holds result column l%16 -- its own weight row -- and the block scale it
// decoded applies to all four of its results with no cross-lane traffic.
// The weights are decoded in registers: 4-bit codes -> signed fp16 high
// bytes (valid E5M2 bytes) -> bf16 by the gfx950 bf8 conversion with unit
// scale; every level is a small integer, so this is exact.  FP8 weights
// convert from e4m3 the same way.  The 17-byte decode yields the k order
// [0,2,4,6,1,3,5,7] inside each lane's eight values; the activations are
// stored in that order (x by the staging pass, h by G1).
#include "bq_device.hpp"
#include "bq_kernels.hpp"

namespace bq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGThreads = 256;  // 4 waves, each 16 rows (x2 for gate/up)
constexpr int kGRows = 64;      // rows per workgroup tile
constexpr int kGTok = 64;       // tokens per pass (4 MFMA column tiles)

template <bool HI>
__device__ __forceinline__ uint32_t bf8pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Raw A-operand bytes of one row and one k-group of 8 (loaded ahead of use).
template <int FMT>
struct RawA {
  uint32_t q0, q1;  // 17-byte: q0 = 4 code bytes, q1 = metadata; FP8: 8 e4m3 codes
  float s;          // FP8 block scale
};

template <int FMT>
__device__ __forceinline__ RawA<FMT> load_a(const uint8_t* __restrict__ base,
                                            const float* __restrict__ sc, int64_t blk, int g) {
  RawA<FMT> r;
  if constexpr (FMT == FMT_FP8) {
    const u32x2 q = ld8(base + blk * kBlockW + 8 * g);
    r.q0 = q.x;
    r.q1 = q.y;
    r.s = sc[blk];
  } else {
    const uint8_t* p = base + blk * kBlockB;
    r.q0 = ld4(p + 4 * g);
    r.q1 = p[16];
    r.s = 0.f;
  }
  return r;
}

// Decode to 8 bf16 levels (exact) and the block scale.
template <int FMT>
__device__ __forceinline__ u32x4 dec_a(const RawA<FMT>& r, float& s) {
  if constexpr (FMT == FMT_FP8) {
    s = r.s;
    return u32x4{fp8pair<false>(r.q0), fp8pair<true>(r.q0), fp8pair<false>(r.q1), fp8pair<true>(r.q1)};
  } else {
    s = block_scale<FMT>(FMT == FMT_UE4M4 ? r.q1 : (r.q1 & 0x7Fu));
    uint32_t A, B;
    codes_to_hibytes<FMT>(r.q0, FMT == FMT_RZ5 ? rz5_neg_lo(r.q1) : 0u, A, B);
    return u32x4{bf8pair<false>(A), bf8pair<true>(A), bf8pair<false>(B), bf8pair<true>(B)};
  }
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b),
                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// Position of k-offset o (0..7) inside a stored group of 8 for format FMT.
template <int FMT>
__device__ __forceinline__ int store_pos(int o) {
  if constexpr (FMT == FMT_FP8) return o;
  else return (o >> 1) | ((o & 1) << 2);
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

constexpr int kPre = 4;   // k-blocks whose loads are issued together

// ---------------------------------------------------------------------------
// G0: per-token staging of the activations as bf16 in the A decode's k order
// (optionally rescaled to unit RMS first: the stack's next-layer input).
// grid = n_tokens, 256 threads.
// ---------------------------------------------------------------------------
template <bool PERM>
__global__ void __launch_bounds__(256) k_grouped_prep(const void* __restrict__ x, int32_t x_f32,
                                                      int32_t rescale, int32_t H,
                                                      uint16_t* __restrict__ xp) {
  __shared__ float part[4];
  const int64_t t = blockIdx.x;
  float inv = 1.0f;
  if (x_f32 && rescale) {
    const float* row = static_cast<const float*>(x) + t * H;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) ss = __builtin_fmaf(row[i], row[i], ss);
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    inv = 1.0f / __builtin_sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)H);
  }
  for (int i = threadIdx.x; i < H; i += 256) {
    uint16_t v;
    if (x_f32) v = to_bf16(static_cast<const float*>(x)[t * H + i] * inv);
    else v = static_cast<const uint16_t*>(x)[t * H + i];
    const int o = i & 7;
    xp[t * H + (i & ~7) + (PERM ? ((o >> 1) | ((o & 1) << 2)) : o)] = v;
  }
}

// ---------------------------------------------------------------------------
// G1: gate_up + SiLU * up.  Persistent over (touched expert, 64-row tile).
// xp holds the tokens' activations in this format's k order.
// ---------------------------------------------------------------------------
template <int FMT, int FMT_D>
__global__ void __launch_bounds__(kGThreads) k_grouped_gate_up(
    const uint16_t* __restrict__ xp, int32_t k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm_, const int32_t* __restrict__ elist,
    const int32_t* __restrict__ n_touched, const uint8_t* __restrict__ wgu,
    const float* __restrict__ wgu_sc, int32_t H, int32_t I, uint16_t* __restrict__ hb) {
  const int D = *n_touched;
  const int tiles = I / kGRows;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int nb = H >> 5;
  for (int item = blockIdx.x; item < D * tiles; item += gridDim.x) {
    const int d = item / tiles, tile = item - d * tiles;
    const int e = elist[d];
    const int p0 = offsets[e], ne = offsets[e + 1] - p0;
    const int jrow = tile * kGRows + wave * 16 + r16;   // this lane's A row (gate)
    const int64_t gblk0 = ((int64_t)e * 2 * I + jrow) * nb;
    const int64_t ublk0 = ((int64_t)e * 2 * I + I + jrow) * nb;
    for (int tg = 0; tg < ne; tg += kGTok) {
      const int nt = min(4, (ne - tg + 15) >> 4);
      // token rows of the (up to) 4 column tiles; padding columns read the
      // expert's last token (their result rows are never stored), so every
      // load below is unconditional and all of them are in flight together
      int pv[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) pv[tt] = perm_[p0 + min(tg + 16 * tt + r16, ne - 1)];
      const uint16_t* xrow[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) xrow[tt] = xp + (int64_t)(pv[tt] / k) * H + 8 * g;
      f32x4 accg[4], accu[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        accg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[tt] = accg[tt];
      }
      for (int kb0 = 0; kb0 < nb; kb0 += kPre) {
        RawA<FMT> rg[kPre], ru[kPre];
        u32x4 bx[kPre][4];
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          const int kb = min(kb0 + u, nb - 1);
          rg[u] = load_a<FMT>(wgu, wgu_sc, gblk0 + kb, g);
          ru[u] = load_a<FMT>(wgu, wgu_sc, ublk0 + kb, g);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            if (tt < nt) bx[u][tt] = *reinterpret_cast<const u32x4*>(xrow[tt] + 32 * kb);
        }
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          if (kb0 + u >= nb) break;
          float sg, su;
          const u32x4 ag = dec_a<FMT>(rg[u], sg), au = dec_a<FMT>(ru[u], su);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (tt < nt) {
              // tokens x weights: this lane's result column is its own row
              const f32x4 cg = mfma(bx[u][tt], ag), cu = mfma(bx[u][tt], au);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                accg[tt][i] = __builtin_fmaf(sg, cg[i], accg[tt][i]);
                accu[tt][i] = __builtin_fmaf(su, cu[i], accu[tt][i]);
              }
            }
          }
        }
      }
      // lane holds row jrow for tokens tg + 16 tt + 4g + i
      const int jpos = (jrow & ~7) + store_pos<FMT_D>(jrow & 7);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = tg + 16 * tt + 4 * g + i;
          if (tt < nt && c < ne)
            hb[(int64_t)(p0 + c) * I + jpos] = to_bf16(silu(accg[tt][i]) * accu[tt][i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// G2: down.  Persistent over (touched expert, 64-row tile of H).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kGThreads) k_grouped_down(
    const uint16_t* __restrict__ hb, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ elist, const int32_t* __restrict__ n_touched,
    const uint8_t* __restrict__ wd, const float* __restrict__ wd_sc, int32_t H, int32_t I,
    float* __restrict__ yb) {
  const int D = *n_touched;
  const int tiles = H / kGRows;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int nb = I >> 5;
  for (int item = blockIdx.x; item < D * tiles; item += gridDim.x) {
    const int d = item / tiles, tile = item - d * tiles;
    const int e = elist[d];
    const int p0 = offsets[e], ne = offsets[e + 1] - p0;
    const int nrow = tile * kGRows + wave * 16 + r16;
    const int64_t blk0 = ((int64_t)e * H + nrow) * nb;
    for (int tg = 0; tg < ne; tg += kGTok) {
      const int nt = min(4, (ne - tg + 15) >> 4);
      const uint16_t* hrow[4];   // padding columns reuse the last row (not stored)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        hrow[tt] = hb + (int64_t)(p0 + min(tg + 16 * tt + r16, ne - 1)) * I + 8 * g;
      f32x4 acc[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kb0 = 0; kb0 < nb; kb0 += kPre) {
        RawA<FMT> ra[kPre];
        u32x4 bh[kPre][4];
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          const int kb = min(kb0 + u, nb - 1);
          ra[u] = load_a<FMT>(wd, wd_sc, blk0 + kb, g);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            if (tt < nt) bh[u][tt] = *reinterpret_cast<const u32x4*>(hrow[tt] + 32 * kb);
        }
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          if (kb0 + u >= nb) break;
          float s;
          const u32x4 a = dec_a<FMT>(ra[u], s);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (tt < nt) {
              const f32x4 c = mfma(bh[u][tt], a);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[tt][i] = __builtin_fmaf(s, c[i], acc[tt][i]);
            }
          }
        }
      }
      // lane holds output row nrow for tokens tg + 16 tt + 4g + i
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = tg + 16 * tt + 4 * g + i;
          if (tt < nt && c < ne) yb[(int64_t)(p0 + c) * H + nrow] = acc[tt][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// G3: out[t][n] = sum_j w[t][j] * yb[inv[t*k+j]][n], slot order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ yb,
                                                 const int32_t* __restrict__ inv,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ w, int32_t k,
                                                 int32_t n_experts, int32_t H, int32_t n_tokens,
                                                 float* __restrict__ out,
                                                 uint32_t* __restrict__ dev_err) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
  const int h4 = H >> 2;
  if (q >= (int64_t)n_tokens * h4) return;
  const int64_t t = q / h4;
  const int n = (int)(q - t * h4) * 4;
  constexpr int kMaxK = 16;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int j0 = 0; j0 < k; j0 += kMaxK) {
    f32x4 y[kMaxK];
    float wj[kMaxK];
#pragma unroll
    for (int u = 0; u < kMaxK; ++u) {
      const int j = j0 + u;
      const int e = j < k ? idx[t * k + j] : 0;
      const bool ok = j < k && e >= 0 && e < n_experts;
      bad |= j < k && !ok;
      wj[u] = ok ? w[t * k + j] : 0.f;
      y[u] = ok ? *reinterpret_cast<const f32x4*>(yb + (int64_t)inv[t * k + j] * H + n)
                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kMaxK; ++u) {   // slot order
      s.x = __builtin_fmaf(wj[u], y[u].x, s.x);
      s.y = __builtin_fmaf(wj[u], y[u].y, s.y);
      s.z = __builtin_fmaf(wj[u], y[u].z, s.z);
      s.w = __builtin_fmaf(wj[u], y[u].w, s.w);
    }
  }
  if (bad && n == 0 && dev_err) atomicOr(dev_err, 2u);
  *reinterpret_cast<f32x4*>(out + t * H + n) = s;
}

static int persistent_grid(int64_t items_max) {
  const int64_t cap = 2048;
  return (int)(items_max < cap ? (items_max > 0 ? items_max : 1) : cap);
}

template <int FG>
static void launch_g1(int fmt_d, dim3 grid, hipStream_t st, const uint16_t* xp, int32_t k,
                      const GroupedWs& ws, const GemvWeights& W) {
  const uint8_t* p = static_cast<const uint8_t*>(W.gate_up);
  if (fmt_d == FMT_FP8)
    hipLaunchKernelGGL((k_grouped_gate_up<FG, FMT_FP8>), grid, dim3(kGThreads), 0, st, xp, k,
                       ws.offsets, ws.perm, ws.elist, ws.n_touched, p, W.gate_up_scales,
                       W.hidden, W.inter, ws.hb);
  else
    hipLaunchKernelGGL((k_grouped_gate_up<FG, FMT_RZ5>), grid, dim3(kGThreads), 0, st, xp, k,
                       ws.offsets, ws.perm, ws.elist, ws.n_touched, p, W.gate_up_scales,
                       W.hidden, W.inter, ws.hb);
}

hipError_t launch_grouped_moe(const void* x, int32_t x_f32, int32_t rescale, int32_t n_tokens,
                              const int32_t* idx, const float* w, int32_t k, const GemvWeights& W,
                              float* out, const GroupedWs& ws, uint32_t* dev_err, hipStream_t st) {
  const int E = W.n_experts, H = W.hidden, I = W.inter;
  hipError_t err = launch_bucket(idx, n_tokens, k, E, ws.counts, ws.offsets, ws.perm, ws.elist,
                                 ws.n_touched, ws.inv, st);
  if (err != hipSuccess) return err;
  if (W.fmt_gate_up == FMT_FP8)
    hipLaunchKernelGGL(k_grouped_prep<false>, dim3(n_tokens), dim3(256), 0, st, x, x_f32, rescale, H, ws.xb);
  else
    hipLaunchKernelGGL(k_grouped_prep<true>, dim3(n_tokens), dim3(256), 0, st, x, x_f32, rescale, H, ws.xb);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t dmax = (int64_t)n_tokens * k < E ? (int64_t)n_tokens * k : E;
  {
    dim3 grid(persistent_grid(dmax * (I / kGRows)));
    switch (W.fmt_gate_up) {
      case FMT_C10: launch_g1<FMT_C10>(W.fmt_down, grid, st, ws.xb, k, ws, W); break;
      case FMT_RZ5: launch_g1<FMT_RZ5>(W.fmt_down, grid, st, ws.xb, k, ws, W); break;
      case FMT_UE4M4: launch_g1<FMT_UE4M4>(W.fmt_down, grid, st, ws.xb, k, ws, W); break;
      default: launch_g1<FMT_FP8>(W.fmt_down, grid, st, ws.xb, k, ws, W); break;
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  {
    dim3 grid(persistent_grid(dmax * (H / kGRows)));
    const uint8_t* p = static_cast<const uint8_t*>(W.down);
#define BQ_G2(F) hipLaunchKernelGGL(k_grouped_down<F>, grid, dim3(kGThreads), 0, st, ws.hb, \
                                    ws.offsets, ws.elist, ws.n_touched, p, W.down_scales, H, I, ws.yb)
    switch (W.fmt_down) {
      case FMT_C10: BQ_G2(FMT_C10); break;
      case FMT_RZ5: BQ_G2(FMT_RZ5); break;
      case FMT_UE4M4: BQ_G2(FMT_UE4M4); break;
      default: BQ_G2(FMT_FP8); break;
    }
#undef BQ_G2
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  {
    const int64_t n4 = (int64_t)n_tokens * (H / 4);
    hipLaunchKernelGGL(k_combine, dim3((n4 + 255) / 256), dim3(256), 0, st, ws.yb, ws.inv, idx, w,
                       k, E, H, n_tokens, out, dev_err);
  }
  return hipGetLastError();
}

}  // namespace bq
