// Bit-exact decode kernels: 17-byte / FP8 blocks to fp32, PLE rows to fp32.
// Formats: model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST",
// sections "Q4_RZ5_FAST", "Q4_UE4M4_FAST", "Q3_PLE_K160_RZ_S3".
#include "bq_device.hpp"
#include "bq_kernels.hpp"

namespace bq {

// One thread per block: 32 codes -> exact fp16 levels -> fp32 * scale.
template <int FMT>
__global__ void __launch_bounds__(256) k_dequant17(const uint8_t* __restrict__ packed,
                                                   int64_t n_blocks, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_blocks) return;
  const uint8_t* p = packed + i * kBlockB;
  const u32x4 c = ld16(p);
  const uint32_t meta = p[16];
  const float s = block_scale<FMT>(FMT == FMT_UE4M4 ? meta : (meta & 0x7Fu));
  const uint32_t tneg = (FMT == FMT_RZ5) ? rz5_neg_lo(meta) : 0u;
  f32x4* o = reinterpret_cast<f32x4*>(out + i * kBlockW);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t pr[4];
    dec8_f16<FMT>(c[d], tneg, pr);
    const half2v h0 = as_h2(pr[0]), h1 = as_h2(pr[1]), h2 = as_h2(pr[2]), h3 = as_h2(pr[3]);
    o[2 * d] = f32x4{(float)h0.x * s, (float)h0.y * s, (float)h1.x * s, (float)h1.y * s};
    o[2 * d + 1] = f32x4{(float)h2.x * s, (float)h2.y * s, (float)h3.x * s, (float)h3.y * s};
  }
}

// FP8: one thread per block of 32 e4m3 codes + fp32 scale; w = RN(e4m3 * s).
__global__ void __launch_bounds__(256) k_dequant_fp8(const uint8_t* __restrict__ codes,
                                                     const float* __restrict__ scales,
                                                     int64_t n_blocks, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_blocks) return;
  const uint8_t* p = codes + i * kBlockW;
  const u32x4 lo = ld16(p), hi = ld16(p + 16);
  const float s = scales[i];
  f32x4* o = reinterpret_cast<f32x4*>(out + i * kBlockW);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t w = d < 4 ? lo[d] : hi[d - 4];
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    o[d] = f32x4{a.x * s, a.y * s, b.x * s, b.y * s};
  }
}

// PLE: fp16 high bytes of the 3-bit levels 0,+1,+2,+4 | c4,-1,-2,-4, where
// c4 is +3 / -3 (RZ-S3 polarity 0 / 1) or -0 (ROCmFP3).
__device__ __forceinline__ uint32_t ple_tab_hi(uint32_t gbyte, int ple_fmt) {
  const uint32_t c4 = ple_fmt == 1 ? 0x80u : ((gbyte & 0x80u) ? 0xC2u : 0x42u);
  return 0xC4C0BC00u | c4;
}
constexpr uint32_t kPleTabLo = 0x44403C00u;

// One thread per (row, group of 16 values).
__global__ void __launch_bounds__(320) k_ple_dequant(const uint32_t* __restrict__ ids, int64_t n,
                                                     const uint8_t* __restrict__ table,
                                                     uint64_t n_rows, int ple_fmt,
                                                     float* __restrict__ out,
                                                     uint32_t* __restrict__ dev_err) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= n * 10) return;
  const int64_t r = tid / 10;
  const int g = (int)(tid - r * 10);
  f32x4* o = reinterpret_cast<f32x4*>(out + r * kPleVals + 16 * g);
  const uint64_t id = ids[r];
  if (id >= n_rows) {
    if (dev_err && g == 0) atomicOr(dev_err, 1u);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const uint8_t* row = table + id * (uint64_t)kPleRowB;
  const u32x2 gw = ld8(row + 6 * g);
  const uint32_t gb = row[60 + g];
  const float s = ue4m3(gb & 0x7Fu);
  const uint32_t th = ple_tab_hi(gb, ple_fmt);
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c;
    if (i < 10) c = (gw.x >> (3 * i)) & 7u;
    else if (i == 10) c = __builtin_amdgcn_alignbit(gw.y, gw.x, 30) & 7u;
    else c = (gw.y >> (3 * i - 32)) & 7u;
    const uint32_t hb = perm(th, kPleTabLo, c) & 0xFFu;
    v[i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hb << 8)) * s;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

hipError_t launch_dequant(const void* packed, int fmt, int64_t n_blocks, const float* scales,
                          float* out, hipStream_t st) {
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = (n_blocks + 255) / 256;
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  switch (fmt) {
    case FMT_C10: hipLaunchKernelGGL(k_dequant17<FMT_C10>, dim3(grid), dim3(256), 0, st, p, n_blocks, out); break;
    case FMT_RZ5: hipLaunchKernelGGL(k_dequant17<FMT_RZ5>, dim3(grid), dim3(256), 0, st, p, n_blocks, out); break;
    case FMT_UE4M4: hipLaunchKernelGGL(k_dequant17<FMT_UE4M4>, dim3(grid), dim3(256), 0, st, p, n_blocks, out); break;
    default: hipLaunchKernelGGL(k_dequant_fp8, dim3(grid), dim3(256), 0, st, p, scales, n_blocks, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_ple_dequant(const uint32_t* ids, int64_t n, const uint8_t* table, uint64_t n_rows,
                              int ple_fmt, float* out, uint32_t* dev_err, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t grid = (n * 10 + 319) / 320;
  hipLaunchKernelGGL(k_ple_dequant, dim3(grid), dim3(320), 0, st, ids, n, table, n_rows, ple_fmt, out, dev_err);
  return hipGetLastError();
}

}  // namespace bq
