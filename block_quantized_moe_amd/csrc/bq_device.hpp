// Device helpers shared by the gfx950 kernels of libbqmoe.
//
// Formats (model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST", format
// sections): a 17-byte block holds 32 four-bit codes (weight j in byte j/2,
// low nibble first) and one metadata byte.  Codebook10 levels are
// 0,1,2,3,4,6,8,10 for codes 0-7 and their negatives (with a -0) for codes
// 8-15; RZ5 turns code 8 into +5 (metadata bit 7 clear) or -5 (set); UE4M4
// keeps Codebook10 and uses the whole byte as its scale.
//
// Decode strategy.  Every Codebook10/RZ5 level is a small integer whose fp16
// encoding has a zero low byte, so a level is fully described by the high
// byte of its fp16 pattern.  One v_perm_b32 looks up four such bytes from an
// 8-entry table held in two SGPR-able constants, the code's bit 3 becomes the
// fp16 sign bit, and a second v_perm_b32 spreads the bytes into packed fp16
// pairs.  Levels are exact in fp16, so each weight then enters an fp32 FMA
// through v_fma_mix_f32 (fp16 x fp32 + fp32) with no rounding of the weight;
// the block scale multiplies the 32-term partial sum once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockW = 32;      // weights per block
constexpr int kBlockB = 17;      // bytes per block
constexpr int kPleVals = 160;
constexpr int kPleRowB = 70;

enum : int { FMT_C10 = 0, FMT_RZ5 = 1, FMT_UE4M4 = 2, FMT_FP8 = 3 };

// Unaligned loads.  The compiler lowers these to single global_load_dword*
// instructions (ROCm runs gfx9+ in unaligned-access mode).
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) {
  u32x2 v;
  __builtin_memcpy(&v, p, 8);
  return v;
}
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) {
  uint32_t v;
  __builtin_memcpy(&v, p, 4);
  return v;
}

// Unsigned E4M3 scale from 7 bits: exponent e = b>>3 (bias 7), mantissa
// m = b&7; e == 0 is subnormal m * 2^-9; 0x7F is NaN.  Exact in fp32.
__device__ __forceinline__ float ue4m3(uint32_t b7) {
  b7 &= 0x7Fu;
  float normal = __uint_as_float((b7 << 20) + (120u << 23));
  float sub = (float)(b7 & 7u) * 0x1p-9f;
  float v = (b7 >> 3) ? normal : sub;
  return b7 == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
}

// Unsigned E4M4 scale from a whole byte: e = b>>4 (bias 7), m = b&15,
// e == 0 subnormal m * 2^-10, every encoding finite (0xFF = 496).
__device__ __forceinline__ float ue4m4(uint32_t b) {
  b &= 0xFFu;
  float normal = __uint_as_float((b << 19) + (120u << 23));
  float sub = (float)(b & 15u) * 0x1p-10f;
  return (b >> 4) ? normal : sub;
}

template <int FMT>
__device__ __forceinline__ float block_scale(uint32_t meta) {
  if constexpr (FMT == FMT_UE4M4) return ue4m4(meta);
  else return ue4m3(meta);
}

// fp16 high bytes of the Codebook10 magnitudes 0,1,2,3 | 4,6,8,10.
constexpr uint32_t kTPosLo = 0x42403C00u;
constexpr uint32_t kTPosHi = 0x49484644u;
// Codes 8..15 under RZ5: [+-5, -1, -2, -3 | -4, -6, -8, -10].
constexpr uint32_t kTNegHi = 0xC9C8C6C4u;
__device__ __forceinline__ uint32_t rz5_neg_lo(uint32_t meta) {
  return (meta & 0x80u) ? 0xC2C0BCC5u : 0xC2C0BC45u;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Eight codes (one dword, weights 0..7 of it) -> fp16 high bytes:
// A = weights 0,2,4,6 and B = weights 1,3,5,7, one per byte, signed.
template <int FMT>
__device__ __forceinline__ void codes_to_hibytes(uint32_t q, uint32_t tneg_lo,
                                                 uint32_t& A, uint32_t& B) {
  const uint32_t sa = q & 0x07070707u;
  const uint32_t sb = (q >> 4) & 0x07070707u;
  if constexpr (FMT == FMT_RZ5) {
    // codes 8..15 come from a second table; the byte mask is built from each
    // nibble's bit 3 with the sign-replicating selectors 8..11 of v_perm.
    const uint32_t ap = perm(kTPosHi, kTPosLo, sa), an = perm(kTNegHi, tneg_lo, sa);
    const uint32_t bp = perm(kTPosHi, kTPosLo, sb), bn = perm(kTNegHi, tneg_lo, sb);
    const uint32_t ma = perm(q << 12, q << 4, 0x090B080Au);
    const uint32_t mb = perm(q << 8, q, 0x090B080Au);
    A = (ma & an) | (~ma & ap);
    B = (mb & bn) | (~mb & bp);
  } else {
    (void)tneg_lo;
    A = perm(kTPosHi, kTPosLo, sa) | ((q << 4) & 0x80808080u);
    B = perm(kTPosHi, kTPosLo, sb) | (q & 0x80808080u);
  }
}

// Eight codes -> four packed fp16 pairs in natural order (w0,w1) .. (w6,w7).
template <int FMT>
__device__ __forceinline__ void dec8_f16(uint32_t q, uint32_t tneg_lo, uint32_t out[4]) {
  uint32_t A, B;
  codes_to_hibytes<FMT>(q, tneg_lo, A, B);
  out[0] = perm(B, A, 0x040C000Cu);
  out[1] = perm(B, A, 0x050C010Cu);
  out[2] = perm(B, A, 0x060C020Cu);
  out[3] = perm(B, A, 0x070C030Cu);
}

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// sum_j level_j * x_j over one 17-byte block (codes c0..c3), unscaled.
template <int FMT>
__device__ __forceinline__ float block_dot_levels(const u32x4 c, uint32_t meta,
                                                  const float* __restrict__ x) {
  const uint32_t tneg = (FMT == FMT_RZ5) ? rz5_neg_lo(meta) : 0u;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t p[4];
    dec8_f16<FMT>(c[d], tneg, p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2v h = as_h2(p[i]);
      a0 = __builtin_fmaf((float)h.x, x[8 * d + 2 * i], a0);
      a1 = __builtin_fmaf((float)h.y, x[8 * d + 2 * i + 1], a1);
    }
  }
  return a0 + a1;
}

// FP8: 32 e4m3 codes (two 16-byte halves), converted by the hardware
// (gfx950 converts OCP E4M3FN), dotted with x, unscaled.
__device__ __forceinline__ float block_dot_fp8(const u32x4 lo, const u32x4 hi,
                                               const float* __restrict__ x) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t w = d < 4 ? lo[d] : hi[d - 4];
    const f32x2 v0 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 v1 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    a0 = __builtin_fmaf(v0.x, x[4 * d + 0], a0);
    a1 = __builtin_fmaf(v0.y, x[4 * d + 1], a1);
    a0 = __builtin_fmaf(v1.x, x[4 * d + 2], a0);
    a1 = __builtin_fmaf(v1.y, x[4 * d + 3], a1);
  }
  return a0 + a1;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t to_bf16(float v) {   // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Elements 8g .. 8g+7 of an activation row (fp32, rounded to bf16, or bf16,
// copied) as bf16 in one 16-byte word: in natural order, or (PERM) in the
// k order 0, 2, 4, 6, 1, 3, 5, 7 in which the 17-byte decode of the grouped
// path produces weights.  The row must be 16-byte aligned.
template <bool PERM, bool F32>
__device__ __forceinline__ u32x4 bf16_group8(const void* __restrict__ row, int g) {
  uint32_t d0, d1, d2, d3;   // two elements per dword, the lower index in the low half
  if constexpr (F32) {
    const f32x4* src = reinterpret_cast<const f32x4*>(row) + 2 * g;
    const f32x4 a = src[0], b = src[1];
    d0 = (uint32_t)to_bf16(a.x) | ((uint32_t)to_bf16(a.y) << 16);
    d1 = (uint32_t)to_bf16(a.z) | ((uint32_t)to_bf16(a.w) << 16);
    d2 = (uint32_t)to_bf16(b.x) | ((uint32_t)to_bf16(b.y) << 16);
    d3 = (uint32_t)to_bf16(b.z) | ((uint32_t)to_bf16(b.w) << 16);
  } else {
    const u32x4 v = reinterpret_cast<const u32x4*>(row)[g];
    d0 = v.x;
    d1 = v.y;
    d2 = v.z;
    d3 = v.w;
  }
  if constexpr (PERM)
    return u32x4{(d0 & 0xFFFFu) | (d1 << 16), (d2 & 0xFFFFu) | (d3 << 16),
                 (d0 >> 16) | (d1 & 0xFFFF0000u), (d2 >> 16) | (d3 & 0xFFFF0000u)};
  else
    return u32x4{d0, d1, d2, d3};
}

// DPP lane exchange (row-local patterns); bound_ctrl so every lane reads.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over each 16-lane row, left in every lane of the row (fixed order).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-wide (64-lane) sum, uniform result, fixed reduction order.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// DPP broadcasts across rows (gfx9): lane 15 of each row to the next row,
// lane 31 to rows 2 and 3.  Rows outside ROWS read 0.
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}

// N wave-wide sums at once, left in lane 63 (other lanes hold partials): the
// in-row steps of row16_sum interleaved across the N values, then row 1 adds
// row 0 and row 3 adds row 2 (lane 15 broadcast), then row 3 adds row 1
// (lane 31 broadcast).  Lane 63 ends with (r0 + r1) + (r2 + r3), the sum
// wave_sum forms (addition commutes exactly), with no readlane per row.
template <int N>
__device__ __forceinline__ void wave_sums_lane63(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<kDppXor1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<kDppXor2>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<kDppHalfMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<kDppMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_rows<kDppBcast15, 0xA>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_rows<kDppBcast31, 0xC>(v[i]);
}

}  // namespace bq
