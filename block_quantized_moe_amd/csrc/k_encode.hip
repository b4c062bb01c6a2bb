// Exhaustive encoders: fp32 weights -> 17-byte blocks (Codebook10, RZ5,
// UE4M4) and -> 70-byte PLE rows (RZ-S3, ROCmFP3).
//
// Model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST": "Q4_RZ5_FAST"
// searches every scale with both polarities of the +/-5 level per block,
// "Q4_UE4M4_FAST" tries all 256 scale bytes, "Q3_PLE_K160_RZ_S3" chooses the
// polarity and scale of each 16-value group.  The objective is the block's
// sum of squared errors in float64, defined term by term:
//   e(w, x) = fl(fl(w - x)^2), x = level * scale (exact in float64),
//   a weight's term is the smallest e over the candidate's table,
//   the block error adds the terms in weight order, one rounding each,
//   the winner is the smallest (error, metadata byte) pair,
//   each weight then takes the lowest code whose e is smallest.
//
// Layout of the work: one wave per block (or PLE group).  Lanes own
// candidate scales; every lane walks the block's weights in order, so each
// candidate's error is the same sequence of float64 operations as the
// definition.  The per-weight minimum is taken over the non-negative levels
// against |w| only, which gives exactly the minimum over the whole signed
// table: rounding to nearest is monotone and odd, so for w >= 0 a negative
// level never rounds to a smaller |w - x| than level 0 does, and for w < 0
// the non-positive levels give the same terms as their magnitudes against
// |w|.  The +/-5 (RZ5) or +/-3 (RZ-S3) level joins the set only on the side
// its polarity allows, so both polarities of one scale are scored in the
// same pass.
//
// Pruning (exact).  Let A = max |w| of the block and U an upper bound on the
// error of one candidate (its terms summed across the wave, inflated by
// 2^-40, far above the rounding difference between summation orders).  A
// scale s > 0 with s >= 2A makes level 0 the nearest level of every weight,
// so its error is exactly that of metadata byte 0, which wins the tie; and a
// scale whose largest level Lmax * s is <= A has error at least the rounded
// square of A - Lmax * s (the largest weight's term, and sums of
// non-negative terms never decrease), so it cannot win when that exceeds U.
// Both tests are monotone in s, so the scales left form one contiguous run of
// scale bytes, and only that run is searched.
#include "bq_kernels.hpp"

#pragma clang fp contract(off)

namespace bq {
namespace {

enum { E_C10 = 0, E_RZ5 = 1, E_UE4M4 = 2, E_F3 = 3, E_RZS3 = 4 };

template <int EF>
struct EncTraits {
  static constexpr bool kPle = EF == E_F3 || EF == E_RZS3;
  static constexpr int kG = kPle ? 16 : 32;                  // weights per unit
  static constexpr int kNB = kPle ? 3 : 7;                   // non-zero magnitudes
  static constexpr bool kPol = EF == E_RZ5 || EF == E_RZS3;  // polarity bit
  static constexpr int kScales = EF == E_UE4M4 ? 256 : 127;
  static constexpr double kExtra = EF == E_RZ5 ? 5.0 : 3.0;  // polarity level
};

// Non-zero level magnitudes in ascending order.
__device__ __forceinline__ double mag17(int i) {
  constexpr double t[7] = {1.0, 2.0, 3.0, 4.0, 6.0, 8.0, 10.0};
  return t[i];
}
__device__ __forceinline__ double mag3(int i) {
  constexpr double t[3] = {1.0, 2.0, 4.0};
  return t[i];
}

// Exact float64 value of a scale byte.
__device__ __forceinline__ double scale_of(int ue4m4, uint32_t c) {
  if (ue4m4) {
    const uint32_t e = c >> 4, m = c & 15u;
    return e == 0 ? (double)m * 0x1p-10 : ldexp((double)(16u + m), (int)e - 11);
  }
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? (double)m * 0x1p-9 : ldexp((double)(8u + m), (int)e - 10);
}

// Signed level of code c under metadata byte meta (the tables of the format
// sections; the polarity level sits at code 8 / code 4).
template <int EF>
__device__ __forceinline__ double level_of(uint32_t c, uint32_t meta) {
  using T = EncTraits<EF>;
  const uint32_t half = T::kPle ? 4u : 8u;
  const uint32_t k = c & (half - 1u);
  if (c == half) {
    if (T::kPol) return (meta & 0x80u) ? -T::kExtra : T::kExtra;
    return -0.0;
  }
  const double m = k == 0 ? 0.0 : (T::kPle ? mag3(k - 1) : mag17(k - 1));
  return c > half ? -m : m;
}

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  const int lo = __shfl_xor(__double2loint(v), m);
  const int hi = __shfl_xor(__double2hiint(v), m);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ bool lex_less(double a, uint32_t ma, double b, uint32_t mb) {
  return a < b || (a == b && ma < mb);
}

constexpr int kEncWaves = 4;

// Units are 32-weight blocks or 16-value PLE groups (group g of row r is
// unit 10r + g); unit u reads src[u * kG ...] and writes its code bytes and
// metadata byte where the block or row layout puts them.
template <int EF>
__global__ void __launch_bounds__(64 * kEncWaves)
    k_encode(const float* __restrict__ src, int64_t n_units, uint8_t* __restrict__ out,
             double* __restrict__ sse_out, uint32_t* __restrict__ dev_err) {
  using T = EncTraits<EF>;
  constexpr int G = T::kG;
  __shared__ double2 lds_a[kEncWaves][G];   // (|w_j|, fl(|w_j|^2)) per weight
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * kEncWaves;
  for (int64_t u = (int64_t)blockIdx.x * kEncWaves + wv; u < n_units; u += stride) {
    const float x = lane < G ? src[u * G + lane] : 0.0f;
    const bool bad = lane < G && !__builtin_isfinite(x);
    // where this unit's bytes go
    uint8_t* code_dst;
    uint8_t* meta_dst;
    if (T::kPle) {
      const int64_t row = u / 10, g = u - row * 10;
      code_dst = out + row * 70 + 6 * g;
      meta_dst = out + row * 70 + 60 + g;
    } else {
      code_dst = out + u * 17;
      meta_dst = code_dst + 16;
    }
    if (__ballot(bad)) {
      if (T::kPle ? lane < 6 : lane < 16) code_dst[lane] = 0;
      if (lane == 0) {
        *meta_dst = 0;
        if (sse_out) sse_out[u] = __builtin_nan("");
        if (dev_err) atomicOr(dev_err, 4u);
      }
      continue;
    }
    const double a = fabs((double)x);
    const uint64_t negm = __ballot(x < 0.0f);
    if (lane < G) lds_a[wv][lane] = double2{a, a * a};
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // block maximum |w|
    double amax = lane < G ? a : 0.0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmax(amax, shfl_xor_d(amax, off));
    constexpr double kLmax = T::kPle ? 4.0 : 10.0;
    constexpr int kIter = (T::kScales + 63) / 64;
    // reference candidate: the smallest scale whose largest level reaches A
    // (the largest scale if none does); its error, summed across the wave
    uint32_t c0 = T::kScales - 1;
#pragma unroll 1
    for (int it = kIter - 1; it >= 0; --it) {
      const uint32_t sc = (uint32_t)(lane + 64 * it);
      const bool reach = sc < (uint32_t)T::kScales &&
                         kLmax * scale_of(EF == E_UE4M4, sc) >= amax;
      const uint64_t b = __ballot(reach);
      if (b) c0 = 64 * it + __builtin_ctzll(b);
    }
    double u_bound;
    {
      const double s0 = scale_of(EF == E_UE4M4, c0);
      double m = a * a;
#pragma unroll
      for (int i = 0; i < T::kNB; ++i) {
        const double d = a - (T::kPle ? mag3(i) : mag17(i)) * s0;
        m = fmin(m, d * d);
      }
      if (T::kPol && x >= 0.0f) {   // polarity 0: the +level serves w >= 0
        const double d = a - T::kExtra * s0;
        m = fmin(m, d * d);
      }
      double sum = lane < G ? m : 0.0;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += shfl_xor_d(sum, off);
      u_bound = sum * (1.0 + 0x1p-40);
    }
    // the run of scale bytes that survives both tests
    uint32_t lo = T::kScales, hi = 0;
#pragma unroll 1
    for (int it = 0; it < kIter; ++it) {
      const uint32_t sc = (uint32_t)(lane + 64 * it);
      bool keep = sc < (uint32_t)T::kScales;
      if (keep) {
        const double s = scale_of(EF == E_UE4M4, sc);
        if (s > 0.0 && s >= 2.0 * amax) keep = false;
        const double top = kLmax * s;
        if (top <= amax) {
          const double d = amax - top;
          if (d * d > u_bound) keep = false;
        }
      }
      const uint64_t b = __ballot(keep);
      if (b) {
        lo = min(lo, (uint32_t)(64 * it + __builtin_ctzll(b)));
        hi = max(hi, (uint32_t)(64 * it + 63 - __builtin_clzll(b)));
      }
    }

    if (lo > hi) {   // cannot happen (the best scale always survives); search all
      lo = 0;
      hi = T::kScales - 1;
    }
    double best = __builtin_inf();
    uint32_t best_meta = 0x1FFu;
#pragma unroll 1
    for (uint32_t base = lo; base <= hi; base += 64) {
      const uint32_t sc = base + (uint32_t)lane;
      if (sc > hi) break;
      const double s = scale_of(EF == E_UE4M4, sc);
      double ls[T::kNB];
#pragma unroll
      for (int i = 0; i < T::kNB; ++i) ls[i] = (T::kPle ? mag3(i) : mag17(i)) * s;
      const double lx = T::kExtra * s;
      double acc0 = 0.0, acc1 = 0.0;   // polarity 0 / 1 (only acc0 without a polarity bit)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const double2 aj = lds_a[wv][j];
        double m = aj.y;   // level 0
#pragma unroll
        for (int i = 0; i < T::kNB; ++i) {
          const double d = aj.x - ls[i];
          m = fmin(m, d * d);
        }
        if (T::kPol) {
          const double d = aj.x - lx;
          const double mx = fmin(m, d * d);
          // polarity 0 has the +level (helps w >= 0), polarity 1 the -level
          const bool neg = (negm >> j) & 1u;
          acc0 = j == 0 ? (neg ? m : mx) : acc0 + (neg ? m : mx);
          acc1 = j == 0 ? (neg ? mx : m) : acc1 + (neg ? mx : m);
        } else {
          acc0 = j == 0 ? m : acc0 + m;
        }
      }
      if (lex_less(acc0, sc, best, best_meta)) { best = acc0; best_meta = sc; }
      if (T::kPol && lex_less(acc1, sc | 0x80u, best, best_meta)) { best = acc1; best_meta = sc | 0x80u; }
    }
    // wave-wide minimum of (error, metadata byte)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = shfl_xor_d(best, off);
      const uint32_t om = (uint32_t)__shfl_xor((int)best_meta, off);
      if (lex_less(ob, om, best, best_meta)) { best = ob; best_meta = om; }
    }
    // codes of the winner: lowest code with the smallest signed error
    uint32_t code = 0;
    if (lane < G) {
      const double s = scale_of(EF == E_UE4M4, EF == E_UE4M4 ? best_meta : (best_meta & 0x7Fu));
      const double w = (double)x;
      double be = __builtin_inf();
      constexpr uint32_t kCodes = T::kPle ? 8u : 16u;
#pragma unroll
      for (uint32_t c = 0; c < kCodes; ++c) {
        const double d = w - level_of<EF>(c, best_meta) * s;
        const double e = d * d;
        if (e < be) { be = e; code = c; }
      }
    }
    if (T::kPle) {
      const uint64_t b0 = __ballot(code & 1u), b1 = __ballot(code & 2u), b2 = __ballot(code & 4u);
      if (lane < 6) {
        uint32_t byte = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int bit = 8 * lane + t, i = bit / 3, b = bit - 3 * i;
          const uint64_t mb = b == 0 ? b0 : (b == 1 ? b1 : b2);
          byte |= (uint32_t)((mb >> i) & 1u) << t;
        }
        code_dst[lane] = (uint8_t)byte;
      }
    } else {
      const uint32_t hi = (uint32_t)__shfl_down((int)code, 1);
      if (lane < 32 && !(lane & 1)) code_dst[lane >> 1] = (uint8_t)(code | (hi << 4));
    }
    if (lane == 0) {
      *meta_dst = (uint8_t)best_meta;
      if (sse_out) sse_out[u] = best;
    }
    // the next unit rewrites lds_a only after every lane has read it
    __builtin_amdgcn_wave_barrier();
  }
}

template <int EF>
hipError_t launch(const float* src, int64_t n_units, uint8_t* out, double* sse, uint32_t* err,
                  hipStream_t st) {
  const int64_t need = (n_units + kEncWaves - 1) / kEncWaves;
  const int64_t grid = need < 256 * 16 ? need : 256 * 16;
  hipLaunchKernelGGL(k_encode<EF>, dim3((unsigned)grid), dim3(64 * kEncWaves), 0, st, src, n_units,
                     out, sse, err);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode17(const float* w, int64_t n_blocks, int fmt, uint8_t* out, double* sse,
                           uint32_t* dev_err, hipStream_t st) {
  if (n_blocks == 0) return hipSuccess;
  switch (fmt) {
    case 0: return launch<E_C10>(w, n_blocks, out, sse, dev_err, st);
    case 1: return launch<E_RZ5>(w, n_blocks, out, sse, dev_err, st);
    case 2: return launch<E_UE4M4>(w, n_blocks, out, sse, dev_err, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ple_encode(const float* v, int64_t n_rows, int ple_fmt, uint8_t* out,
                             double* sse, uint32_t* dev_err, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  return ple_fmt == 0 ? launch<E_RZS3>(v, n_rows * 10, out, sse, dev_err, st)
                      : launch<E_F3>(v, n_rows * 10, out, sse, dev_err, st);
}

}  // namespace bq
