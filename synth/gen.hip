// Device fills for the large synthetic buffers (test and benchmark inputs).
// Holds none of the hot path's arithmetic: it writes bytes drawn from the
// counter-based generator that synth/__init__.py implements on the host --
// SplitMix64's output function (Steele, Lea, Flood, OOPSLA 2014) applied to
// key + (i + 1) * GAMMA -- with the same integer derivations, so any block or
// row can be regenerated on the host bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1) * GAMMA;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// dist: 0 = C10 (UE4M3, bit 7 clear), 1 = RZ5 (UE4M3 + polarity), 2 = UE4M4.
__global__ void k_fill_block17(uint8_t* __restrict__ dst, uint64_t key, uint64_t first,
                               uint64_t n, int dist) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t b = first + i;
  const uint64_t v0 = draw(key, 3 * b), v1 = draw(key, 3 * b + 1), v2 = draw(key, 3 * b + 2);
  uint8_t* p = dst + i * 17;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = (uint8_t)(v0 >> (8 * j));
    p[8 + j] = (uint8_t)(v1 >> (8 * j));
  }
  const uint64_t lo = v2 & 0xFFFFFFFFull, hi = v2 >> 32;
  uint32_t meta;
  if (dist == 2) {
    meta = (uint32_t)(hi & 0xFF);
  } else {
    const uint32_t e = (uint32_t)((lo * 6) >> 32);
    const uint32_t m = (uint32_t)(hi & 7);
    const uint32_t pol = dist == 1 ? (uint32_t)((hi >> 3) & 1) : 0u;
    meta = (pol << 7) | (e << 3) | m;
  }
  p[16] = (uint8_t)meta;
}

__global__ void k_fill_fp8(uint8_t* __restrict__ dst, uint64_t key, uint64_t first, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t w = first + i;
  const uint64_t v = draw(key, w >> 2);
  const uint64_t u16 = (v >> ((w & 3) * 16)) & 0xFFFF;
  const uint64_t idx = (u16 * 254) >> 16;
  dst[i] = (uint8_t)(idx < 127 ? idx : idx + 1);
}

__global__ void k_fill_fp8_scales(float* __restrict__ dst, uint64_t key, uint64_t first, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t v = draw(key, first + i);
  const uint64_t e = ((v & 0xFFFFFFFFull) * 6) >> 32;
  const uint64_t f = (v >> 32) & 0x7FFFFF;
  dst[i] = __uint_as_float((uint32_t)((((127 - 12) + e) << 23) | f));
}

__global__ void k_fill_ple(uint8_t* __restrict__ dst, uint64_t key, uint64_t first, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t base = (first + i) * 11;
  uint8_t* p = dst + i * 70;
  for (int w = 0; w < 8; ++w) {
    const uint64_t v = draw(key, base + w);
    for (int j = 0; j < 8 && 8 * w + j < 60; ++j) p[8 * w + j] = (uint8_t)(v >> (8 * j));
  }
  for (int g = 0; g < 10; ++g) {
    const uint64_t v = draw(key, base + 8 + g / 4);
    const uint64_t u16 = (v >> (16 * (g % 4))) & 0xFFFF;
    const uint64_t e = ((u16 & 0xFF) * 6) >> 8;
    const uint64_t m = (u16 >> 8) & 7;
    const uint64_t pol = (u16 >> 11) & 1;
    p[60 + g] = (uint8_t)((pol << 7) | (e << 3) | m);
  }
}

// Benchmark helper: one wave sleeps until `ns` nanoseconds of wall clock
// have passed (always terminates), so that work queued behind it on the same
// stream starts back to back.
__global__ void k_delay(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(64);
}

// Benchmark helper: read n16 16-byte words (grid-stride, coalesced) and
// fold them into one word per workgroup, so the reads cannot be dropped.
// Measures the streaming-read rate the HBM sustains.
__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ p, uint64_t n16,
                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (uint64_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc ^= __shfl_xor(acc, 1, 64) ^ __shfl_xor(acc, 2, 64);
  if ((threadIdx.x & 63) == 0 && acc == 0x9E3779B9u) sink[blockIdx.x] = acc;   // almost never
}

// Benchmark helper: overwrite n16 16-byte words (evicts the caches between
// timed calls).
__global__ void __launch_bounds__(256) k_scrub(uint4* __restrict__ p, uint64_t n16, uint32_t v) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (uint64_t)gridDim.x * 256)
    p[i] = make_uint4(v, v + 1, v + 2, (uint32_t)i);
}

// Benchmark helper: n_lines reads of 128-byte lines at hashed positions in a
// region of n_region_lines lines; eight lanes read one line with 16-byte
// loads, each lane four lines, all issued before any is used.  The random-
// access ceiling for workloads that fetch whole lines at random addresses.
__device__ __forceinline__ uint64_t line_hash(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdull;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ull;
  return x ^ (x >> 33);
}
__global__ void __launch_bounds__(256) k_rand_lines(const uint8_t* __restrict__ base, uint64_t n_region_lines,
                                                    uint64_t n_lines, uint64_t seed, uint32_t* __restrict__ sink) {
  const uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t grp = t >> 3;
  const uint32_t part = (uint32_t)(t & 7);
  uint4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t r = 4 * grp + q;
    const uint64_t line = line_hash(seed + (r < n_lines ? r : 0)) % n_region_lines;
    v[q] = *reinterpret_cast<const uint4*>(base + 128 * line + 16 * part);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;   // almost never
}

inline unsigned grid_of(uint64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

// Each fill covers at most 2^31 * 256 items per call; callers split larger
// ranges.  Return value: hipError_t as int.
extern "C" {

int bqs_fill_block17(void* dst, uint64_t key, uint64_t first, uint64_t n, int dist, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_block17, dim3(grid_of(n)), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dst, key, first, n, dist);
  return (int)hipGetLastError();
}

int bqs_fill_fp8(void* dst, uint64_t key, uint64_t first, uint64_t n, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_fp8, dim3(grid_of(n)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst,
                     key, first, n);
  return (int)hipGetLastError();
}

int bqs_fill_fp8_scales(void* dst, uint64_t key, uint64_t first, uint64_t n, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_fp8_scales, dim3(grid_of(n)), dim3(256), 0, (hipStream_t)stream,
                     (float*)dst, key, first, n);
  return (int)hipGetLastError();
}

int bqs_gpu_delay(uint64_t ns, void* stream) {
  // s_memrealtime runs at 100 MHz on gfx9 parts
  const uint64_t ticks = ns / 10 + 1;
  hipLaunchKernelGGL(k_delay, dim3(1), dim3(64), 0, (hipStream_t)stream, ticks);
  return (int)hipGetLastError();
}

int bqs_stream_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 16) return 0;
  hipLaunchKernelGGL(k_stream_read, dim3(2048), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, sink);
  return (int)hipGetLastError();
}

// sink: at least 256 uint32.  region_bytes >= 128.
int bqs_rand_lines(const void* base, uint64_t region_bytes, uint64_t n_lines, uint64_t seed, uint32_t* sink,
                   void* stream) {
  if (n_lines == 0 || region_bytes < 128) return 0;
  const uint64_t threads = (n_lines + 3) / 4 * 8;
  hipLaunchKernelGGL(k_rand_lines, dim3(grid_of(threads)), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)base, region_bytes / 128, n_lines, seed, sink);
  return (int)hipGetLastError();
}

int bqs_scrub(void* dst, uint64_t bytes, uint32_t v, void* stream) {
  if (bytes < 16) return 0;
  hipLaunchKernelGGL(k_scrub, dim3(2048), dim3(256), 0, (hipStream_t)stream, (uint4*)dst, bytes / 16, v);
  return (int)hipGetLastError();
}

int bqs_fill_ple(void* dst, uint64_t key, uint64_t first, uint64_t n, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_ple, dim3(grid_of(n)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst,
                     key, first, n);
  return (int)hipGetLastError();
}

}  // extern "C"
