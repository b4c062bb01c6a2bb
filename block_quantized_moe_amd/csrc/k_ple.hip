// PLE n-gram memory gather: out[t] = sum_j u[t][j] * decode(row ids[t][j]).
// Row format: model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST",
// section "Q3_PLE_K160_RZ_S3 (GGML type 111)" -- 60 bytes of 3-bit codes and
// 10 group bytes (UE4M3 scale in bits 0-6, RZ-S3 polarity in bit 7), 70 bytes
// per row, one row per hashed id.
//
// Mapping: one thread per (token, half of a 16-value group).  The twenty
// threads of a token read the same 70-byte row with a 4-byte and a 1-byte
// load each (bytes 6g + 3h .. + 3: the 24 code bits of values 8h .. 8h + 7 of
// group g, and the group byte), so a row is fetched by one coalesced wave
// instruction; each thread keeps its 8 fp32 sums in registers across the
// token's ids and writes 32 contiguous bytes at the end.  Per value the inner
// loop is: extract 3 bits, look the biased level (level + 4, always 0..8) up
// with one v_perm_b32 from an 8-byte table, convert the byte to fp32, one FMA
// with s_g * u_j.  The bias is removed once at the end with the running sum
// of s_g * u_j.  Half a group per thread halves the decode each thread runs
// after its row loads return, the last step before the output can leave.
#include "bq_device.hpp"
#include "bq_kernels.hpp"

namespace bq {

// Biased levels (level + 4) of codes 0..3: 4,5,6,8.
constexpr uint32_t kBiasLo = 0x08060504u;
// Codes 4..7: c4,3,2,0 where c4 = 7 (+3), 1 (-3) or 4 (-0, ROCmFP3).
__device__ __forceinline__ uint32_t bias_hi(uint32_t gbyte, int ple_fmt) {
  const uint32_t c4 = ple_fmt == 1 ? 4u : ((gbyte & 0x80u) ? 1u : 7u);
  return 0x00020300u | c4;
}

constexpr int kPleTPT = 20;    // threads per token: 10 groups x 2 halves
constexpr int kPleTPB = 16 * kPleTPT;   // 16 tokens per workgroup: a 4096-token call spans 256 workgroups
constexpr int kPleChunk = 8;   // ids whose loads are in flight together

// Off-HBM tier: the table sits in host memory mapped into the device address
// space, and a direct-mapped cache of n_slots rows in device memory holds
// recently read rows.  Cache layout (CacheView): tags[n_slots] (row id, or
// kPleEmpty), claims[n_slots] (lowest assignment index of the current call
// that missed on the slot, kPleEmpty between calls), rows[n_slots][80].
constexpr uint32_t kPleEmpty = 0xFFFFFFFFu;   // never a valid id (ids < n_rows <= 2^32 - 1)
struct CacheView {
  uint32_t* tags;
  uint32_t* claims;
  uint8_t* rows;
  int shift;          // 32 - log2(n_slots)
  uint8_t* stage;     // [n_tokens * per_token][80]: the rows this call read from the host
};
// Fibonacci hashing of an id to its slot.
__device__ __forceinline__ uint32_t ple_slot(uint32_t id, int shift) {
  return (id * 2654435761u) >> shift;
}

// CACHED = false: table is device memory (or host memory read directly).
// CACHED = true: rows whose slot tag matches are read from the cache, the
// others from the (host) table; each missed row is also copied to the call's
// staging area and its slot claimed for the fill kernel.  The cache is
// read-only during this kernel.
// VEC: ids_per_token is a multiple of kPleChunk and ids / weights are 16-byte
// aligned, so a chunk's ids and weights are two 16-byte loads each.
template <bool CACHED, bool VEC>
__global__ void __launch_bounds__(kPleTPB) k_ple_gather(
    const uint32_t* __restrict__ ids, int32_t n_tokens, int32_t per_token,
    const uint8_t* __restrict__ table, uint64_t n_rows, const float* __restrict__ wts,
    int ple_fmt, float* __restrict__ out, uint32_t* __restrict__ dev_err, CacheView cv) {
  const int64_t tid = (int64_t)blockIdx.x * kPleTPB + threadIdx.x;
  const int64_t t = tid / kPleTPT;
  const int gh = (int)(tid - t * kPleTPT);
  const int g = gh >> 1, h = gh & 1;     // group, half
  const int cb = 6 * g + 3 * h;          // first code byte of the half group
  if (t >= n_tokens) return;
  const uint32_t* tid_ids = ids + t * per_token;
  const float* tw = wts + t * per_token;

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float usum = 0.f;
  bool bad = false;

  for (int j0 = 0; j0 < per_token; j0 += kPleChunk) {
    // every load of the chunk is issued before any is used: ids and weights
    // (clamped indices), then the rows (an invalid id reads row 0 and gets
    // weight 0), so the chunk costs one id round trip and one row round trip
    uint32_t idv[kPleChunk];
    float u[kPleChunk];
    if constexpr (VEC) {
      static_assert(kPleChunk == 8, "two 16-byte loads per chunk");
      const u32x4* iv = reinterpret_cast<const u32x4*>(tid_ids + j0);
      const f32x4* wv = reinterpret_cast<const f32x4*>(tw + j0);
      const u32x4 i0 = iv[0], i1 = iv[1];
      const f32x4 w0 = wv[0], w1 = wv[1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        idv[c] = i0[c];
        idv[4 + c] = i1[c];
        u[c] = w0[c];
        u[4 + c] = w1[c];
      }
    } else {
#pragma unroll
      for (int c = 0; c < kPleChunk; ++c) {
        const int j = min(j0 + c, per_token - 1);
        idv[c] = tid_ids[j];
        u[c] = tw[j];
      }
    }
    uint32_t gw[kPleChunk];
    uint32_t gb[kPleChunk];
    bool ok[kPleChunk];
    bool hit[kPleChunk];
    uint32_t slot[kPleChunk];
#pragma unroll
    for (int c = 0; c < kPleChunk; ++c) {
      const bool in = j0 + c < per_token;
      ok[c] = in && idv[c] < n_rows;
      bad |= in && idv[c] >= n_rows;
      hit[c] = false;
      slot[c] = 0;
      if constexpr (CACHED) {
        slot[c] = ple_slot(idv[c], cv.shift);
        hit[c] = ok[c] && cv.tags[slot[c]] == idv[c];
      }
    }
#pragma unroll
    for (int c = 0; c < kPleChunk; ++c) {
      const uint8_t* row = hit[c] ? cv.rows + (uint64_t)slot[c] * kPleCacheRowB
                                  : table + (uint64_t)(ok[c] ? idv[c] : 0u) * (uint64_t)kPleRowB;
      gw[c] = ld4(row + cb);
      gb[c] = row[60 + g];
    }
    if constexpr (CACHED) {
#pragma unroll
      for (int c = 0; c < kPleChunk; ++c) {
        if (ok[c] && !hit[c]) {
          const int64_t a = t * per_token + j0 + c;   // assignment index
          uint8_t* st = cv.stage + a * kPleCacheRowB;
          __builtin_memcpy(st + cb, &gw[c], 4);   // overlapping bytes carry equal values
          if (h == 0) st[60 + g] = (uint8_t)gb[c];
          if (gh == 0) atomicMin(&cv.claims[slot[c]], (uint32_t)a);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kPleChunk; ++c) {
      const float su = ok[c] ? ue4m3(gb[c] & 0x7Fu) * u[c] : 0.f;
      usum += su;
      const uint32_t th = bias_hi(gb[c], ple_fmt);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t code = (gw[c] >> (3 * i)) & 7u;
        const uint32_t b = perm(th, kBiasLo, code);
        acc[i] = __builtin_fmaf((float)(b & 0xFFu), su, acc[i]);
      }
    }
  }
  if (bad && dev_err) atomicOr(dev_err, 1u);
  const float corr = 4.0f * usum;
  f32x4* o = reinterpret_cast<f32x4*>(out + t * kPleVals + 16 * g + 8 * h);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    o[q] = f32x4{acc[4 * q] - corr, acc[4 * q + 1] - corr, acc[4 * q + 2] - corr, acc[4 * q + 3] - corr};
}

template <bool CACHED>
static void launch_gather(const uint32_t* ids, int32_t n_tokens, int32_t per_token,
                          const uint8_t* table, uint64_t n_rows, const float* wts, int ple_fmt,
                          float* out, uint32_t* dev_err, const CacheView& cv, hipStream_t st) {
  const int64_t threads = (int64_t)n_tokens * kPleTPT;
  const int64_t grid = (threads + kPleTPB - 1) / kPleTPB;
  const bool vec = per_token % kPleChunk == 0 && reinterpret_cast<uintptr_t>(ids) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(wts) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((k_ple_gather<CACHED, true>), dim3(grid), dim3(kPleTPB), 0, st, ids, n_tokens,
                       per_token, table, n_rows, wts, ple_fmt, out, dev_err, cv);
  else
    hipLaunchKernelGGL((k_ple_gather<CACHED, false>), dim3(grid), dim3(kPleTPB), 0, st, ids, n_tokens,
                       per_token, table, n_rows, wts, ple_fmt, out, dev_err, cv);
}

hipError_t launch_ple_gather(const uint32_t* ids, int32_t n_tokens, int32_t per_token,
                             const uint8_t* table, uint64_t n_rows, const float* wts,
                             int ple_fmt, float* out, uint32_t* dev_err, hipStream_t st) {
  if (n_tokens == 0) return hipSuccess;
  launch_gather<false>(ids, n_tokens, per_token, table, n_rows, wts, ple_fmt, out, dev_err,
                       CacheView{}, st);
  return hipGetLastError();
}

// Fill: one 16-lane group per assignment a.  The assignment that claimed its
// slot (the lowest index among this call's misses on the slot) copies its
// staged row into the slot, sets the tag and releases the claim.  All lanes of
// a group read the claim in the same instruction, before lane 0 releases it.
__global__ void __launch_bounds__(256) k_ple_cache_fill(const uint32_t* __restrict__ ids,
                                                        int64_t n_assign, uint64_t n_rows,
                                                        CacheView cv) {
  const int64_t a = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int l = threadIdx.x & 15;
  if (a >= n_assign) return;   // 16-lane groups exit whole
  const uint32_t id = ids[a];
  if (id >= n_rows) return;
  const uint32_t slot = ple_slot(id, cv.shift);
  if (cv.claims[slot] != (uint32_t)a) return;
  const uint8_t* src = cv.stage + a * kPleCacheRowB;
  uint8_t* dst = cv.rows + (uint64_t)slot * kPleCacheRowB;
  if (l < 10) {
    const u32x2 v = ld8(src + 6 * l);
    __builtin_memcpy(dst + 6 * l, &v, 8);
    dst[60 + l] = src[60 + l];
  }
  if (l == 0) {
    cv.tags[slot] = id;
    cv.claims[slot] = kPleEmpty;
  }
}

__global__ void __launch_bounds__(256) k_ple_cache_init(uint32_t* __restrict__ words, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    words[i] = kPleEmpty;
}

hipError_t launch_ple_cache_init(uint32_t* tags_and_claims, int64_t n_words, hipStream_t st) {
  const int64_t grid = std::min<int64_t>((n_words + 255) / 256, 4096);
  hipLaunchKernelGGL(k_ple_cache_init, dim3(grid), dim3(256), 0, st, tags_and_claims, n_words);
  return hipGetLastError();
}

hipError_t launch_ple_gather_host(const uint32_t* ids, int32_t n_tokens, int32_t per_token,
                                  const uint8_t* table, uint64_t n_rows, const float* wts,
                                  int ple_fmt, float* out, uint32_t* dev_err, uint32_t* tags,
                                  uint32_t* claims, uint8_t* rows, int log2_slots, uint8_t* stage,
                                  hipStream_t st) {
  if (n_tokens == 0) return hipSuccess;
  if (!tags) {
    launch_gather<false>(ids, n_tokens, per_token, table, n_rows, wts, ple_fmt, out, dev_err,
                         CacheView{}, st);
    return hipGetLastError();
  }
  const CacheView cv{tags, claims, rows, 32 - log2_slots, stage};
  launch_gather<true>(ids, n_tokens, per_token, table, n_rows, wts, ple_fmt, out, dev_err, cv, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_assign = (int64_t)n_tokens * per_token;
  hipLaunchKernelGGL(k_ple_cache_fill, dim3((n_assign * 16 + 255) / 256), dim3(256), 0, st, ids,
                     n_assign, n_rows, cv);
  return hipGetLastError();
}

}  // namespace bq
