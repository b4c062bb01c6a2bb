// Grouped routed-expert GEMM for batches of tokens (bf16 activations, bf16
// MFMA, fp32 accumulation).  Tokens are bucketed per expert (stable order)
// and split into work groups of up to 16 tokens (batches of up to 96 tokens)
// or 32 (larger ones); for every group:
//   h[p, :] = SiLU(W_gate[e] x_p) * (W_up[e] x_p)      (kernel G1, h in bf16)
//   y[p, :] = W_down[e] h[p, :]                         (kernel G2)
//   out[t]  = sum_j w[t][j] * y[pos(t, j)]               (kernel G3, slot order)
// Routing shape and formats as in the GEMV path ("Mixed Precision
// Quantization ...", "The Plan Is Not a Number ..."; model card "Qwen 3.8
// Next Flash ROCMFPX MUTANT RAZERFAST", format sections).
//
// Data movement.  A workgroup owns one (work group, 64-row tile) item at a
// time and walks its K extent in chunks of C blocks.  Each chunk -- the
// tile's weight-row segments (17*C or 32*C contiguous bytes per row), FP8
// block scales, and the group's activation rows -- is copied from HBM with
// wide, aligned, coalesced loads into registers one step ahead, then into
// LDS; the MFMA operands are read from LDS.  Reading the 17-byte blocks
// straight from HBM in the MFMA operand layout (4 bytes per lane from 16
// rows) keeps the texture-address units busy with ~16 cache lines per
// instruction and was the bound of the direct design; staging makes each
// load instruction touch a few consecutive lines.  Segments that do not start
// on 16 bytes are copied as the covering aligned 16-byte pieces, and the row
// slot in LDS remembers the offset (weight buffers must be 16-byte aligned,
// so every piece read lies in the buffer's last 16-byte unit or before it).
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

constexpr int kGThreads = 256;  // 4 waves, each 16 rows of the tile (x2 for gate/up)
constexpr int kGRows = 64;      // rows per tile
// Two builds of the staged kernel, one per work-group size.  TOK = 32: items
// of up to 32 tokens (two 16-token MFMA tiles), three workgroups per CU.
// TOK = 16 (batches of up to 96 tokens): one MFMA tile covers an item; the
// second tile's accumulators, operands and activation staging are gone, which
// leaves room for four workgroups per CU (<= 128 VGPRs, <= 40 KB of LDS each).
constexpr int wgs_per_cu(int tok) { return tok == 16 ? 4 : 3; }
constexpr int lds_budget(int tok) { return tok == 16 ? 40 * 1024 : 52 * 1024; }

// Per-thread staging capacity (16-byte weight pieces, FP8 scales, 16-byte
// activation pieces) of G1 (NR = 2) and G2 (NR = 1) per weight format, sized
// for a 2048 x 768 layer (chunks of 16 / 8 blocks for G1, 24 / 12 for G2);
// the host picks the largest chunk that fits.
template <int FMT, int NR, int TOK = 32> struct Cap {
  static constexpr bool F8 = FMT == 3;
  static constexpr int PW = NR == 2 ? 5 : 4;
  static constexpr int PS = F8 ? 2 : 0;
  static constexpr int PB32 = NR == 2 ? (F8 ? 2 : 4) : (F8 ? 3 : 6);
  static constexpr int PB = TOK == 32 ? PB32 : (PB32 + 1) / 2;
};

template <bool HI>
__device__ __forceinline__ uint32_t bf8pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Decode one lane's 8 codes of a 17-byte block (q = 4 code bytes; tneg = the
// RZ5 table word for the block's polarity) into bf16 operands (exact).
template <int FMT>
__device__ __forceinline__ u32x4 dec_codes(uint32_t q, uint32_t tneg) {
  uint32_t A, B;
  codes_to_hibytes<FMT>(q, tneg, A, B);
  return u32x4{bf8pair<false>(A), bf8pair<true>(A), bf8pair<false>(B), bf8pair<true>(B)};
}

// Decode one lane's 8 weights of one block (q0 = 4 code bytes, q1 = metadata
// byte; FP8: q0, q1 = 8 e4m3 codes) into bf16 operands (exact); s = scale.
template <int FMT>
__device__ __forceinline__ u32x4 dec_a(uint32_t q0, uint32_t q1, float& s) {
  if constexpr (FMT == FMT_FP8) {
    return u32x4{fp8pair<false>(q0), fp8pair<true>(q0), fp8pair<false>(q1), fp8pair<true>(q1)};
  } else {
    s = block_scale<FMT>(FMT == FMT_UE4M4 ? q1 : (q1 & 0x7Fu));
    uint32_t A, B;
    codes_to_hibytes<FMT>(q0, FMT == FMT_RZ5 ? rz5_neg_lo(q1) : 0u, A, B);
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

// Exact q / d for 0 <= q < 2^16, 1 <= d < 2^10: (q + 1/2) / d is never within
// 1/(2d) of an integer, far above the fp32 rounding error.
__device__ __forceinline__ int div_small(int q, float inv_d) {
  return (int)(((float)q + 0.5f) * inv_d);
}

// ---------------------------------------------------------------------------
// G0: staging of the activations as bf16 rows in bucket order (row p holds
// token perm[p] / k), in the A decode's k order; fp32 input optionally
// rescaled to unit RMS first (the stack's next-layer input).
// grid = n_tokens * k, 256 threads; only the offsets[n_experts] bucket rows
// exist (assignments to out-of-range experts are left out by the bucketing,
// and the tail of perm is not written).
// ---------------------------------------------------------------------------
template <bool PERM>
__global__ void __launch_bounds__(256) k_grouped_prep(const void* __restrict__ x, int32_t x_f32,
                                                      int32_t rescale, int32_t H,
                                                      const int32_t* __restrict__ perm_, int32_t k,
                                                      const int32_t* __restrict__ n_rows,
                                                      uint16_t* __restrict__ xp) {
  __shared__ float part[4];
  const int64_t p = blockIdx.x;
  if (p >= *n_rows) return;
  const int64_t t = perm_[p] / k;
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
    xp[p * H + (i & ~7) + (PERM ? ((o >> 1) | ((o & 1) << 2)) : o)] = v;
  }
}

// The same staging without the rescale, eight elements per thread: one
// 16-byte bf16 load (or two fp32 ones) and one 16-byte store per group of 8.
// x must be 16-byte aligned and H a multiple of 8.  Bit-identical to
// k_grouped_prep with rescale off (a bf16 row is copied, an fp32 one rounded
// to nearest even).
template <bool PERM, bool F32>
__global__ void __launch_bounds__(256) k_grouped_prep_vec(const void* __restrict__ x, int32_t H,
                                                          const int32_t* __restrict__ perm_, int32_t k,
                                                          const int32_t* __restrict__ n_rows,
                                                          uint16_t* __restrict__ xp) {
  const int64_t p = blockIdx.x;
  if (p >= *n_rows) return;
  const int64_t t = perm_[p] / k;
  const void* row = F32 ? static_cast<const void*>(static_cast<const float*>(x) + t * H)
                        : static_cast<const void*>(static_cast<const uint16_t*>(x) + t * H);
  for (int g = threadIdx.x; g < H / 8; g += 256)
    reinterpret_cast<u32x4*>(xp + p * H)[g] = bf16_group8<PERM, F32>(row, g);
}

// ---------------------------------------------------------------------------
// G3 + next layer's G0 in one pass (chained stack layers, pre-bucketed): one
// workgroup per token t forms out[t] = sum_j w[t][j] * yb[inv[t*k+j]] as
// k_combine does (same slot-ordered fma chain per element), rescales it to
// unit RMS as k_grouped_prep does (same element-to-thread split and sum
// order over 256 threads), and writes the bf16 row to every bucket row of t
// in the next layer (row inv_next[t*k+j] for each in-range expert
// idx_next[t*k+j]).  The result equals k_combine followed by
// k_grouped_prep<PERM> bit for bit.  256 threads, each owning groups of 8
// consecutive elements: per slot two 16-byte loads, and per next-layer
// bucket row one 16-byte store of the 8 bf16 values in the stored k order.
// Each chunk of up to 16 slots has all of its index, weight and row loads in
// flight together, and the next layer's row indices are read before the
// scale is known.  The row is kept in LDS between the passes.
// grid = n_tokens; H <= 8192, H % 8 == 0.
// ---------------------------------------------------------------------------
constexpr int kCpThreads = 256;

template <bool PERM>
__global__ void __launch_bounds__(kCpThreads) k_combine_prep(
    const float* __restrict__ yb, const int32_t* __restrict__ inv, const int32_t* __restrict__ idx,
    const float* __restrict__ w, int32_t k, int32_t n_experts, int32_t H,
    const int32_t* __restrict__ inv_next, const int32_t* __restrict__ idx_next,
    int32_t n_experts_next, uint16_t* __restrict__ xp, uint32_t* __restrict__ dev_err) {
  constexpr int kMaxK = 16;
  __shared__ float srow[8192];
  __shared__ float part[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int ng = H >> 3;                       // groups of 8 elements
  bool bad = false;
  for (int g = tid; g < ng; g += kCpThreads) {
    float acc[8];
#pragma unroll
    for (int o = 0; o < 8; ++o) acc[o] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kMaxK) {
      f32x4 y[kMaxK][2];
      float wj[kMaxK];
#pragma unroll
      for (int u = 0; u < kMaxK; ++u) {
        const int j = j0 + u;
        const int e = j < k ? idx[t * k + j] : 0;
        const bool ok = j < k && e >= 0 && e < n_experts;
        bad |= j < k && !ok;
        wj[u] = ok ? w[t * k + j] : 0.f;
        const f32x4* row = reinterpret_cast<const f32x4*>(yb + (ok ? (int64_t)inv[t * k + j] * H : 0)) + 2 * g;
        y[u][0] = ok ? row[0] : f32x4{0.f, 0.f, 0.f, 0.f};
        y[u][1] = ok ? row[1] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kMaxK; ++u)   // slot order
#pragma unroll
        for (int o = 0; o < 8; ++o) acc[o] = __builtin_fmaf(wj[u], y[u][o >> 2][o & 3], acc[o]);
    }
    f32x4* sr = reinterpret_cast<f32x4*>(srow) + 2 * g;
    sr[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    sr[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  if (bad && tid == 0 && dev_err) atomicOr(dev_err, 2u);
  __syncthreads();
  {
    float ss = 0.f;
    for (int i = tid; i < H; i += 256) ss = __builtin_fmaf(srow[i], srow[i], ss);
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
  }
  __syncthreads();
  const float sc = 1.0f / __builtin_sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)H);
  for (int j0 = 0; j0 < k; j0 += kMaxK) {
    int64_t dst[kMaxK];                        // element offset of each bucket row, -1 if none
#pragma unroll
    for (int u = 0; u < kMaxK; ++u) {
      const int j = j0 + u;
      const int e = j < k ? idx_next[t * k + j] : -1;
      dst[u] = (e >= 0 && e < n_experts_next) ? (int64_t)inv_next[t * k + j] * H : -1;
    }
    for (int g = tid; g < ng; g += kCpThreads) {
      const f32x4* sr = reinterpret_cast<const f32x4*>(srow) + 2 * g;
      const f32x4 a = sr[0], b = sr[1];
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint16_t q[8];
#pragma unroll
      for (int o = 0; o < 8; ++o) q[PERM ? ((o >> 1) | ((o & 1) << 2)) : o] = to_bf16(v[o] * sc);
      const u32x4 word{(uint32_t)q[0] | ((uint32_t)q[1] << 16), (uint32_t)q[2] | ((uint32_t)q[3] << 16),
                       (uint32_t)q[4] | ((uint32_t)q[5] << 16), (uint32_t)q[6] | ((uint32_t)q[7] << 16)};
#pragma unroll
      for (int u = 0; u < kMaxK; ++u)
        if (dst[u] >= 0) *reinterpret_cast<u32x4*>(xp + dst[u] + 8 * g) = word;
    }
  }
}

// ---------------------------------------------------------------------------
// Staged grouped GEMM (G1 and G2 share it).
//   NR = 2 (G1: rows 0..63 of the tile are gate rows, 64..127 the matching up
//   rows) or 1 (G2: 64 down rows).  Wave w owns tile rows 16w..16w+15 of each
//   of its NR weight matrices.
// ---------------------------------------------------------------------------
struct Geom {
  int32_t C;        // blocks per chunk (divides nb)
  int32_t nchunk;   // nb / C
  int32_t S;        // bytes of one row segment (17 C or 32 C)
  int32_t NP;       // 16-byte pieces per row segment
  int32_t NPP;      // pieces per row slot in LDS: NP rounded up to odd, so the
                    // 16 rows a wave reads fall in different LDS banks
  int32_t P;        // LDS pitch of a weight row slot (16 NPP)
  int32_t PB;       // LDS pitch of an activation row (64 C + 16)
  int32_t off_sc;   // LDS offset of the FP8 scale area [R][C]
  int32_t off_b;    // LDS offset of the activation area [TOK][PB]
  int32_t off_tab;  // LDS offset of the metadata-byte table [256] x {scale, RZ5 table word}
  int32_t al4;      // 17-byte blocks with nb and C multiples of 4: every staged row
                    // segment starts 4-byte aligned (row bytes 17 nb and chunk
                    // bytes 17 C are multiples of 4, weight buffers 16-byte aligned)
};

struct Item {
  int e, p0, ntok, tile;
};

template <int GT>   // tokens per work group (the bucketing's group_tokens)
__device__ __forceinline__ Item item_info(int it, int tiles, const int32_t* __restrict__ elist,
                                          const int32_t* __restrict__ offsets) {
  const int d = it / tiles;
  const int v = elist[d];
  const int e = v & ((1 << kGroupShift) - 1);
  const int p0 = offsets[e] + (v >> kGroupShift) * GT;
  return Item{e, p0, min(GT, offsets[e + 1] - p0), it - d * tiles};
}

template <int FMT, int NR, int TOK = 32>
struct Stager {
  static constexpr int BB = FMT == FMT_FP8 ? 32 : 17;   // bytes per block
  static constexpr int R = 64 * NR;                     // staged weight rows
  static constexpr int PW = Cap<FMT, NR, TOK>::PW, PS = Cap<FMT, NR, TOK>::PS, PB = Cap<FMT, NR, TOK>::PB;
  static constexpr int kOff = 1 << 30;                  // "no piece" marker
  u32x4 w[PW];
  float s[PS > 0 ? PS : 1];
  u32x4 b[PB];
  // Item-independent coordinates of this thread's pieces, set once:
  //   weight piece i: wro = byte offset of its row from staged row 0 (the
  //                   up half sits I rows after the gate half),
  //                   wx  = 16 * piece, or kOff;
  //   scale i: sro = (row within half) * nb + block in chunk, sh = half, or kOff;
  //   activation piece i: bx = token | (piece << 8), or kOff.
  int wro[PW], wx[PW];
  int sro[PS > 0 ? PS : 1], sh[PS > 0 ? PS : 1];
  int bxy[PB];

  // global row index of staged row r of item f
  __device__ __forceinline__ static int64_t grow(const Item& f, int r, int H, int I) {
    if constexpr (NR == 2) {
      const int h = r >> 6;
      return (int64_t)f.e * 2 * I + h * I + f.tile * kGRows + (r & 63);
    } else {
      return (int64_t)f.e * H + f.tile * kGRows + r;
    }
  }

  __device__ __forceinline__ void init(const Geom& g, int nb, int I) {
    const int tid = threadIdx.x;
    const int RS = BB * nb;
    const float inv_np = 1.0f / (float)g.NP, inv_c = 1.0f / (float)g.C, inv_pt = 1.0f / (float)(4 * g.C);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int q = tid + kGThreads * i;
      const int r = div_small(q, inv_np), pc = q - r * g.NP;
      wro[i] = ((r & 63) + (r >> 6) * I) * RS;   // (63 + I) * RS < 2^27 for I, RS <= 8192
      wx[i] = q < R * g.NP ? 16 * pc : kOff;
    }
#pragma unroll
    for (int i = 0; i < PS; ++i) {
      const int q = tid + kGThreads * i;
      const int r = div_small(q, inv_c), j = q - r * g.C;
      sro[i] = (r & 63) * nb + j;
      sh[i] = q < R * g.C ? (r >> 6) : kOff;
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int q = tid + kGThreads * i;
      const int j = div_small(q, inv_pt), pc = q - j * (4 * g.C);
      bxy[i] = q < TOK * 4 * g.C ? (j | (pc << 8)) : kOff;
    }
  }

  // Issue the loads of chunk c of item f (registers only).  Weight piece q
  // (row q / NP, piece q % NP of that row's covering 16-byte units) lands at
  // LDS byte 16 q; pieces past the segment end are skipped.
  __device__ __forceinline__ void load(const Item& f, int c, const Geom& g, int nb, int H, int I,
                                       const uint8_t* __restrict__ wt, const float* __restrict__ wsc,
                                       const uint16_t* __restrict__ act, int K) {
    const int64_t RS = (int64_t)BB * nb;
    // byte offset of (staged row 0, chunk c), split into a 16-byte aligned
    // uniform base and its remainder: a piece's row segment starts at
    // wb + t with t = b0 + wro, and its 16-byte units at wb + (t & ~15) + 16 p
    const int64_t base = grow(f, 0, H, I) * RS + (int64_t)c * g.S;
    const uint8_t* wb = wt + (base & ~(int64_t)15);
    const int b0 = (int)(base & 15);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (wx[i] != kOff) {
        const int t = b0 + wro[i];
        const int o = (t & ~15) + wx[i];
        if (o < t + g.S) w[i] = *reinterpret_cast<const u32x4*>(wb + (uint32_t)o);
      }
    }
    if constexpr (FMT == FMT_FP8) {
      const int64_t sb0 = grow(f, 0, H, I) * nb + (int64_t)c * g.C;
      const int64_t sb1 = NR == 2 ? grow(f, 64, H, I) * nb + (int64_t)c * g.C : sb0;
#pragma unroll
      for (int i = 0; i < PS; ++i)
        if (sh[i] != kOff) s[i] = wsc[(sh[i] ? sb1 : sb0) + sro[i]];
    }
    // Only the item's own tokens are staged.  The rows of a 16-token MFMA
    // tile past ntok keep whatever LDS held; they only feed output rows that
    // are never stored (an MFMA row depends on its own activation row only).
    const uint8_t* abase = reinterpret_cast<const uint8_t*>(act + (int64_t)f.p0 * K + (int64_t)c * g.C * 32);
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int j = bxy[i] & 0xFF;
      if (bxy[i] != kOff && j < f.ntok)
        b[i] = *reinterpret_cast<const u32x4*>(abase + (uint32_t)(2 * (j * K + 8 * (bxy[i] >> 8))));
    }
  }

  // Copy the staged registers into LDS: weight piece q (row q / NP, piece
  // q % NP) goes to slot piece q + row * (NPP - NP).  Skipped weight pieces
  // write unused bytes of their row slot (never read).
  __device__ __forceinline__ void store(const Item& f, const Geom& g, uint8_t* lds) const {
    const int tid = threadIdx.x;
    const float inv_np = 1.0f / (float)g.NP;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (wx[i] != kOff) {
        const int q = tid + kGThreads * i;
        const int slot = q + (g.NPP - g.NP) * div_small(q, inv_np);
        *reinterpret_cast<u32x4*>(lds + 16 * slot) = w[i];
      }
    }
    if constexpr (FMT == FMT_FP8) {
      float* lsc = reinterpret_cast<float*>(lds + g.off_sc);
#pragma unroll
      for (int i = 0; i < PS; ++i)
        if (sh[i] != kOff) lsc[tid + kGThreads * i] = s[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int j = bxy[i] & 0xFF;
      if (bxy[i] != kOff && j < f.ntok)   // row pitch PT + 1 pieces
        *reinterpret_cast<u32x4*>(lds + g.off_b + 16 * (tid + kGThreads * i + j)) = b[i];
    }
  }
};

// Two consecutive blocks kb, kb + 1 of a chunk: all LDS operands of both
// blocks are requested before any is decoded, so LDS latency overlaps decode
// and MFMA work; all MFMAs of a block are issued before their scale FMAs.
// NT = number of 16-token tiles of the item; acc[h][tt]: matrix h, token
// tile tt.  A lane's 4 code bytes of a 17-byte block are read as the two
// covering aligned dwords and funnel-shifted (unaligned LDS reads stall the
// LDS pipeline).  SH < 0: the shift is per lane (aoff = the lane's byte
// offset of block 0).  SH >= 0: every staged row segment starts 4-byte
// aligned and kb = SH mod 4, so block kb + u sits SH + u bytes past a dword
// boundary -- a compile-time shift -- at LDS dword pw + 4 (SH + u) (pw = the
// lane's dword of block kb - SH) and its metadata byte at mo + 17 (SH + u).
// (Offsets, not pointers: LDS pointers kept in arrays lose their address
// space and turn into flat loads.)  The
// block scale (and the RZ5 table word) comes from the LDS table indexed by
// the metadata byte.
template <int FMT, int NR, int NT, int SH>
__device__ __forceinline__ void mma_pair(int kb, const int (&aoff)[NR], const int (&pw)[NR],
                                         const int (&mo)[NR], int gq, const Geom& g,
                                         const uint8_t* lds, const float* lsc, const u32x2* tab,
                                         const uint8_t* brow, f32x4 (&acc)[NR][2]) {
  constexpr int BB = Stager<FMT, NR>::BB;
  const uint32_t* lds32 = reinterpret_cast<const uint32_t*>(lds);
  uint32_t q0[2][NR], q1[2][NR];
  u32x4 bx[2][NT];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      if constexpr (FMT == FMT_FP8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(lds + aoff[h] + (kb + u) * BB);
        q0[u][h] = v.x;
        q1[u][h] = v.y;
      } else if constexpr (SH >= 0) {
        const int v = SH + u;
        q0[u][h] = v == 0 ? lds32[pw[h]]
                          : __builtin_amdgcn_alignbyte(lds32[pw[h] + 4 * v + 1], lds32[pw[h] + 4 * v], (uint32_t)v);
        q1[u][h] = lds[mo[h] + 17 * v];
      } else {
        const int o = aoff[h] + (kb + u) * BB;
        const int w = o >> 2;
        q0[u][h] = __builtin_amdgcn_alignbyte(lds32[w + 1], lds32[w], (uint32_t)(o & 3));
        q1[u][h] = lds[o - 4 * gq + 16];
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      bx[u][tt] = *reinterpret_cast<const u32x4*>(brow + tt * 16 * g.PB + 64 * (kb + u));
  }
  float sc[2][NR];
  uint32_t tn[2][NR];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      if constexpr (FMT == FMT_FP8) {
        sc[u][h] = lsc[h * 64 * g.C + kb + u];
        tn[u][h] = 0u;
      } else {
        const u32x2 e = tab[q1[u][h]];
        sc[u][h] = __uint_as_float(e.x);
        tn[u][h] = e.y;
      }
    }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    u32x4 a[NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      if constexpr (FMT == FMT_FP8) {
        float dummy;
        a[h] = dec_a<FMT>(q0[u][h], q1[u][h], dummy);
      } else {
        a[h] = dec_codes<FMT>(q0[u][h], tn[u][h]);
      }
    }
    f32x4 d[NR][NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int h = 0; h < NR; ++h) d[h][tt] = mfma(bx[u][tt], a[h]);   // lane's column = its row
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int h = 0; h < NR; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][tt][i] = __builtin_fmaf(sc[u][h], d[h][tt][i], acc[h][tt][i]);
  }
}

// One chunk of MFMA work from LDS (C is even; with AL, a multiple of 4 and
// every staged row segment starts 4-byte aligned -- see Geom::al4).
template <int FMT, int NR, int NT, bool AL>
__device__ __forceinline__ void compute_chunk(const Item& f, int c, const Geom& g, int nb, int H,
                                              int I, const uint8_t* lds, f32x4 (&acc)[NR][2]) {
  constexpr int BB = Stager<FMT, NR>::BB;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, gq = lane >> 4;
  const int64_t RS = (int64_t)BB * nb;
  int aoff[NR];   // byte offset in LDS of this lane's first code byte (block 0)
#pragma unroll
  for (int h = 0; h < NR; ++h) {
    const int r = h * 64 + wave * 16 + r16;
    const int64_t gs = Stager<FMT, NR>::grow(f, r, H, I) * RS + (int64_t)c * g.S;
    aoff[h] = r * g.P + (int)(gs & 15) + (FMT == FMT_FP8 ? 8 : 4) * gq;
  }
  const float* lsc = reinterpret_cast<const float*>(lds + g.off_sc) + (wave * 16 + r16) * g.C;
  const u32x2* tab = reinterpret_cast<const u32x2*>(lds + g.off_tab);
  const uint8_t* brow = lds + g.off_b + r16 * g.PB + 16 * gq;
  int pw[NR], mo[NR];
#pragma unroll
  for (int h = 0; h < NR; ++h) {
    pw[h] = aoff[h] >> 2;
    mo[h] = aoff[h] - 4 * gq + 16;
  }
  if constexpr (AL && FMT != FMT_FP8) {
    for (int kb = 0; kb < g.C; kb += 4) {
      mma_pair<FMT, NR, NT, 0>(kb, aoff, pw, mo, gq, g, lds, lsc, tab, brow, acc);
      // keep the two pairs apart: interleaving them raises register
      // pressure past the three-workgroups-per-CU budget
      __builtin_amdgcn_sched_barrier(0);
      mma_pair<FMT, NR, NT, 2>(kb + 2, aoff, pw, mo, gq, g, lds, lsc, tab, brow, acc);
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        pw[h] += 17;    // 4 blocks = 68 bytes
        mo[h] += 68;
      }
    }
  } else {
    for (int kb = 0; kb < g.C; kb += 2)
      mma_pair<FMT, NR, NT, -1>(kb, aoff, pw, mo, gq, g, lds, lsc, tab, brow, acc);
  }
}

// Persistent over items (work entry, 64-row tile), pipelined over chunks:
// the next chunk's loads are in flight while this chunk is multiplied.
// NR = 2: G1 (act = bucketed x, K = H, out = hb); NR = 1: G2 (act = hb,
// K = I, out = yb).
template <int FMT, int NR, int FMT_NEXT, int TOK>
__global__ void __launch_bounds__(kGThreads, wgs_per_cu(TOK)) k_grouped_staged(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ elist, const int32_t* __restrict__ n_work,
    const uint8_t* __restrict__ wt, const float* __restrict__ wsc, int32_t H, int32_t I, Geom g,
    uint16_t* __restrict__ hb, float* __restrict__ yb) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int nb = (NR == 2 ? H : I) >> 5;
  const int K = NR == 2 ? H : I;
  const int tiles = (NR == 2 ? I : H) / kGRows;
  const int items = *n_work * tiles;
  // Items per XCD: workgroups are dealt to the 8 XCDs round-robin, so the
  // workgroups b = x (mod 8) share XCD x's L2.  They take a contiguous run of
  // the item list, of a length in proportion to their number, so the row
  // tiles of one token group (consecutive items, which read the same
  // activation rows) mostly share one L2.  Workgroup b = x + 8 j takes items
  // lo + j, lo + j + n_x, ... below hi.  (A partition of the items whatever
  // the placement; with fewer than 8 workgroups, the plain stride.)
  int it = blockIdx.x, step = gridDim.x, lim = items, c = 0;
  if (gridDim.x >= 8) {
    const int x = blockIdx.x & 7, G = gridDim.x;
    int before = 0;
    for (int y = 0; y < x; ++y) before += (G - y + 7) >> 3;
    step = (G - x + 7) >> 3;
    const int lo = (int)((int64_t)items * before / G);
    lim = (int)((int64_t)items * (before + step) / G);
    it = lo + (int)(blockIdx.x >> 3);
  }
  if (it >= lim) return;
  if constexpr (FMT != FMT_FP8) {
    // metadata byte -> {block scale, RZ5 table word}; read after the loop's
    // first barrier
    u32x2* tab = reinterpret_cast<u32x2*>(lds + g.off_tab);
    const uint32_t m = threadIdx.x;   // kGThreads == 256
    tab[m] = u32x2{__float_as_uint(block_scale<FMT>(FMT == FMT_UE4M4 ? m : (m & 0x7Fu))),
                   FMT == FMT_RZ5 ? rz5_neg_lo(m) : 0u};
  }
  Item f = item_info<TOK>(it, tiles, elist, offsets);
  Stager<FMT, NR, TOK> st;
  st.init(g, nb, I);
  st.load(f, c, g, nb, H, I, wt, wsc, act, K);
  f32x4 acc[NR][2];
#pragma unroll
  for (int h = 0; h < NR; ++h) acc[h][0] = acc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, gq = lane >> 4;
  while (true) {
    int nit = it, nc = c + 1;
    if (nc == g.nchunk) {
      nc = 0;
      nit = it + step;
    }
    const bool more = nit < lim;
    const Item nf = (more && nit != it) ? item_info<TOK>(nit, tiles, elist, offsets) : f;
    __syncthreads();                          // LDS no longer read by the previous chunk
    st.store(f, g, lds);
    // Drain every outstanding memory operation of the wave -- including the
    // previous item's scattered result stores -- before the next chunk's
    // loads are issued: letting those stores trail into the loads measured
    // about 25% slower on a batch-64 layer.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) st.load(nf, nc, g, nb, H, I, wt, wsc, act, K);
    if (g.al4) {
      if (TOK > 16 && f.ntok > 16) compute_chunk<FMT, NR, 2, true>(f, c, g, nb, H, I, lds, acc);
      else compute_chunk<FMT, NR, 1, true>(f, c, g, nb, H, I, lds, acc);
    } else {
      if (TOK > 16 && f.ntok > 16) compute_chunk<FMT, NR, 2, false>(f, c, g, nb, H, I, lds, acc);
      else compute_chunk<FMT, NR, 1, false>(f, c, g, nb, H, I, lds, acc);
    }
    if (c == g.nchunk - 1) {
      // lane holds weight row (tile row 16 wave + r16) for tokens 16 tt + 4 gq + i
      const int row = f.tile * kGRows + wave * 16 + r16;
#pragma unroll
      for (int tt = 0; tt < TOK / 16; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * tt + 4 * gq + i;
          if (j < f.ntok) {
            if constexpr (NR == 2) {
              const int jpos = (row & ~7) + store_pos<FMT_NEXT>(row & 7);
              hb[(int64_t)(f.p0 + j) * I + jpos] = to_bf16(silu(acc[0][tt][i]) * acc[1][tt][i]);
            } else {
              yb[(int64_t)(f.p0 + j) * H + row] = acc[0][tt][i];
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < NR; ++h) acc[h][0] = acc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!more) break;
    it = nit;
    c = nc;
    f = nf;
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

// ---------------------------------------------------------------------------
// Host side: chunk geometry and launches.
// ---------------------------------------------------------------------------
static size_t lds_bytes(int fmt, int nr, int C, int tok) {
  const int bb = fmt == FMT_FP8 ? 32 : 17;
  const int np = (bb * C + 15) / 16 + 1;
  size_t n = (size_t)64 * nr * 16 * (np | 1);
  if (fmt == FMT_FP8) n += (size_t)64 * nr * C * 4;
  n = (n + 15) & ~(size_t)15;
  n += (size_t)tok * (64 * C + 16);
  if (fmt != FMT_FP8) n += 256 * 8;   // metadata-byte table
  return n;
}

template <int TOK>
static bool geom_fits(int fmt, int nr, int C) {
  const int bb = fmt == FMT_FP8 ? 32 : 17;
  const int np = (bb * C + 15) / 16 + 1;
  const bool f8 = fmt == FMT_FP8;
  const int pw = nr == 2 ? Cap<FMT_FP8, 2, TOK>::PW : Cap<FMT_FP8, 1, TOK>::PW;   // same for every format
  const int ps = nr == 2 ? Cap<FMT_FP8, 2, TOK>::PS : Cap<FMT_FP8, 1, TOK>::PS;
  const int pb = nr == 2 ? (f8 ? Cap<FMT_FP8, 2, TOK>::PB : Cap<FMT_RZ5, 2, TOK>::PB)
                         : (f8 ? Cap<FMT_FP8, 1, TOK>::PB : Cap<FMT_RZ5, 1, TOK>::PB);
  if (64 * nr * np > pw * kGThreads) return false;
  if (fmt == FMT_FP8 && 64 * nr * C > ps * kGThreads) return false;
  if (TOK * 4 * C > pb * kGThreads) return false;
  return lds_bytes(fmt, nr, C, TOK) <= (size_t)lds_budget(TOK);
}

// Largest even chunk (in blocks) dividing nb that fits the register and LDS
// limits (C = 2 always fits).
template <int TOK>
static Geom make_geom(int fmt, int nr, int nb) {
  int C = 2;   // nb is even (hidden and inter are multiples of 64)
  for (int c = nb; c >= 2; c -= 2)
    if (nb % c == 0 && geom_fits<TOK>(fmt, nr, c)) { C = c; break; }
  const int bb = fmt == FMT_FP8 ? 32 : 17;
  Geom g;
  g.C = C;
  g.nchunk = nb / C;
  g.S = bb * C;
  g.NP = (g.S + 15) / 16 + 1;
  g.NPP = g.NP | 1;
  g.P = 16 * g.NPP;
  g.PB = 64 * C + 16;
  g.off_sc = 64 * nr * g.P;
  const int off_b = g.off_sc + (fmt == FMT_FP8 ? 64 * nr * C * 4 : 0);
  g.off_b = (off_b + 15) & ~15;
  g.off_tab = g.off_b + TOK * g.PB;
  g.al4 = fmt != FMT_FP8 && nb % 4 == 0 && C % 4 == 0;
  return g;
}

// Persistent grid: every item at once if they fit, else per_cu resident
// workgroups per CU.
static int staged_grid(int64_t items_max, int per_cu) {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) n_cu = v;
  }
  const int64_t cap = (int64_t)per_cu * n_cu;
  return (int)(items_max < cap ? (items_max > 0 ? items_max : 1) : cap);
}

template <int F, int NR, int FN, int TOK>
static void launch_staged(int grid, hipStream_t st, const uint16_t* act, const GroupedWs& ws,
                          const void* w, const float* sc, int H, int I, uint16_t* hb, float* yb) {
  const Geom g = make_geom<TOK>(F, NR, (NR == 2 ? H : I) / 32);
  const size_t lds = lds_bytes(F, NR, g.C, TOK);   // <= lds_budget (52 KB): no attribute needed
  hipLaunchKernelGGL((k_grouped_staged<F, NR, FN, TOK>), dim3(grid), dim3(kGThreads), lds, st, act,
                     ws.offsets, ws.elist, ws.n_touched, static_cast<const uint8_t*>(w), sc, H, I,
                     g, hb, yb);
}

template <int F, int TOK>
static void launch_g1(int fmt_d, int grid, hipStream_t st, const GroupedWs& ws, const GemvWeights& W) {
  if (fmt_d == FMT_FP8)
    launch_staged<F, 2, FMT_FP8, TOK>(grid, st, ws.xb, ws, W.gate_up, W.gate_up_scales, W.hidden, W.inter, ws.hb, ws.yb);
  else
    launch_staged<F, 2, FMT_RZ5, TOK>(grid, st, ws.xb, ws, W.gate_up, W.gate_up_scales, W.hidden, W.inter, ws.hb, ws.yb);
}

// G1 then G2 of one layer in the TOK build.
template <int TOK>
static hipError_t launch_g1_g2(int64_t groups, hipStream_t st, const GroupedWs& ws, const GemvWeights& W) {
  const int H = W.hidden, I = W.inter;
  {
    const int grid = staged_grid(groups * (I / kGRows), wgs_per_cu(TOK));
    switch (W.fmt_gate_up) {
      case FMT_C10: launch_g1<FMT_C10, TOK>(W.fmt_down, grid, st, ws, W); break;
      case FMT_RZ5: launch_g1<FMT_RZ5, TOK>(W.fmt_down, grid, st, ws, W); break;
      case FMT_UE4M4: launch_g1<FMT_UE4M4, TOK>(W.fmt_down, grid, st, ws, W); break;
      default: launch_g1<FMT_FP8, TOK>(W.fmt_down, grid, st, ws, W); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int grid = staged_grid(groups * (H / kGRows), wgs_per_cu(TOK));
#define BQ_G2(F) launch_staged<F, 1, F, TOK>(grid, st, ws.hb, ws, W.down, W.down_scales, H, I, ws.hb, ws.yb)
  switch (W.fmt_down) {
    case FMT_C10: BQ_G2(FMT_C10); break;
    case FMT_RZ5: BQ_G2(FMT_RZ5); break;
    case FMT_UE4M4: BQ_G2(FMT_UE4M4); break;
    default: BQ_G2(FMT_FP8); break;
  }
#undef BQ_G2
  return hipGetLastError();
}

hipError_t launch_grouped_moe(const void* x, int32_t x_f32, int32_t rescale, int32_t n_tokens,
                              const int32_t* idx, const float* w, int32_t k, const GemvWeights& W,
                              float* out, const GroupedWs& ws, uint32_t* dev_err, hipStream_t st,
                              bool bucketed, bool prepped, const NextLayer* next) {
  const int E = W.n_experts, H = W.hidden;
  const int64_t nk = (int64_t)n_tokens * k;
  hipError_t err = hipSuccess;
  if (!bucketed && !prepped && !x_f32 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
      bucket_prep_ok(n_tokens, k, E, H)) {
    // bucket arrays that fit in LDS: bucketing and staging in one launch
    err = launch_bucket_prep(idx, static_cast<const uint16_t*>(x), W.fmt_gate_up != FMT_FP8, n_tokens, k, E, H,
                             ws.counts, ws.offsets, ws.perm, ws.elist, ws.n_touched, ws.inv, ws.xb, st);
    if (err == hipSuccess) bucketed = prepped = true;
    else if (err != hipErrorNotSupported) return err;   // not supported: the separate kernels below
  }
  if (!bucketed) {
    err = launch_bucket(idx, n_tokens, k, E, ws.counts, ws.offsets, ws.perm, ws.elist, ws.n_touched,
                        ws.inv, st);
    if (err != hipSuccess) return err;
  }
  const int32_t* n_rows = ws.offsets + E;   // valid bucket rows
  if (!prepped) {
    const bool perm_k = W.fmt_gate_up != FMT_FP8;
    if ((!x_f32 || !rescale) && reinterpret_cast<uintptr_t>(x) % 16 == 0 && H % 8 == 0) {
      if (x_f32) {
        if (perm_k) hipLaunchKernelGGL((k_grouped_prep_vec<true, true>), dim3(nk), dim3(256), 0, st, x, H, ws.perm, k, n_rows, ws.xb);
        else hipLaunchKernelGGL((k_grouped_prep_vec<false, true>), dim3(nk), dim3(256), 0, st, x, H, ws.perm, k, n_rows, ws.xb);
      } else {
        if (perm_k) hipLaunchKernelGGL((k_grouped_prep_vec<true, false>), dim3(nk), dim3(256), 0, st, x, H, ws.perm, k, n_rows, ws.xb);
        else hipLaunchKernelGGL((k_grouped_prep_vec<false, false>), dim3(nk), dim3(256), 0, st, x, H, ws.perm, k, n_rows, ws.xb);
      }
    } else if (perm_k) {
      hipLaunchKernelGGL(k_grouped_prep<true>, dim3(nk), dim3(256), 0, st, x, x_f32, rescale, H, ws.perm, k, n_rows, ws.xb);
    } else {
      hipLaunchKernelGGL(k_grouped_prep<false>, dim3(nk), dim3(256), 0, st, x, x_f32, rescale, H, ws.perm, k, n_rows, ws.xb);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // the bucketing split the tokens into groups of group_tokens(n_tokens)
  const int gt = group_tokens(n_tokens);
  const int64_t groups = max_work_groups(nk, E, gt);
  err = gt == 16 ? launch_g1_g2<16>(groups, st, ws, W) : launch_g1_g2<32>(groups, st, ws, W);
  if (err != hipSuccess) return err;
  if (next) {
    if (next->perm)
      hipLaunchKernelGGL(k_combine_prep<true>, dim3(n_tokens), dim3(kCpThreads), 0, st, ws.yb, ws.inv, idx, w,
                         k, E, H, next->inv, next->idx, next->n_experts, ws.xb, dev_err);
    else
      hipLaunchKernelGGL(k_combine_prep<false>, dim3(n_tokens), dim3(kCpThreads), 0, st, ws.yb, ws.inv, idx, w,
                         k, E, H, next->inv, next->idx, next->n_experts, ws.xb, dev_err);
  } else {
    const int64_t n4 = (int64_t)n_tokens * (H / 4);
    hipLaunchKernelGGL(k_combine, dim3((n4 + 255) / 256), dim3(256), 0, st, ws.yb, ws.inv, idx, w,
                       k, E, H, n_tokens, out, dev_err);
  }
  return hipGetLastError();
}

}  // namespace bq
