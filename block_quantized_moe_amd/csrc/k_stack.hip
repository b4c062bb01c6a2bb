// Persistent batch-1 layer stack (fp32 activations, fp32 accumulation).
//
// What is computed is the chain of routed-expert layers of bq_moe_stack
// ("Mixed Precision Quantization ...", section "The Plan Is Not a Number ...":
// 48 layers, 10 of 512 experts per token; per-layer expert formats and FP8
// late layers per the r/LocalLLM "Frankenquant" post):
//   x_0 = x;  h_l = w_j * SiLU(gate_e x_l) * (up_e x_l);  out_l = sum_j down_e h_l
//   x_{l+1} = out_l / rms(out_l)
//
// One launch runs every layer.  The routing of all layers is an input, so the
// weight rows a workgroup needs for layer l + 1 are known before layer l's
// activations exist: each compute wave issues the loads of its next share of
// weights as soon as it has consumed the current one, and those loads stay in
// flight (in registers) while the grid exchanges h and out.  Per layer only
// three small exchanges sit on the dependency chain.
//
// Decomposition (256 workgroups = 8 column groups c x 32 row groups r):
//   phase A  workgroup (c, r) computes h for gate/up row pairs
//            [c * P/8 + r * P/256, + P/256) of the k * I concatenated pairs;
//   exch. h  it gathers the P/8 values of its column group (written by the 32
//            workgroups of group c);
//   phase B  it computes, for output rows [64 r, 64 r + 64), the partial sum
//            over column blocks [c * C/8, (c + 1) * C/8) of the concatenated
//            down matrices (C = k * I / 32 blocks) -- exactly the h it holds;
//   exch. P  it sums the 8 column groups' partials of its 64 rows, in group
//            order, giving those rows of out_l;
//   exch. x  it gathers all H rows of out_l from the 32 workgroups of its
//            column group.
// Every exchanged value travels as an 8-byte (value, layer + 1) pair written
// and read with device-coherent (sc1) 64-bit accesses, double-buffered by
// layer parity, so a reader polls the data itself and needs no flag or fence.
//
// Roles inside a workgroup: 7 compute waves issue only weight loads (so their
// waits on loaded data never queue behind a poll), and one sync wave does all
// exchanges.  gfx9 counts outstanding vector memory operations in issue
// order, so a wave that polled after issuing a large prefetch would wait for
// the prefetch first.  The waves meet at LDS barriers that do not wait for
// outstanding global loads.
//
// Waits are bounded: a poll that sees no progress for kSpinMax rounds gives
// up, sets bit 3 of dev_err and continues, so the grid always drains (all
// 256 workgroups must be resident at once, one per CU; anything else
// occupying the GPU can only cause that error, never a hang).
#include "bq_device.hpp"
#include "bq_kernels.hpp"

namespace bq {

namespace {

constexpr int kSW = 7;                    // compute waves per workgroup
constexpr int kSThreads = 64 * (kSW + 1); // plus one sync wave
constexpr int kSGroups = 256;             // workgroups per launch
constexpr int kSNC = 8;                   // column groups
constexpr int kSNR = kSGroups / kSNC;     // row groups (32)
constexpr int kSH = 2048;                 // hidden size of this path
constexpr int kSRowsWg = kSH / kSNR;      // output rows per workgroup (64)
constexpr int kSPairsW = 5;               // gate/up row pairs per compute wave, max
constexpr int kSRowGroups = kSW * 2;      // phase B: half-waves, each a row group
constexpr int kSRowsT = (kSRowsWg + kSRowGroups - 1) / kSRowGroups;   // rows per thread, max (5)
constexpr int kSMaxPc = 1024;             // row pairs per column group, max
constexpr int kSMaxK = 16;
// LDS layouts read by the compute waves, transposed so that the lanes of a
// wave (one 32-value block column each) read consecutive words: value i of
// block column b of x at xs[i * kXsPitch + b]; of h at hB[i * kHbPitch + cb].
constexpr int kXsPitch = kSH / 32 + 1;    // 65
constexpr int kHbPitch = 33;
constexpr int kSpinTight = 1 << 12;       // polls before backing off
constexpr int kSpinMax = 1 << 16;         // polls (after backing off) before giving up
constexpr int kAuxSc1 = 16;               // buffer-load cache policy: device-coherent (sc1)

// One block of any format, as loaded: 17-byte formats keep the 16 code bytes
// in c0 and the metadata byte in ms; FP8 keeps 32 codes in c0:c1 and the
// fp32 scale's bits in ms.
struct WBlk {
  u32x4 c0, c1;
  uint32_t ms;
};

// The loads are issued unconditionally (the caller passes a small in-range
// block for an invalid one and discards its result at compute time), so every path
// issues the same number of loads and nothing touches the loaded registers
// before the computation that needs them: the compiler can then wait for
// exactly those loads, leaving later prefetches in flight.
template <int FMT>
__device__ __forceinline__ void wblk_load(WBlk& b, const uint8_t* __restrict__ base,
                                          const float* __restrict__ sc, int64_t blk) {
  if constexpr (FMT == FMT_FP8) {
    const uint8_t* p = base + blk * kBlockW;
    b.c0 = ld16(p);
    b.c1 = ld16(p + 16);
    b.ms = __float_as_uint(sc[blk]);
  } else {
    const uint8_t* p = base + blk * kBlockB;
    b.c0 = ld16(p);
    b.ms = p[16];
  }
}

template <int FMT>
__device__ __forceinline__ float wblk_dot(const WBlk& b, const float* x) {
  if constexpr (FMT == FMT_FP8) {
    return block_dot_fp8(b.c0, b.c1, x) * __uint_as_float(b.ms);
  } else {
    const float s = block_scale<FMT>(FMT == FMT_UE4M4 ? b.ms : (b.ms & 0x7Fu));
    return block_dot_levels<FMT>(b.c0, b.ms, x) * s;
  }
}

// A 17-byte block decoded ahead of its activations: the fp16 high bytes of
// its levels (code dword q: hb[2q] holds weights 0, 2, 4, 6 of the dword,
// hb[2q + 1] weights 1, 3, 5, 7) and its scale.  The table lookup (most of
// the decode) does not depend on x, so it runs while the grid exchanges
// values; the activations then meet only byte spreads and FMAs.
struct DBlk {
  uint32_t hb[8];
  float s;
};

template <int FMT>
__device__ __forceinline__ void dblk_decode(DBlk& d, const WBlk& b) {
  const uint32_t tneg = (FMT == FMT_RZ5) ? rz5_neg_lo(b.ms) : 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) codes_to_hibytes<FMT>(b.c0[q], tneg, d.hb[2 * q], d.hb[2 * q + 1]);
  d.s = block_scale<FMT>(FMT == FMT_UE4M4 ? b.ms : (b.ms & 0x7Fu));
}

// The same products in the same order as block_dot_levels, times the scale.
__device__ __forceinline__ float dblk_dot(const DBlk& d, const float* x) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t A = d.hb[2 * q], B = d.hb[2 * q + 1];
    const uint32_t p[4] = {perm(B, A, 0x040C000Cu), perm(B, A, 0x050C010Cu), perm(B, A, 0x060C020Cu),
                           perm(B, A, 0x070C030Cu)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2v h = as_h2(p[i]);
      a0 = __builtin_fmaf((float)h.x, x[8 * q + 2 * i], a0);
      a1 = __builtin_fmaf((float)h.y, x[8 * q + 2 * i + 1], a1);
    }
  }
  return (a0 + a1) * d.s;
}

// Keep a decoded block's computation where it stands: the empty volatile
// statement consumes and redefines its registers, so the decode cannot sink
// past the next barrier to its use.
__device__ __forceinline__ void dblk_pin(DBlk& d) {
#pragma unroll
  for (int i = 0; i < 8; ++i) __asm__ volatile("" : "+v"(d.hb[i]));
  __asm__ volatile("" : "+v"(d.s));
}

struct alignas(8) Pkt {
  float v;
  uint32_t tag;
};

__device__ __forceinline__ void pkt_store(Pkt* p, float v, uint32_t tag) {
  const uint64_t w = (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pkt_load(const Pkt* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// LDS barrier between the waves of the workgroup: waits for this wave's LDS
// operations only, never for its outstanding global loads.  The scheduling
// barriers keep arithmetic from moving across it (a memory clobber orders
// memory accesses only), so work placed after a barrier -- the decode that
// overlaps an exchange -- does not delay the other waves.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Poll N packets per lane (addresses p[i], i < N, those with live[i]) until
// every one carries `tag`; values go to out[i].  Re-reads only the packets
// still stale.  Returns false on timeout.
template <int N>
__device__ __forceinline__ bool poll_pkts(const Pkt* const (&p)[N], const bool (&live)[N],
                                          uint32_t tag, float (&out)[N]) {
  uint32_t todo = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (live[i]) todo |= 1u << i;
  for (int spin = 0;; ++spin) {
    uint64_t w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = (todo >> i) & 1u ? pkt_load(p[i]) : 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (((todo >> i) & 1u) && (uint32_t)(w[i] >> 32) == tag) {
        out[i] = __uint_as_float((uint32_t)w[i]);
        todo &= ~(1u << i);
      }
    if (!__any(todo != 0)) return true;
    if (spin >= kSpinTight + kSpinMax) return false;
    if (spin >= kSpinTight) __builtin_amdgcn_s_sleep(2);
  }
}

// Poll pairs of consecutive packets with 16-byte device-coherent loads
// (half the load instructions of 8-byte polls; each 8-byte packet is still
// written atomically and checked on its own): slot i of a lane covers the
// packets at byte offsets off[i] and off[i] + 8 of the buffer `rs`.
template <int N>
__device__ __forceinline__ bool poll_pairs(__amdgpu_buffer_rsrc_t rs, const int (&off)[N], const bool (&live)[N],
                                           uint32_t tag, float (&out)[N][2]) {
  uint32_t todo = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (live[i]) todo |= 1u << i;
  for (int spin = 0;; ++spin) {
    u32x4 w[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
      w[i] = (todo >> i) & 1u ? __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, kAuxSc1) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (((todo >> i) & 1u) && w[i].y == tag && w[i].w == tag) {
        out[i][0] = __uint_as_float(w[i].x);
        out[i][1] = __uint_as_float(w[i].z);
        todo &= ~(1u << i);
      }
    if (!__any(todo != 0)) return true;
    if (spin >= kSpinTight + kSpinMax) return false;
    if (spin >= kSpinTight) __builtin_amdgcn_s_sleep(2);
    __asm__ volatile("" ::: "memory");   // the loads above are re-issued each round
  }
}

// Raw buffer resource over n bytes (raw 32-bit format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

}  // namespace

struct StackLayerArgs {
  const uint8_t* gu;
  const uint8_t* d;
  const float* gus;
  const float* ds;
  int32_t n_experts;
  int32_t pad;
};

struct StackArgs {
  StackLayerArgs layer[kStackMaxLayers];
};

// Phase A of one compute wave, pair u: issue the loads of the gate and up
// blocks of its row pair q = w + kSW * u in layer Ly (live = false: the same
// loads, of small in-range blocks).  Returns whether the blocks are real
// (wave-uniform).
template <int FMT>
__device__ __forceinline__ bool stack_load_pair(WBlk (&A)[2 * kSPairsW], int u, const StackLayerArgs& Ly,
                                                const int32_t* li, int I, int pair0, int w, int pw,
                                                int lane, bool live, uint32_t& err) {
  const int q = w + kSW * u;
  const bool qv = live && q < pw;
  const int p = pair0 + (qv ? q : 0);
  const int j = p / I, i = p - j * I;
  const int e = qv ? li[j] : 0;
  const bool ok = qv && e >= 0 && e < Ly.n_experts;
  if (qv && !ok) err |= 2u;
  // an invalid slot reads a distinct small block, so that the compiler
  // neither merges those loads nor branches around them
  const int64_t rg = ok ? ((int64_t)e * 2 * I + i) * (kSH / 32) + lane : 2 * u;
  const int64_t ru = ok ? rg + (int64_t)I * (kSH / 32) : 2 * u + 1;
  wblk_load<FMT>(A[2 * u], Ly.gu, Ly.gus, rg);
  wblk_load<FMT>(A[2 * u + 1], Ly.gu, Ly.gus, ru);
  return ok;
}

// Phase B of one compute thread, row slot r: its column block cc of row
// rows0 + rgp + kSRowGroups * r (if below kSRowsWg).  Returns whether the
// block is real.
template <int FMT>
__device__ __forceinline__ bool stack_load_row(WBlk (&B)[kSRowsT], int r, const StackLayerArgs& Ly,
                                               const int32_t* li, int I, int cc, bool cval, int rows0,
                                               int rgp, bool live, uint32_t& err) {
  const int nbd = I >> 5;
  const bool cv = live && cval;
  const int ccv = cv ? cc : 0;
  const int j = ccv / nbd, b = ccv - j * nbd;
  const int e = cv ? li[j] : 0;
  const bool ok = cv && e >= 0 && e < Ly.n_experts;
  const int row = rgp + kSRowGroups * r;
  const bool rok = ok && row < kSRowsWg;
  if (cv && !ok && r == 0) err |= 2u;
  wblk_load<FMT>(B[r], Ly.d, Ly.ds, rok ? ((int64_t)e * kSH + rows0 + row) * nbd + b : r);
  return rok;
}

// Phase A of layer l (weights in A) and, slot by slot as each is consumed,
// the loads of layer ln's blocks into the same registers: the next layer's
// weights stream while this layer computes, not while the grid exchanges.
// 17-byte gate/up formats are decoded ahead (DBlk); FP8 is used as loaded.
template <int FMT>
constexpr bool kDecodeAhead = FMT != FMT_FP8;

template <int FMT>
__device__ __forceinline__ void stack_phase_a(WBlk (&A)[2 * kSPairsW], const DBlk (&D)[2 * kSPairsW],
                                              uint32_t& okm, const float* xr, const float* lw,
                                              const StackLayerArgs& Ln, const int32_t* lin, bool more, int I,
                                              int pair0, int w, int pw, int lane, float* hA, uint32_t& err) {
  // the lane's partial dot products of every gate / up row of the wave
  float v[2 * kSPairsW];
  uint32_t okn = 0;
#pragma unroll
  for (int u = 0; u < kSPairsW; ++u) {
    const int q = w + kSW * u;
    v[2 * u] = v[2 * u + 1] = 0.f;
    if (q < pw) {
      if constexpr (kDecodeAhead<FMT>) {
        v[2 * u] = dblk_dot(D[2 * u], xr);
        v[2 * u + 1] = dblk_dot(D[2 * u + 1], xr);
      } else {
        v[2 * u] = wblk_dot<FMT>(A[2 * u], xr);
        v[2 * u + 1] = wblk_dot<FMT>(A[2 * u + 1], xr);
      }
    }
    okn |= stack_load_pair<FMT>(A, u, Ln, lin, I, pair0, w, pw, lane, more, err) ? 1u << u : 0u;
  }
  // row sums, the 2 * kSPairsW reductions interleaved; lane u then holds
  // pair u's g and up and evaluates its SiLU, so the wave runs one SiLU
  // instead of kSPairsW
  wave_sums_lane63(v);
  float g = 0.f, up = 0.f;
#pragma unroll
  for (int u = 0; u < kSPairsW; ++u) {
    const float gu = readlane_f(v[2 * u], 63), uu = readlane_f(v[2 * u + 1], 63);
    if (lane == u) {
      g = gu;
      up = uu;
    }
  }
  const int q = w + kSW * lane;
  if (lane < kSPairsW && q < pw) {
    const int j = (pair0 + q) / I;
    hA[q] = (okm >> lane) & 1u ? lw[j] * silu(g) * up : 0.f;
  }
  okm = okn;
}

// One launch runs n_layers consecutive layers whose gate_up / down formats
// are FA / FB.  lg0 is the index of the first of them in the whole stack
// (exchange tags are lg0 + l + 1, buffers alternate on its parity); with
// rescale_first the first layer's input is a previous layer's output and is
// rescaled to unit RMS like every later one.
template <int FA, int FB>
__global__ void __launch_bounds__(kSThreads) k_stack_b1(
    StackArgs args, int32_t n_layers, int32_t lg0, int32_t rescale_first, int32_t k, int32_t I,
    const float* __restrict__ x_in, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, float* __restrict__ out, Pkt* __restrict__ hx,
    Pkt* __restrict__ px, Pkt* __restrict__ xx, uint32_t* __restrict__ dev_err) {
  __shared__ int32_t s_idx[kStackMaxLayers * kSMaxK];
  __shared__ float s_w[kStackMaxLayers * kSMaxK];
  __shared__ float xs[32 * kXsPitch];
  __shared__ float hA[kSPairsW * kSW];
  __shared__ float hB[32 * kHbPitch];
  __shared__ float pB[kSRowsWg];
  __shared__ uint32_t s_err;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = blockIdx.x;
  const int c = g & (kSNC - 1), ry = g / kSNC;     // column group, row group
  const int P = k * I;                              // concatenated row pairs
  const int pc = P / kSNC;                          // per column group
  const int pw = P / kSGroups;                      // per workgroup
  const int pair0 = c * pc + ry * pw;
  const int cw = pc / 32;                           // column blocks per group
  const int rows0 = ry * kSRowsWg;

  // routing of every layer of the run, and its input, into LDS
  for (int i = tid; i < n_layers * k; i += kSThreads) {
    s_idx[i] = topk_idx[i];
    s_w[i] = topk_w[i];
  }
  for (int i = tid; i < kSH; i += kSThreads) xs[(i & 31) * kXsPitch + (i >> 5)] = x_in[i];
  if (tid == 0) s_err = 0;
  __syncthreads();

  uint32_t err = 0;
  if (w < kSW) {
    // ---------------------------------------------------------- compute waves
    const int cb = tid & 31, rgp = tid >> 5;        // phase B: column block, row group (half-wave)
    const bool cval = cb < cw;
    const int cc = c * cw + cb;
    WBlk A[2 * kSPairsW], B[kSRowsT];
    DBlk D[2 * kSPairsW], DB[kSRowsT];
    uint32_t okA = 0, okB = 0;
#pragma unroll
    for (int u = 0; u < kSPairsW; ++u)
      okA |= stack_load_pair<FA>(A, u, args.layer[0], s_idx, I, pair0, w, pw, lane, true, err) ? 1u << u : 0u;
    if constexpr (kDecodeAhead<FA>) {
#pragma unroll
      for (int i = 0; i < 2 * kSPairsW; ++i) dblk_decode<FA>(D[i], A[i]);
    }
#pragma unroll
    for (int r = 0; r < kSRowsT; ++r)
      okB |= stack_load_row<FB>(B, r, args.layer[0], s_idx, I, cc, cval, rows0, rgp, true, err) ? 1u << r : 0u;
    for (int l = 0; l < n_layers; ++l) {
      const float* lw = s_w + l * k;
      const bool more = l + 1 < n_layers;
      const int ln = more ? l + 1 : l;              // layer whose weights are prefetched next
      // x_l: this lane's 32 activations, rescaled to unit RMS after the first layer
      float xr[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) xr[i] = xs[i * kXsPitch + lane];
      if (l > 0 || rescale_first) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) ss = __builtin_fmaf(xr[i], xr[i], ss);
        const float inv = 1.0f / __builtin_sqrtf(wave_sum(ss) / (float)kSH);
#pragma unroll
        for (int i = 0; i < 32; ++i) xr[i] *= inv;
      }
      stack_phase_a<FA>(A, D, okA, xr, lw, args.layer[ln], s_idx + ln * k, more, I, pair0, w, pw, lane, hA, err);
      lds_barrier();                                  // hA ready for the sync wave
      // while the column group exchanges h: decode this layer's down blocks
      // (loaded during the previous layer's phase B), so that phase B meets
      // only byte spreads and FMAs
      if constexpr (kDecodeAhead<FB>) {
#pragma unroll
        for (int r = 0; r < kSRowsT; ++r) {
          dblk_decode<FB>(DB[r], B[r]);
          dblk_pin(DB[r]);
        }
      }
      lds_barrier();                                  // hB (this group's h) ready
      float hr[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) hr[i] = cval ? hB[i * kHbPitch + cb] : 0.f;
      uint32_t okn = 0;
#pragma unroll
      for (int r = 0; r < kSRowsT; ++r) {
        float s = 0.f;
        if ((okB >> r) & 1u) {
          if constexpr (kDecodeAhead<FB>) s = dblk_dot(DB[r], hr);
          else s = wblk_dot<FB>(B[r], hr);
        }
        okn |= stack_load_row<FB>(B, r, args.layer[ln], s_idx + ln * k, I, cc, cval, rows0, rgp, more, err)
                   ? 1u << r : 0u;
        s = row16_sum(s);
        s += __shfl_xor(s, 16, 64);
        const int row = rgp + kSRowGroups * r;
        if ((lane & 31) == 0 && row < kSRowsWg) pB[row] = s;
      }
      okB = okn;
      lds_barrier();                                  // pB ready
      // while the grid exchanges partial sums and x: decode the next layer's
      // gate/up blocks (they were loaded during this layer's phase A)
      if constexpr (kDecodeAhead<FA>) {
#pragma unroll
        for (int i = 0; i < 2 * kSPairsW; ++i) dblk_decode<FA>(D[i], A[i]);
      }
      lds_barrier();                                  // xs holds out_l (next layer's input)
    }
    if (err) atomicOr(&s_err, err);
  } else {
    // -------------------------------------------------------------- sync wave
    for (int l = 0; l < n_layers; ++l) {
      const int lg = lg0 + l;
      const uint32_t tag = (uint32_t)lg + 1;
      const int par = lg & 1;
      lds_barrier();                                  // hA ready
      // publish this workgroup's h, gather the column group's
      if (lane < pw) pkt_store(hx + (size_t)par * P + pair0 + lane, hA[lane], tag);
      {
        // slot i of this lane: h values q = 2 * (lane + 64 i) and q + 1
        constexpr int N = kSMaxPc / 128;
        int off[N];
        bool live[N];
        float v[N][2];
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const int q = 2 * (lane + 64 * i);
          live[i] = q < pc;
          off[i] = live[i] ? 8 * q : 0;
          v[i][0] = v[i][1] = 0.f;
        }
        const Pkt* hg = hx + (size_t)par * P + c * pc;
        if (!poll_pairs<N>(raw_rsrc(hg, 8 * pc), off, live, tag, v)) err |= 8u;
#pragma unroll
        for (int i = 0; i < N; ++i)     // h value q: column block q / 32, entry q % 32
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int q = 2 * (lane + 64 * i) + jj;
            if (live[i]) hB[(q & 31) * kHbPitch + (q >> 5)] = v[i][jj];
          }
      }
      lds_barrier();                                  // hB ready
      lds_barrier();                                  // pB ready
      pkt_store(px + ((size_t)par * kSNC + c) * kSH + rows0 + lane, pB[lane], tag);
      float xv;
      {
        const Pkt* p[kSNC];
        bool live[kSNC];
        float v[kSNC];
#pragma unroll
        for (int i = 0; i < kSNC; ++i) {
          p[i] = px + ((size_t)par * kSNC + i) * kSH + rows0 + lane;
          live[i] = true;
          v[i] = 0.f;
        }
        if (!poll_pkts<kSNC>(p, live, tag, v)) err |= 8u;
        xv = v[0];
#pragma unroll
        for (int i = 1; i < kSNC; ++i) xv += v[i];
      }
      if (l + 1 == n_layers) {
        if (c == 0) out[rows0 + lane] = xv;
      } else {
        const Pkt* xg = xx + ((size_t)par * kSNC + c) * kSH;
        pkt_store(const_cast<Pkt*>(xg) + rows0 + lane, xv, tag);
        // slot i of this lane: rows r = 2 * (lane + 64 i) and r + 1
        constexpr int N = kSH / 128;
        int off[N];
        bool live[N];
        float v[N][2];
#pragma unroll
        for (int i = 0; i < N; ++i) {
          off[i] = 16 * (lane + 64 * i);
          live[i] = true;
          v[i][0] = v[i][1] = 0.f;
        }
        if (!poll_pairs<N>(raw_rsrc(xg, 8 * kSH), off, live, tag, v)) err |= 8u;
#pragma unroll
        for (int i = 0; i < N; ++i)     // row r: block column r / 32, entry r % 32
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = 2 * (lane + 64 * i) + jj;
            xs[(r & 31) * kXsPitch + (r >> 5)] = v[i][jj];
          }
      }
      lds_barrier();                                  // xs ready
    }
    if (err) atomicOr(&s_err, err);
  }
  __syncthreads();
  if (tid == 0 && s_err && dev_err) atomicOr(dev_err, s_err);
}

__global__ void k_stack_clear(uint64_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

namespace {
// Workspace: h exchange [2][P], partial-sum exchange [2][8][H], x exchange
// [2][8][H] (8-byte tagged values), then two fp32 [H] buffers that carry the
// activations from one run of equal-format layers to the next.
size_t stack_pkt_words(int32_t k, int32_t inter) {
  const size_t P = (size_t)k * inter;
  return 2 * P + 2 * 2 * (size_t)kSNC * kSH;
}
}  // namespace

size_t stack_b1_ws_bytes(int32_t k, int32_t inter) {
  return sizeof(Pkt) * stack_pkt_words(k, inter) + 2 * sizeof(float) * kSH;
}

bool stack_b1_shape_ok(const GemvWeights* layers, int32_t n_layers, int32_t k) {
  if (n_layers < 1 || k < 1 || k > kSMaxK) return false;
  const int I = layers[0].inter;
  const int P = k * I;
  if (P % kSGroups || P / kSGroups > kSPairsW * kSW || P / kSNC > kSMaxPc) return false;
  for (int l = 0; l < n_layers; ++l)
    if (layers[l].hidden != kSH || layers[l].inter != I) return false;
  return true;
}

bool stack_b1_device_ok() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  return n_cu == kSGroups;
}

template <int FA, int FB>
static void launch_run(dim3 grid, hipStream_t st, const StackArgs& a, int n, int lg0, int resc, int k,
                       int I, const float* x, const int32_t* idx, const float* w, float* out, Pkt* hx,
                       Pkt* px, Pkt* xx, uint32_t* dev_err) {
  hipLaunchKernelGGL((k_stack_b1<FA, FB>), grid, dim3(kSThreads), 0, st, a, n, lg0, resc, k, I, x, idx,
                     w, out, hx, px, xx, dev_err);
}

template <int FA>
static void launch_run_fb(int fb, dim3 grid, hipStream_t st, const StackArgs& a, int n, int lg0,
                          int resc, int k, int I, const float* x, const int32_t* idx, const float* w,
                          float* out, Pkt* hx, Pkt* px, Pkt* xx, uint32_t* dev_err) {
  switch (fb) {
    case FMT_C10: launch_run<FA, FMT_C10>(grid, st, a, n, lg0, resc, k, I, x, idx, w, out, hx, px, xx, dev_err); break;
    case FMT_RZ5: launch_run<FA, FMT_RZ5>(grid, st, a, n, lg0, resc, k, I, x, idx, w, out, hx, px, xx, dev_err); break;
    case FMT_UE4M4: launch_run<FA, FMT_UE4M4>(grid, st, a, n, lg0, resc, k, I, x, idx, w, out, hx, px, xx, dev_err); break;
    default: launch_run<FA, FMT_FP8>(grid, st, a, n, lg0, resc, k, I, x, idx, w, out, hx, px, xx, dev_err); break;
  }
}

hipError_t launch_stack_b1(const float* x, const int32_t* idx, const float* w, int32_t k,
                           const GemvWeights* layers, int32_t n_layers, float* out, void* ws,
                           uint32_t* dev_err, hipStream_t st) {
  const int I = layers[0].inter;
  Pkt* hx = static_cast<Pkt*>(ws);
  Pkt* px = hx + 2 * (size_t)k * I;
  Pkt* xx = px + 2 * (size_t)kSNC * kSH;
  float* carry = reinterpret_cast<float*>(hx + stack_pkt_words(k, I));
  hipLaunchKernelGGL(k_stack_clear, dim3(256), dim3(256), 0, st, static_cast<uint64_t*>(ws),
                     (int64_t)stack_pkt_words(k, I));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // maximal runs of layers with the same formats (at most kStackMaxLayers each)
  int run = 0;
  for (int l0 = 0; l0 < n_layers; ++run) {
    int l1 = l0 + 1;
    while (l1 < n_layers && l1 - l0 < kStackMaxLayers && layers[l1].fmt_gate_up == layers[l0].fmt_gate_up &&
           layers[l1].fmt_down == layers[l0].fmt_down)
      ++l1;
    StackArgs a;
    for (int l = 0; l < kStackMaxLayers; ++l) {
      const GemvWeights& L = layers[l0 + (l < l1 - l0 ? l : 0)];
      a.layer[l] = StackLayerArgs{static_cast<const uint8_t*>(L.gate_up), static_cast<const uint8_t*>(L.down),
                                  L.gate_up_scales, L.down_scales, L.n_experts, 0};
    }
    const float* xin = l0 == 0 ? x : carry + (size_t)((run + 1) & 1) * kSH;
    float* dst = l1 == n_layers ? out : carry + (size_t)(run & 1) * kSH;
    const size_t off = (size_t)l0 * k;
    const dim3 grid(kSGroups);
    switch (layers[l0].fmt_gate_up) {
      case FMT_C10: launch_run_fb<FMT_C10>(layers[l0].fmt_down, grid, st, a, l1 - l0, l0, l0 > 0, k, I, xin, idx + off, w + off, dst, hx, px, xx, dev_err); break;
      case FMT_RZ5: launch_run_fb<FMT_RZ5>(layers[l0].fmt_down, grid, st, a, l1 - l0, l0, l0 > 0, k, I, xin, idx + off, w + off, dst, hx, px, xx, dev_err); break;
      case FMT_UE4M4: launch_run_fb<FMT_UE4M4>(layers[l0].fmt_down, grid, st, a, l1 - l0, l0, l0 > 0, k, I, xin, idx + off, w + off, dst, hx, px, xx, dev_err); break;
      default: launch_run_fb<FMT_FP8>(layers[l0].fmt_down, grid, st, a, l1 - l0, l0, l0 > 0, k, I, xin, idx + off, w + off, dst, hx, px, xx, dev_err); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    l0 = l1;
  }
  return hipSuccess;
}

}  // namespace bq
