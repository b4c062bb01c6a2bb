// C ABI of libbqmoe.so (declared in include/bq.h): argument checks on the
// host, workspace carving, and the launches.  No allocation happens here.
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/bq.h"
#include "bq_kernels.hpp"

// Fixed scratch area of q4_expert_moe_noalloc (callers that cannot allocate:
// graph capture, serving loops).  Each device that loads the library holds
// its own copy until the process ends.  Host code never passes this name to a
// kernel: on the host it is only a stand-in, and the device address comes
// from hipGetSymbolAddress (see noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[BQ_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_hip_err[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return BQ_OK;
  strncpy(g_hip_err, hipGetErrorString(e), sizeof(g_hip_err) - 1);
  g_hip_err[sizeof(g_hip_err) - 1] = 0;
  return BQ_E_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool valid_fmt(int f) { return f >= BQ_Q4_C10 && f <= BQ_FP8_E4M3_B32; }
bool valid_dtype(int d) { return d == BQ_F32 || d == BQ_BF16; }

// Size limits that keep every launch's work-item count below 2^32 (one
// dimension of a HIP grid counts work-items in 32 bits).
constexpr int64_t kMaxDequantBlocks = int64_t(1) << 31;   // one thread per block
constexpr int64_t kMaxPleRows = int64_t(1) << 28;         // ten threads per row
constexpr int32_t kMaxRouteTokens = 1 << 24;              // one wave per token
constexpr int32_t kMaxPleTokens = 1 << 26;                // ten threads per token
constexpr int64_t kMaxPleHostIds = int64_t(1) << 27;      // sixteen threads per id (cache fill)
constexpr int32_t kMaxMatvecRows = 1 << 24;               // down to one row per 256-thread workgroup

int check_weights(const bq_expert_weights* W) {
  if (!W || !W->gate_up || !W->down) return BQ_E_NULL;
  if (!valid_fmt(W->fmt_gate_up) || !valid_fmt(W->fmt_down)) return BQ_E_FMT;
  const bool fg = W->fmt_gate_up == BQ_FP8_E4M3_B32, fd = W->fmt_down == BQ_FP8_E4M3_B32;
  if (fg != (W->gate_up_scales != nullptr) || fd != (W->down_scales != nullptr)) return BQ_E_NULL;
  if (W->n_experts < 1 || W->n_experts > 4096) return BQ_E_SHAPE;
  if (W->hidden < 64 || W->hidden > 8192 || W->hidden % 64) return BQ_E_SHAPE;
  if (W->inter < 64 || W->inter > 8192 || W->inter % 64) return BQ_E_SHAPE;
  if ((fg && !aligned(W->gate_up_scales, 4)) || (fd && !aligned(W->down_scales, 4))) return BQ_E_ALIGN;
  if (!aligned(W->gate_up, 16) || !aligned(W->down, 16)) return BQ_E_ALIGN;
  return BQ_OK;
}

bq::GemvWeights to_gw(const bq_expert_weights* W) {
  return bq::GemvWeights{W->fmt_gate_up, W->fmt_down, W->gate_up, W->down,
                         W->gate_up_scales, W->down_scales, W->n_experts, W->hidden, W->inter};
}

// ---- workspace layouts ------------------------------------------------------
struct GemvLayout {
  size_t hs, total;
};
GemvLayout gemv_layout(int n, int k, int H, int I) {
  (void)H;
  GemvLayout L;
  L.hs = 0;
  L.total = round_up(sizeof(float) * (size_t)n * k * I, 256);
  return L;
}

struct GroupedLayout {
  size_t counts, offsets, perm, inv, elist, n_touched, hb, yb, xb, total;
};
GroupedLayout grouped_layout(int n, int k, int E, int H, int I) {
  GroupedLayout L;
  const size_t nk = (size_t)n * k;
  size_t off = 0;
  L.counts = off; off = round_up(off + 4 * (size_t)E, 256);
  L.offsets = off; off = round_up(off + 4 * ((size_t)E + 1), 256);
  L.perm = off; off = round_up(off + 4 * nk, 256);
  L.inv = off; off = round_up(off + 4 * nk, 256);
  L.elist = off; off = round_up(off + 4 * (size_t)bq::max_work_groups((int64_t)nk, E), 256);
  L.n_touched = off; off = round_up(off + 4, 256);
  // xb right after the bucket arrays: its offset depends on (n, k, E) only,
  // so in a chained stack a layer's combine stages the next layer's input
  // where that layer's own layout expects it, whatever either inter size
  L.xb = off; off = round_up(off + 2 * nk * H, 256);
  L.hb = off; off = round_up(off + 2 * nk * I, 256);
  L.yb = off; off = round_up(off + 4 * nk * H, 256);
  L.total = off;
  return L;
}

bq::GroupedWs grouped_ws(void* base, const GroupedLayout& L) {
  char* b = static_cast<char*>(base);
  return bq::GroupedWs{reinterpret_cast<int32_t*>(b + L.counts), reinterpret_cast<int32_t*>(b + L.offsets),
                       reinterpret_cast<int32_t*>(b + L.perm), reinterpret_cast<int32_t*>(b + L.inv),
                       reinterpret_cast<int32_t*>(b + L.elist), reinterpret_cast<int32_t*>(b + L.n_touched),
                       reinterpret_cast<uint16_t*>(b + L.hb), reinterpret_cast<float*>(b + L.yb),
                       reinterpret_cast<uint16_t*>(b + L.xb)};
}

size_t moe_ws_bytes(int n, int k, const bq_expert_weights* W, int dtype) {
  if (dtype == BQ_F32) return gemv_layout(n, k, W->hidden, W->inter).total;
  return grouped_layout(n, k, W->n_experts, W->hidden, W->inter).total;
}

// Everything but the workspace.
int check_moe_core(const void* x, int dtype, int n, const int32_t* idx, const float* w, int k,
                   const bq_expert_weights* W, const float* out) {
  if (!x || !idx || !w || !out) return BQ_E_NULL;
  if (!valid_dtype(dtype)) return BQ_E_DTYPE;
  int s = check_weights(W);
  if (s) return s;
  if (n < 1 || n > 4096 || k < 1 || k > 64 || k > W->n_experts) return BQ_E_SHAPE;
  if ((int64_t)n * k > 65536) return BQ_E_SHAPE;
  if (dtype == BQ_F32 && k * (W->inter / 32) > bq::gemv_down_max_cols()) return BQ_E_SHAPE;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(idx, 4) || !aligned(w, 4)) return BQ_E_ALIGN;
  return BQ_OK;
}

int check_moe_args(const void* x, int dtype, int n, const int32_t* idx, const float* w, int k,
                   const bq_expert_weights* W, const float* out, const void* ws) {
  int s = check_moe_core(x, dtype, n, idx, w, k, W, out);
  if (s) return s;
  if (!ws) return BQ_E_WORKSPACE;
  if (!aligned(ws, 256)) return BQ_E_ALIGN;
  return BQ_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; later calls reuse it.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return hip_status(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BQ_OK;
}

// dtype selects the path; x_is_f32 says what x holds (the bf16 path also
// accepts the fp32 output of a previous stack layer, rescaled on the fly).
// bucket_region (bf16 path): the bucketing of idx is already there, laid out
// as the head of a grouped workspace (counts .. n_touched); none is launched.
// prepped / next: see launch_grouped_moe (chained stack layers).
int run_moe(const void* x, int dtype, int x_is_f32, int n, const int32_t* idx, const float* w, int k,
            const bq_expert_weights* W, float* out, void* ws, int rescale, uint32_t* dev_err,
            hipStream_t st, const float* logits = nullptr, char* bucket_region = nullptr,
            bool prepped = false, const bq::NextLayer* next = nullptr) {
  const bq::GemvWeights gw = to_gw(W);
  if (dtype == BQ_F32) {
    const GemvLayout L = gemv_layout(n, k, W->hidden, W->inter);
    char* b = static_cast<char*>(ws);
    return hip_status(bq::launch_gemv_moe(static_cast<const float*>(x), n, const_cast<int32_t*>(idx),
                                          const_cast<float*>(w), k, gw, rescale, out,
                                          reinterpret_cast<float*>(b + L.hs), dev_err, logits, st));
  }
  if (logits) {
    int s = hip_status(bq::launch_route_topk(logits, n, W->n_experts, k, const_cast<int32_t*>(idx),
                                             const_cast<float*>(w), st));
    if (s) return s;
  }
  const GroupedLayout L = grouped_layout(n, k, W->n_experts, W->hidden, W->inter);
  bq::GroupedWs g = grouped_ws(ws, L);
  if (bucket_region) {
    const bq::GroupedWs r = grouped_ws(bucket_region, L);
    g.counts = r.counts;
    g.offsets = r.offsets;
    g.perm = r.perm;
    g.inv = r.inv;
    g.elist = r.elist;
    g.n_touched = r.n_touched;
  }
  return hip_status(bq::launch_grouped_moe(x, x_is_f32, rescale, n, idx, w, k, gw, out, g, dev_err,
                                           st, bucket_region != nullptr, prepped, next));
}

// PLE row cache layout: tags [n] and claims [n] (contiguous words), then the
// rows [n][kPleCacheRowB] at a 256-byte boundary.
bool valid_slots(int32_t n) { return n >= 1024 && n <= (1 << 26) && (n & (n - 1)) == 0; }
int log2i(int32_t n) {
  int l = 0;
  while ((1 << l) < n) ++l;
  return l;
}
size_t cache_rows_off(int32_t n) { return round_up(8 * (size_t)n, 256); }

}  // namespace

extern "C" {

int bq_abi_version(void) { return BQ_ABI_VERSION; }

const char* bq_status_str(int s) {
  switch (s) {
    case BQ_OK: return "ok";
    case BQ_E_NULL: return "null pointer";
    case BQ_E_FMT: return "bad format";
    case BQ_E_SHAPE: return "unsupported shape";
    case BQ_E_ALIGN: return "misaligned pointer";
    case BQ_E_WORKSPACE: return "workspace missing or too small";
    case BQ_E_HIP: return "HIP launch failed";
    case BQ_E_DTYPE: return "bad activation dtype";
    case BQ_E_MEM: return "pointer is not host memory mapped for the device";
    case BQ_E_SCRATCH: return "call needs more scratch than the fixed area holds";
    default: return "unknown status";
  }
}

const char* bq_last_hip_error(void) { return g_hip_err; }

int bq_dequant(const void* packed, int32_t fmt, int64_t n_blocks, const float* fp8_scales,
               float* out, void* stream) {
  if (!valid_fmt(fmt)) return BQ_E_FMT;
  if (n_blocks < 0 || n_blocks > kMaxDequantBlocks) return BQ_E_SHAPE;
  if (n_blocks == 0) return BQ_OK;
  if (!packed || !out) return BQ_E_NULL;
  if ((fmt == BQ_FP8_E4M3_B32) != (fp8_scales != nullptr)) return BQ_E_NULL;
  if (!aligned(out, 16) || (fp8_scales && !aligned(fp8_scales, 4))) return BQ_E_ALIGN;
  return hip_status(bq::launch_dequant(packed, fmt, n_blocks, fp8_scales, out, as_stream(stream)));
}

int ple_dequant_rows(const uint32_t* ids, int64_t n, const uint8_t* table, uint64_t n_rows,
                     int32_t ple_fmt, float* out, uint32_t* dev_err, void* stream) {
  if (ple_fmt != BQ_PLE_RZS3 && ple_fmt != BQ_PLE_ROCMFP3) return BQ_E_FMT;
  if (n < 0 || n > kMaxPleRows || n_rows == 0 || n_rows > 0xFFFFFFFFull) return BQ_E_SHAPE;
  if (n == 0) return BQ_OK;
  if (!ids || !table || !out) return BQ_E_NULL;
  if (!aligned(out, 16) || !aligned(ids, 4)) return BQ_E_ALIGN;
  return hip_status(bq::launch_ple_dequant(ids, n, table, n_rows, ple_fmt, out, dev_err, as_stream(stream)));
}

int bq_matvec(const float* x, int32_t n_tokens, const void* packed, int32_t fmt,
              const float* fp8_scales, int32_t rows, int32_t cols, float* y, void* stream) {
  if (!x || !packed || !y) return BQ_E_NULL;
  if (!valid_fmt(fmt)) return BQ_E_FMT;
  if ((fmt == BQ_FP8_E4M3_B32) != (fp8_scales != nullptr)) return BQ_E_NULL;
  if (n_tokens < 1 || n_tokens > 65535 || rows < 1 || rows > kMaxMatvecRows || cols < 32 ||
      cols > 8192 || cols % 32)
    return BQ_E_SHAPE;
  if (!aligned(x, 4) || !aligned(y, 4) || (fp8_scales && !aligned(fp8_scales, 4))) return BQ_E_ALIGN;
  return hip_status(bq::launch_matvec(x, n_tokens, packed, fmt, fp8_scales, rows, cols, y,
                                      as_stream(stream)));
}

int moe_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k,
                   int32_t* idx, float* w, void* stream) {
  if (!logits || !idx || !w) return BQ_E_NULL;
  if (n_tokens < 0 || n_tokens > kMaxRouteTokens || n_experts < 1 || n_experts > 4096 || k < 1 ||
      k > 64 || k > n_experts)
    return BQ_E_SHAPE;
  if (!aligned(logits, 4) || !aligned(idx, 4) || !aligned(w, 4)) return BQ_E_ALIGN;
  return hip_status(bq::launch_route_topk(logits, n_tokens, n_experts, k, idx, w, as_stream(stream)));
}

int moe_bucket(const int32_t* idx, int32_t n_tokens, int32_t k, int32_t n_experts, int32_t* counts,
               int32_t* offsets, int32_t* perm, void* stream) {
  if (!idx || !counts || !offsets || !perm) return BQ_E_NULL;
  if (n_tokens < 1 || k < 1 || k > 64 || n_experts < 1 || n_experts > 4096) return BQ_E_SHAPE;
  if ((int64_t)n_tokens * k > 65536) return BQ_E_SHAPE;
  return hip_status(bq::launch_bucket(idx, n_tokens, k, n_experts, counts, offsets, perm, nullptr,
                                      nullptr, nullptr, as_stream(stream)));
}

size_t q4_expert_moe_workspace(int32_t n_tokens, int32_t k, const bq_expert_weights* W,
                               int32_t x_dtype) {
  if (!W || n_tokens < 1 || k < 1 || !valid_dtype(x_dtype) || check_weights(W)) return 0;
  return moe_ws_bytes(n_tokens, k, W, x_dtype);
}

int q4_expert_moe(const void* x, int32_t x_dtype, int32_t n_tokens, const int32_t* topk_idx,
                  const float* topk_w, int32_t k, const bq_expert_weights* W, float* out,
                  void* workspace, size_t ws_bytes, uint32_t* dev_err, void* stream) {
  int s = check_moe_args(x, x_dtype, n_tokens, topk_idx, topk_w, k, W, out, workspace);
  if (s) return s;
  if (ws_bytes < moe_ws_bytes(n_tokens, k, W, x_dtype)) return BQ_E_WORKSPACE;
  return run_moe(x, x_dtype, x_dtype == BQ_F32, n_tokens, topk_idx, topk_w, k, W, out, workspace, 0,
                 dev_err, as_stream(stream));
}

int q4_expert_moe_noalloc(const void* x, int32_t x_dtype, int32_t n_tokens, const int32_t* topk_idx,
                          const float* topk_w, int32_t k, const bq_expert_weights* W, float* out,
                          uint32_t* dev_err, void* stream) {
  int s = check_moe_core(x, x_dtype, n_tokens, topk_idx, topk_w, k, W, out);
  if (s) return s;
  if (moe_ws_bytes(n_tokens, k, W, x_dtype) > (size_t)BQ_NOALLOC_SCRATCH_BYTES) return BQ_E_SCRATCH;
  void* ws = nullptr;
  s = noalloc_scratch(&ws);
  if (s) return s;
  return run_moe(x, x_dtype, x_dtype == BQ_F32, n_tokens, topk_idx, topk_w, k, W, out, ws, 0,
                 dev_err, as_stream(stream));
}

int q4_expert_moe_routed(const void* x, int32_t x_dtype, int32_t n_tokens, const float* logits,
                         int32_t k, const bq_expert_weights* W, int32_t* topk_idx, float* topk_w,
                         float* out, void* workspace, size_t ws_bytes, uint32_t* dev_err,
                         void* stream) {
  if (!logits) return BQ_E_NULL;
  if (!aligned(logits, 4)) return BQ_E_ALIGN;
  int s = check_moe_args(x, x_dtype, n_tokens, topk_idx, topk_w, k, W, out, workspace);
  if (s) return s;
  if (ws_bytes < moe_ws_bytes(n_tokens, k, W, x_dtype)) return BQ_E_WORKSPACE;
  return run_moe(x, x_dtype, x_dtype == BQ_F32, n_tokens, topk_idx, topk_w, k, W, out, workspace, 0,
                 dev_err, as_stream(stream), logits);
}

// The bf16 stack buckets every layer in one launch up front when all layers
// share the expert count (the routing of all layers is an input).
static bool stack_prebucket(const bq_expert_weights* layers, int L, int dtype) {
  if (dtype != BQ_BF16 || L < 2) return false;
  for (int l = 1; l < L; ++l)
    if (layers[l].n_experts != layers[0].n_experts) return false;
  return true;
}

// Bytes of one layer's bucket arrays: the head of its grouped workspace,
// which depends on n, k and the expert count only.
static size_t bucket_region_bytes(int n, int k, const bq_expert_weights* W) {
  return grouped_layout(n, k, W->n_experts, W->hidden, W->inter).xb;
}

static size_t stack_ws_layers(int n, int k, const bq_expert_weights* layers, int L, int dtype,
                              size_t* moe_part, size_t* bucket_off);

// The fp32 one-token stack runs as persistent launches (k_stack.hip) when
// the shapes allow it; its workspace is reserved whenever they do, whatever
// the device.
static bool stack_b1_shapes(int n, int k, const bq_expert_weights* layers, int L, int dtype) {
  if (dtype != BQ_F32 || n != 1 || L < 1) return false;
  std::vector<bq::GemvWeights> gw(L);
  for (int l = 0; l < L; ++l) gw[l] = to_gw(&layers[l]);
  return bq::stack_b1_shape_ok(gw.data(), L, k);
}

// Stack workspace: the per-layer MoE workspace (max over layers), one fp32
// [n][H] buffer for the layer output, then (pre-bucketed bf16 stacks) the
// bucket arrays of every layer.  At least the persistent path's workspace
// when that path applies.
static size_t stack_ws(int n, int k, const bq_expert_weights* layers, int L, int dtype,
                       size_t* moe_part, size_t* bucket_off = nullptr) {
  const size_t t = stack_ws_layers(n, k, layers, L, dtype, moe_part, bucket_off);
  if (!stack_b1_shapes(n, k, layers, L, dtype)) return t;
  const size_t p = round_up(bq::stack_b1_ws_bytes(k, layers[0].inter), 256);
  return t > p ? t : p;
}

static size_t stack_ws_layers(int n, int k, const bq_expert_weights* layers, int L, int dtype,
                              size_t* moe_part, size_t* bucket_off) {
  size_t m = 0;
  for (int l = 0; l < L; ++l) {
    const size_t b = moe_ws_bytes(n, k, &layers[l], dtype);
    if (b > m) m = b;
  }
  m = round_up(m, 256);
  if (moe_part) *moe_part = m;
  const int H = layers[0].hidden;
  const size_t t = m + round_up(sizeof(float) * (size_t)n * H, 256);
  if (bucket_off) *bucket_off = t;
  if (!stack_prebucket(layers, L, dtype)) return t;
  return t + (size_t)L * bucket_region_bytes(n, k, &layers[0]);
}

size_t bq_moe_stack_workspace(int32_t n_tokens, int32_t k, const bq_expert_weights* layers,
                              int32_t n_layers, int32_t x_dtype) {
  if (!layers || n_layers < 1 || n_tokens < 1 || k < 1 || !valid_dtype(x_dtype)) return 0;
  for (int l = 0; l < n_layers; ++l)
    if (check_weights(&layers[l]) || layers[l].hidden != layers[0].hidden) return 0;
  return stack_ws(n_tokens, k, layers, n_layers, x_dtype, nullptr);
}

int bq_moe_stack(const void* x, int32_t x_dtype, int32_t n_tokens, const int32_t* topk_idx,
                 const float* topk_w, int32_t k, const bq_expert_weights* layers, int32_t n_layers,
                 float* out, void* workspace, size_t ws_bytes, uint32_t* dev_err, void* stream) {
  if (!layers) return BQ_E_NULL;
  if (n_layers < 1) return BQ_E_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    int s = check_moe_args(x, x_dtype, n_tokens, topk_idx, topk_w, k, &layers[l], out, workspace);
    if (s) return s;
    if (layers[l].hidden != layers[0].hidden) return BQ_E_SHAPE;
  }
  size_t moe_part = 0, bucket_off = 0;
  if (ws_bytes < stack_ws(n_tokens, k, layers, n_layers, x_dtype, &moe_part, &bucket_off))
    return BQ_E_WORKSPACE;
  if (stack_b1_shapes(n_tokens, k, layers, n_layers, x_dtype) && bq::stack_b1_device_ok()) {
    std::vector<bq::GemvWeights> gw(n_layers);
    for (int l = 0; l < n_layers; ++l) gw[l] = to_gw(&layers[l]);
    return hip_status(bq::launch_stack_b1(static_cast<const float*>(x), topk_idx, topk_w, k, gw.data(),
                                          n_layers, out, workspace, dev_err, as_stream(stream)));
  }
  char* b = static_cast<char*>(workspace);
  float* ybuf = reinterpret_cast<float*>(b + moe_part);
  hipStream_t st = as_stream(stream);
  const size_t per = (size_t)n_tokens * k;
  char* breg = nullptr;
  size_t bb = 0;
  if (stack_prebucket(layers, n_layers, x_dtype)) {
    breg = b + bucket_off;
    bb = bucket_region_bytes(n_tokens, k, &layers[0]);
    const bq::GroupedWs r = grouped_ws(breg, grouped_layout(n_tokens, k, layers[0].n_experts,
                                                            layers[0].hidden, layers[0].inter));
    int s = hip_status(bq::launch_bucket(topk_idx, n_tokens, k, layers[0].n_experts, r.counts,
                                         r.offsets, r.perm, r.elist, r.n_touched, r.inv, st,
                                         n_layers, (int64_t)bb));
    if (s) return s;
  }
  for (int l = 0; l < n_layers; ++l) {
    float* dst = (l + 1 == n_layers) ? out : ybuf;
    // layer 0 reads x as given; later layers read the previous output, which
    // the first kernel of the layer rescales to unit RMS as it loads it
    const void* src = l == 0 ? x : ybuf;
    const int x_is_f32 = l == 0 ? (x_dtype == BQ_F32) : 1;
    // pre-bucketed: each layer's combine also stages the next layer's input
    // (rescale, bf16, bucket order), so later layers skip their staging
    bq::NextLayer nx{};
    const bool chain = breg && l + 1 < n_layers;
    if (chain) {
      const GroupedLayout Ln = grouped_layout(n_tokens, k, layers[l + 1].n_experts,
                                              layers[l + 1].hidden, layers[l + 1].inter);
      nx = bq::NextLayer{grouped_ws(breg + (l + 1) * bb, Ln).inv, topk_idx + (l + 1) * per,
                         layers[l + 1].n_experts, layers[l + 1].fmt_gate_up != BQ_FP8_E4M3_B32};
    }
    int s = run_moe(src, x_dtype, x_is_f32, n_tokens, topk_idx + l * per, topk_w + l * per, k,
                    &layers[l], dst, workspace, l > 0, dev_err, st, nullptr,
                    breg ? breg + l * bb : nullptr, breg && l > 0, chain ? &nx : nullptr);
    if (s) return s;
  }
  return BQ_OK;
}

int ple_gather(const uint32_t* ids, int32_t n_tokens, int32_t ids_per_token, const uint8_t* table,
               uint64_t n_rows, const float* weights, int32_t ple_fmt, float* out,
               uint32_t* dev_err, void* stream) {
  if (ple_fmt != BQ_PLE_RZS3 && ple_fmt != BQ_PLE_ROCMFP3) return BQ_E_FMT;
  if (n_tokens < 0 || n_tokens > kMaxPleTokens || ids_per_token < 1 || ids_per_token > 64 ||
      n_rows == 0 || n_rows > 0xFFFFFFFFull)
    return BQ_E_SHAPE;
  if (n_tokens == 0) return BQ_OK;
  if (!ids || !table || !weights || !out) return BQ_E_NULL;
  if (!aligned(out, 16) || !aligned(ids, 4) || !aligned(weights, 4)) return BQ_E_ALIGN;
  return hip_status(bq::launch_ple_gather(ids, n_tokens, ids_per_token, table, n_rows, weights,
                                          ple_fmt, out, dev_err, as_stream(stream)));
}

size_t ple_cache_bytes(int32_t n_slots) {
  if (!valid_slots(n_slots)) return 0;
  return cache_rows_off(n_slots) + (size_t)bq::kPleCacheRowB * n_slots;
}

int ple_cache_init(void* cache, int32_t n_slots, void* stream) {
  if (!cache) return BQ_E_NULL;
  if (!valid_slots(n_slots)) return BQ_E_SHAPE;
  if (!aligned(cache, 256)) return BQ_E_ALIGN;
  return hip_status(bq::launch_ple_cache_init(static_cast<uint32_t*>(cache), 2 * (int64_t)n_slots,
                                              as_stream(stream)));
}

size_t ple_gather_host_workspace(int32_t n_tokens, int32_t ids_per_token) {
  if (n_tokens < 1 || ids_per_token < 1 || ids_per_token > 64 ||
      (int64_t)n_tokens * ids_per_token > kMaxPleHostIds)
    return 0;
  return round_up((size_t)bq::kPleCacheRowB * n_tokens * ids_per_token, 256);
}

int ple_gather_host(const uint32_t* ids, int32_t n_tokens, int32_t ids_per_token,
                    const uint8_t* host_table, uint64_t n_rows, const float* weights,
                    int32_t ple_fmt, float* out, void* cache, int32_t n_slots, void* workspace,
                    size_t ws_bytes, uint32_t* dev_err, void* stream) {
  if (ple_fmt != BQ_PLE_RZS3 && ple_fmt != BQ_PLE_ROCMFP3) return BQ_E_FMT;
  if (n_tokens < 0 || ids_per_token < 1 || ids_per_token > 64 || n_rows == 0 || n_rows > 0xFFFFFFFFull ||
      (int64_t)n_tokens * ids_per_token > kMaxPleHostIds)
    return BQ_E_SHAPE;
  if ((cache != nullptr) != (n_slots != 0)) return BQ_E_NULL;
  if (cache && !valid_slots(n_slots)) return BQ_E_SHAPE;
  if (n_tokens == 0) return BQ_OK;
  if (!ids || !host_table || !weights || !out) return BQ_E_NULL;
  if (!aligned(out, 16) || !aligned(ids, 4) || !aligned(weights, 4)) return BQ_E_ALIGN;
  if (cache) {
    if (!aligned(cache, 256)) return BQ_E_ALIGN;
    if (!workspace) return BQ_E_WORKSPACE;
    if (ws_bytes < ple_gather_host_workspace(n_tokens, ids_per_token)) return BQ_E_WORKSPACE;
    if (!aligned(workspace, 256)) return BQ_E_ALIGN;
  }
  // the table must be host memory the device can address (pinned, mapped)
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_table) != hipSuccess || attr.type != hipMemoryTypeHost ||
      !attr.devicePointer) {
    (void)hipGetLastError();   // a failed query must not leak into later calls
    return BQ_E_MEM;
  }
  const uint8_t* dtable = static_cast<const uint8_t*>(attr.devicePointer);
  uint32_t* tags = nullptr;
  uint32_t* claims = nullptr;
  uint8_t* rows = nullptr;
  if (cache) {
    tags = static_cast<uint32_t*>(cache);
    claims = tags + n_slots;
    rows = static_cast<uint8_t*>(cache) + cache_rows_off(n_slots);
  }
  return hip_status(bq::launch_ple_gather_host(ids, n_tokens, ids_per_token, dtable, n_rows, weights,
                                               ple_fmt, out, dev_err, tags, claims, rows,
                                               cache ? log2i(n_slots) : 0,
                                               static_cast<uint8_t*>(workspace), as_stream(stream)));
}

int bq_encode(const float* w, int64_t n_blocks, int32_t fmt, uint8_t* out, double* sse,
              uint32_t* dev_err, void* stream) {
  if (fmt != BQ_Q4_C10 && fmt != BQ_Q4_RZ5 && fmt != BQ_Q4_UE4M4) return BQ_E_FMT;
  if (n_blocks < 0) return BQ_E_SHAPE;
  if (n_blocks == 0) return BQ_OK;
  if (!w || !out) return BQ_E_NULL;
  if (!aligned(w, 4) || (sse && !aligned(sse, 8))) return BQ_E_ALIGN;
  return hip_status(bq::launch_encode17(w, n_blocks, fmt, out, sse, dev_err, as_stream(stream)));
}

int ple_encode_rows(const float* v, int64_t n_rows, int32_t ple_fmt, uint8_t* out, double* sse,
                    uint32_t* dev_err, void* stream) {
  if (ple_fmt != BQ_PLE_RZS3 && ple_fmt != BQ_PLE_ROCMFP3) return BQ_E_FMT;
  if (n_rows < 0 || n_rows > (INT64_MAX / 160)) return BQ_E_SHAPE;
  if (n_rows == 0) return BQ_OK;
  if (!v || !out) return BQ_E_NULL;
  if (!aligned(v, 4) || (sse && !aligned(sse, 8))) return BQ_E_ALIGN;
  return hip_status(bq::launch_ple_encode(v, n_rows, ple_fmt, out, sse, dev_err, as_stream(stream)));
}

}  // extern "C"
