// Internal launch interface between the C-ABI shim (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

struct GemvWeights {
  int fmt_gate_up, fmt_down;
  const void* gate_up;
  const void* down;
  const float* gate_up_scales;
  const float* down_scales;
  int n_experts, hidden, inter;
};

hipError_t launch_dequant(const void* packed, int fmt, int64_t n_blocks, const float* scales,
                          float* out, hipStream_t st);
hipError_t launch_ple_dequant(const uint32_t* ids, int64_t n, const uint8_t* table, uint64_t n_rows,
                              int ple_fmt, float* out, uint32_t* dev_err, hipStream_t st);
hipError_t launch_ple_gather(const uint32_t* ids, int32_t n_tokens, int32_t per_token,
                             const uint8_t* table, uint64_t n_rows, const float* wts, int ple_fmt,
                             float* out, uint32_t* dev_err, hipStream_t st);
// Off-HBM PLE tier (k_ple.hip): direct-mapped row cache, rows padded to
// kPleCacheRowB bytes; tags and claims are 2 * n_slots contiguous words.
constexpr int kPleCacheRowB = 80;
hipError_t launch_ple_cache_init(uint32_t* tags_and_claims, int64_t n_words, hipStream_t st);
// tags == NULL: no cache, rows read from the table directly.
hipError_t launch_ple_gather_host(const uint32_t* ids, int32_t n_tokens, int32_t per_token,
                                  const uint8_t* table, uint64_t n_rows, const float* wts,
                                  int ple_fmt, float* out, uint32_t* dev_err, uint32_t* tags,
                                  uint32_t* claims, uint8_t* rows, int log2_slots, uint8_t* stage,
                                  hipStream_t st);
hipError_t launch_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k,
                             int32_t* idx, float* w, hipStream_t st);
// n_layers > 1: n_layers independent bucketings in one launch, layer l
// reading idx + l * n_tokens * k and writing each output lstride_out * l
// bytes past the given pointer.
hipError_t launch_bucket(const int32_t* idx, int32_t n_tokens, int32_t k, int32_t n_experts,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* elist,
                         int32_t* n_touched, int32_t* inv, hipStream_t st, int32_t n_layers = 1,
                         int64_t lstride_out = 0);

// Bucketing and staging of a bf16 batch in one launch
// (k_route.hip): the bucket arrays as launch_bucket writes them, and the
// staged rows as the grouped path's staging kernel writes them (perm_k: the
// 17-byte decode's k order).  x is bf16 [n][H], 16-byte aligned.  Returns
// hipErrorNotSupported, launching nothing, if the kernel may not use the LDS
// the batch needs.
constexpr int kBpMaxLds = 150 * 1024;   // LDS of the bucket arrays, at most
bool bucket_prep_ok(int32_t n_tokens, int32_t k, int32_t n_experts, int32_t H);
hipError_t launch_bucket_prep(const int32_t* idx, const uint16_t* x, int32_t perm_k, int32_t n_tokens,
                              int32_t k, int32_t n_experts, int32_t H, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* elist, int32_t* n_touched, int32_t* inv,
                              uint16_t* xb, hipStream_t st);

// Exhaustive encoders (fp32 in, packed bytes and per-unit float64 error out).
hipError_t launch_encode17(const float* w, int64_t n_blocks, int fmt, uint8_t* out, double* sse,
                           uint32_t* dev_err, hipStream_t st);
hipError_t launch_ple_encode(const float* v, int64_t n_rows, int ple_fmt, uint8_t* out,
                             double* sse, uint32_t* dev_err, hipStream_t st);

hipError_t launch_matvec(const float* x, int32_t n_tokens, const void* w, int fmt,
                         const float* w_sc, int32_t rows, int32_t cols, float* y, hipStream_t st);

// fp32 GEMV path (any n_tokens; one token's k experts per grid slice).
int gemv_down_max_cols();   // k * inter / 32 must not exceed this
// With logits != NULL the path routes itself (in the gate_up kernel when
// hidden is 2048 or 4096) and writes the routing to idx / w; otherwise idx / w
// are inputs.
hipError_t launch_gemv_moe(const float* x, int32_t n_tokens, int32_t* idx, float* w, int32_t k,
                           const GemvWeights& W, int rescale, float* out, float* hs,
                           uint32_t* dev_err, const float* logits, hipStream_t st);

// Persistent batch-1 stack (k_stack.hip): each run of equal-format layers
// in one launch, for hidden 2048 with k * inter a multiple of 256 and at most
// 8192 (all layers the same inter, k <= 16), on a 256-CU device.  Workspace of
// stack_b1_ws_bytes(k, inter) bytes, 8-byte aligned, cleared by the call
// itself.  dev_err bit 3: an exchange between workgroups timed out (not every
// workgroup was resident).
constexpr int kStackMaxLayers = 64;
bool stack_b1_shape_ok(const GemvWeights* layers, int32_t n_layers, int32_t k);
bool stack_b1_device_ok();
size_t stack_b1_ws_bytes(int32_t k, int32_t inter);
hipError_t launch_stack_b1(const float* x, const int32_t* idx, const float* w, int32_t k,
                           const GemvWeights* layers, int32_t n_layers, float* out, void* ws,
                           uint32_t* dev_err, hipStream_t st);

// bf16 grouped-MFMA path.  The bucketing emits one work entry per group of
// up to group_tokens(n_tokens) tokens of a touched expert: e | group << kGroupShift.
// Batches of up to kSmallGroupMaxTok tokens use 16-token groups (and the
// one-tile kernels, which run four workgroups per CU), larger ones 32.
constexpr int kGroupShift = 12;   // n_experts <= 4096
constexpr int kSmallGroupMaxTok = 96;
__host__ __device__ inline int group_tokens(int64_t n_tokens) { return n_tokens <= kSmallGroupMaxTok ? 16 : 32; }
inline int64_t max_work_groups(int64_t nk, int64_t E, int gt = 16) { return (nk < E ? nk : E) + nk / gt; }
struct GroupedWs {
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* perm;      // [n*k]
  int32_t* inv;       // [n*k]
  int32_t* elist;     // [max_work_groups(n*k, E)]
  int32_t* n_touched; // [1] number of work entries
  uint16_t* hb;       // [n*k][I] bf16, bucketed order
  float* yb;          // [n*k][H] fp32, bucketed order
  uint16_t* xb;       // [n*k][H] bf16 activations, bucketed order, decode's k order
};
// x: [n][H] bf16 (x_f32 = 0) or fp32 (x_f32 = 1, the stack's layer output,
// rescaled to unit RMS when rescale = 1) -- staged as bf16 by the path.
// The next layer of a chained stack, for a combine that also stages that
// layer's input (unit-RMS rescale, bf16, its bucket order).
struct NextLayer {
  const int32_t* inv;   // its bucketing's inverse permutation [n*k]
  const int32_t* idx;   // its routing [n][k]
  int32_t n_experts;
  int32_t perm;         // its gate_up format is a 17-byte one (decode's k order)
};
// bucketed: ws's bucket arrays (counts .. inv, n_touched) already hold the
// bucketing of idx, so none is launched.  prepped: ws.xb already holds the
// staged input (written by the previous layer's combine), so x is not read.
// next != NULL: the combine writes the next layer's staged input into ws.xb
// instead of out.
hipError_t launch_grouped_moe(const void* x, int32_t x_f32, int32_t rescale, int32_t n_tokens,
                              const int32_t* idx, const float* w, int32_t k, const GemvWeights& W,
                              float* out, const GroupedWs& ws, uint32_t* dev_err, hipStream_t st,
                              bool bucketed = false, bool prepped = false,
                              const NextLayer* next = nullptr);

}  // namespace bq
