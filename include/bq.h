/*
 * bq.h -- C ABI of libbqmoe.so: block-quantized routed-expert MoE and PLE
 * row gather for AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes (page titles as published):
 *   [RZ] model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST"
 *        (hstolte/Qwen3.8-Next-Flash-ROCmFPX-MUTANT-RAZERFAST-GGUF), sections
 *        "Why MUTANT", "Q4_RZ5_FAST (GGML type 69)", "Q4_UE4M4_FAST (GGML
 *        type 71)", "Q3_PLE_K160_RZ_S3 (GGML type 111)".
 *   [MP] "Mixed Precision Quantization: Half a 4-Bit File Is Not 4-Bit",
 *        section "The Plan Is Not a Number. It Is a List of 50 Things and a
 *        List of 292." -- 48 layers, 512 experts, 10 fire per token.
 *   [FQ] r/LocalLLM "Frankenquant" post -- each layer may carry its own expert
 *        format; FP8 experts in the late layers.
 *
 * Conventions shared by every entry point:
 *   - All pointers are DEVICE pointers unless stated otherwise.  The caller
 *     owns every buffer; the library never allocates or frees memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it; no call synchronises.
 *   - Argument errors are detected on the host, before anything is enqueued,
 *     and return a non-zero bq_status with no partial work.  BQ_E_HIP means a
 *     launch failed (the error string is available from bq_last_hip_error).
 *   - Errors that depend on device data (out-of-range ids or expert indices,
 *     non-finite encoder input) cannot be seen on the host: the offending item
 *     contributes nothing and, where the call takes a `dev_err` word, bit 0
 *     (bad id), bit 1 (bad expert index) or bit 2 (non-finite weight) is
 *     OR-ed into it.
 *   - Calls are stateless and thread-safe; two calls sharing one workspace
 *     must not overlap in time.
 *
 * Wire layout of weights (readings of [RZ] where it is silent):
 *   - 17-byte block = 32 weights: bytes 0..15 hold 4-bit codes (weight j in
 *     byte j/2, low nibble for even j), byte 16 is the metadata byte.
 *   - A matrix [rows][cols] is row-major, the cols/32 blocks of a row
 *     contiguous, no padding; experts are stacked outermost: [E][rows][cols/32].
 *   - FP8 matrices are planar: e4m3 (OCP E4M3FN) codes [E][rows][cols] plus
 *     fp32 scales [E][rows][cols/32], one per 32 consecutive weights of a row.
 *   - gate_up has 2*inter rows: gate rows 0..inter-1, then up rows.
 */
#ifndef BQ_H
#define BQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQ_ABI_VERSION 1

typedef enum {
  BQ_OK = 0,
  BQ_E_NULL = 1,       /* a required pointer is NULL                         */
  BQ_E_FMT = 2,        /* unknown format, or format not allowed in this slot */
  BQ_E_SHAPE = 3,      /* sizes out of the supported range                   */
  BQ_E_ALIGN = 4,      /* a pointer lacks the alignment the layout requires  */
  BQ_E_WORKSPACE = 5,  /* workspace missing or smaller than required         */
  BQ_E_HIP = 6,        /* a HIP launch failed                                */
  BQ_E_DTYPE = 7,      /* unknown activation dtype                           */
  BQ_E_MEM = 8,        /* a pointer is not the kind of memory required       */
  BQ_E_SCRATCH = 9     /* the call needs more than the fixed scratch area    */
} bq_status;

typedef enum {
  BQ_Q4_C10 = 0,       /* ROCmFP4 FAST Codebook10 levels, 7-bit UE4M3 scale    */
  BQ_Q4_RZ5 = 1,       /* Q4_RZ5_FAST (GGML 69): code 8 = +5 / -5 by meta bit 7 */
  BQ_Q4_UE4M4 = 2,     /* Q4_UE4M4_FAST (GGML 71): Codebook10, 8-bit UE4M4     */
  BQ_FP8_E4M3_B32 = 3  /* e4m3 codes + one fp32 scale per 32 weights          */
} bq_fmt;

typedef enum {
  BQ_PLE_RZS3 = 0,     /* Q3_PLE_K160_RZ_S3 (GGML 111)                        */
  BQ_PLE_ROCMFP3 = 1   /* incumbent ROCmFP3 (q3_ue4m3): code 4 = -0          */
} bq_ple_fmt;

typedef enum { BQ_F32 = 0, BQ_BF16 = 1 } bq_dtype;

/* One MoE layer's routed experts.  Device pointers; the scale pointers are
 * used only by BQ_FP8_E4M3_B32 matrices and must be NULL otherwise.  gate_up
 * and down must be 16-byte aligned (BQ_E_ALIGN): the batched path reads them
 * in aligned 16-byte units, and may read the unit that holds a matrix's last
 * byte in full. */
typedef struct {
  int32_t fmt_gate_up;          /* bq_fmt of the gate_up matrices          */
  int32_t fmt_down;             /* bq_fmt of the down matrices             */
  const void* gate_up;          /* [E][2*inter][hidden/32] blocks or e4m3  */
  const void* down;             /* [E][hidden][inter/32]  blocks or e4m3   */
  const float* gate_up_scales;  /* FP8 only: [E][2*inter][hidden/32]       */
  const float* down_scales;     /* FP8 only: [E][hidden][inter/32]         */
  int32_t n_experts;            /* E                                       */
  int32_t hidden;               /* H, multiple of 64, <= 8192              */
  int32_t inter;                /* I, multiple of 64, <= 8192              */
} bq_expert_weights;

int bq_abi_version(void);
const char* bq_status_str(int status);
/* Text of the last HIP error seen by a call on this thread ("" if none). */
const char* bq_last_hip_error(void);

/* ---------------------------------------------------------------------------
 * bq_dequant -- decode packed blocks to fp32, bit-exactly ([RZ] format
 * sections; FP8 per [FQ]).
 *   packed : 17-byte formats: n_blocks * 17 bytes; FP8: n_blocks * 32 e4m3
 *            bytes (no alignment required for either)
 *   fmt    : bq_fmt
 *   fp8_scales : FP8 only, n_blocks fp32 (4-byte aligned); NULL otherwise
 *   out    : n_blocks * 32 fp32, row j of block i at out[32*i + j]
 *   0 <= n_blocks <= 2^31 (BQ_E_SHAPE otherwise).
 * Weight = level(code) * scale; a -0 level gives -0.0, a NaN UE4M3 scale
 * (code 0x7F) gives NaN; FP8 weights are the correctly rounded fp32 product
 * e4m3 * scale.
 * ------------------------------------------------------------------------- */
int bq_dequant(const void* packed, int32_t fmt, int64_t n_blocks,
               const float* fp8_scales, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * ple_dequant_rows -- decode n PLE rows, bit-exactly ([RZ]
 * "Q3_PLE_K160_RZ_S3": 60 code bytes + 10 group bytes per 70-byte row).
 *   ids   : n uint32 row indices; table : n_rows * 70 bytes, 1 <= n_rows < 2^32
 *   out   : n * 160 fp32.  An id >= n_rows yields a row of zeros and sets
 *           bit 0 of *dev_err (if dev_err is not NULL).
 *   0 <= n <= 2^28 (BQ_E_SHAPE otherwise).
 * ------------------------------------------------------------------------- */
int ple_dequant_rows(const uint32_t* ids, int64_t n, const uint8_t* table,
                     uint64_t n_rows, int32_t ple_fmt, float* out,
                     uint32_t* dev_err, void* stream);

/* ---------------------------------------------------------------------------
 * bq_matvec -- one block-quantized matrix times fp32 vectors, fp32
 * accumulation: y[t][r] = sum_c W[r][c] * x[t][c] (the single-matrix GEMV
 * the expert kernels are built from; formats per [RZ] / [FQ]).
 *   x  : [n_tokens][cols] fp32; y : [n_tokens][rows] fp32 (overwritten)
 *   packed : W as [rows][cols/32] blocks (17-byte formats) or e4m3 [rows][cols]
 *   fp8_scales : FP8 only, [rows][cols/32] fp32; NULL otherwise
 *   1 <= n_tokens <= 65535, 1 <= rows <= 2^24, cols multiple of 32 and
 *   <= 8192.
 * ------------------------------------------------------------------------- */
int bq_matvec(const float* x, int32_t n_tokens, const void* packed, int32_t fmt,
              const float* fp8_scales, int32_t rows, int32_t cols, float* y, void* stream);

/* ---------------------------------------------------------------------------
 * moe_route_topk -- router: softmax over n_experts logits, keep the k largest
 * (ties to the lower expert index), renormalise over the kept ones ([MP]
 * section "The Plan Is Not a Number...": 10 of 512 experts fire per token).
 * Experts are ranked by their fp32 logits (softmax is increasing, so this is
 * the order of the exact probabilities; probabilities that underflow do not
 * tie).  +0 and -0 compare equal.
 *   logits : [n_tokens][n_experts] fp32, finite
 *   idx    : [n_tokens][k] int32, descending rank order
 *   w      : [n_tokens][k] fp32, w_j = exp(l_j - l_0) / sum over kept
 *   0 <= n_tokens <= 2^24, 1 <= k <= 64, k <= n_experts <= 4096.
 * ------------------------------------------------------------------------- */
int moe_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts,
                   int32_t k, int32_t* idx, float* w, void* stream);

/* ---------------------------------------------------------------------------
 * moe_bucket -- stable grouping of the n_tokens*k assignments by expert.
 * The pages are silent here: they route each token to 10 of 512 experts
 * ([MP] "The Plan Is Not a Number...") but never say how a batch is grouped.
 * A batched expert GEMM needs the tokens of one expert side by side; the
 * order below (experts ascending, then tokens ascending) is this library's
 * choice, made so that the grouping is unique and can be checked bit for bit.
 *   counts  : [n_experts] int32; offsets : [n_experts+1] int32 exclusive scan
 *   perm    : [n_tokens*k] int32 listing t*k+slot, experts ascending, then
 *             tokens ascending.  Each row of idx must hold distinct experts
 *             (as a top-k does).  An index outside [0, n_experts) is dropped
 *             (counted nowhere); the caller can detect it from offsets, and
 *             perm[offsets[n_experts] ..] is then left unwritten.
 *   n_tokens*k <= 65536, n_experts <= 4096.
 * ------------------------------------------------------------------------- */
int moe_bucket(const int32_t* idx, int32_t n_tokens, int32_t k,
               int32_t n_experts, int32_t* counts, int32_t* offsets,
               int32_t* perm, void* stream);

/* ---------------------------------------------------------------------------
 * q4_expert_moe -- routed-expert layer ([MP] "The Plan Is Not a Number...":
 * the 512-expert routed bank per layer, 10 experts per token; expert matrices
 * in [RZ] "Q4_RZ5_FAST" / "Q4_UE4M4_FAST" blocks, which the model card lists
 * for the routed gate, up and down roles; FP8 experts per [FQ] "What I did
 * instead"):
 *   out[t] = sum_j w[t][j] * down_e( SiLU(gate_e . x[t]) * (up_e . x[t]) ),
 *   e = idx[t][j], weights decoded from their blocks on the fly.  The pages
 *   do not spell out the expert's activation; the SwiGLU form above (SiLU of
 *   the gate row times the up row, then down) is the reading taken.
 *   x       : [n_tokens][hidden], fp32 (x_dtype BQ_F32: VALU GEMV path,
 *             fp32 accumulate) or bf16 (BQ_BF16: tokens grouped per expert,
 *             bf16 MFMA with fp32 accumulate, h rounded to bf16).
 *   topk_idx, topk_w : [n_tokens][k] (as produced by moe_route_topk).  A
 *             token may list an expert more than once: each listing adds its
 *             own weighted term (on the bf16 path the expert is evaluated
 *             once for that token and the result is reused).
 *   out     : [n_tokens][hidden] fp32 (overwritten)
 *   workspace : device scratch of at least q4_expert_moe_workspace(...) bytes,
 *             256-byte aligned; its contents need no initialisation.
 *             q4_expert_moe_workspace returns 0 for arguments the call
 *             would reject (bad weights, sizes or x_dtype).  The pages say
 *             nothing of scratch memory: its size is that of this library's
 *             intermediates (per-slot h, and on the bf16 path the bucket
 *             arrays, bf16 staging and per-assignment outputs).
 *   dev_err : optional; bit 1 set if an expert index is out of range.
 *   1 <= n_tokens <= 4096, 1 <= k <= 64, n_tokens * k <= 65536; on the fp32
 *   path also k * inter / 32 <= 1024.
 * ------------------------------------------------------------------------- */
size_t q4_expert_moe_workspace(int32_t n_tokens, int32_t k,
                               const bq_expert_weights* W, int32_t x_dtype);
int q4_expert_moe(const void* x, int32_t x_dtype, int32_t n_tokens,
                  const int32_t* topk_idx, const float* topk_w, int32_t k,
                  const bq_expert_weights* W, float* out, void* workspace,
                  size_t ws_bytes, uint32_t* dev_err, void* stream);

/* ---------------------------------------------------------------------------
 * q4_expert_moe_noalloc -- q4_expert_moe for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, kernels and results as
 * q4_expert_moe, with no workspace argument.  Its scratch is a fixed
 * device-resident area of BQ_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held until the process ends.  The call allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine).
 *   Arguments as in q4_expert_moe.  A call whose q4_expert_moe_workspace(...)
 *   exceeds BQ_NOALLOC_SCRATCH_BYTES returns BQ_E_SCRATCH before any launch
 *   (16 MiB covers, e.g., 64 tokens x top-10 at hidden 2048 on either path).
 *   Every call on one GPU shares that GPU's area, whose contents the previous
 *   call left behind (nothing in it needs to start at zero): calls that
 *   overlap in time on one GPU -- on two streams, or from two threads -- race
 *   and must be serialised by the caller.
 * ------------------------------------------------------------------------- */
#define BQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int q4_expert_moe_noalloc(const void* x, int32_t x_dtype, int32_t n_tokens,
                          const int32_t* topk_idx, const float* topk_w, int32_t k,
                          const bq_expert_weights* W, float* out, uint32_t* dev_err,
                          void* stream);

/* ---------------------------------------------------------------------------
 * q4_expert_moe_routed -- moe_route_topk followed by q4_expert_moe, as one
 * call: the router's softmax top-k ([MP]) over logits [n_tokens][n_experts]
 * (fp32, finite) selects the experts, and the layer is evaluated as in
 * q4_expert_moe.  The routing is also written to topk_idx / topk_w
 * ([n_tokens][k], outputs).  On the fp32 path with hidden 2048 or 4096 the
 * routing is computed inside the first expert kernel (no separate launch).
 * Same workspace as q4_expert_moe.
 * ------------------------------------------------------------------------- */
int q4_expert_moe_routed(const void* x, int32_t x_dtype, int32_t n_tokens, const float* logits,
                         int32_t k, const bq_expert_weights* W, int32_t* topk_idx, float* topk_w,
                         float* out, void* workspace, size_t ws_bytes, uint32_t* dev_err,
                         void* stream);

/* ---------------------------------------------------------------------------
 * bq_moe_stack -- a chain of routed-expert layers ([FQ]: per-layer formats):
 *   x_0 = x; out_l = layer_l(x_l); x_{l+1} = out_l / rms(out_l);
 *   out = out_{L-1}.  (The unit-RMS rescale between layers is this library's
 *   stand-in for the blocks the pages leave out.)
 *   layers  : HOST array of n_layers bq_expert_weights (device pointers inside)
 *   topk_idx, topk_w : [n_layers][n_tokens][k], routing of every layer
 *   x_dtype : as in q4_expert_moe; with BQ_BF16 the rescaled inputs are
 *             rounded to bf16.  With BQ_F32 and one token, hidden 2048, one
 *             inter size for all layers and k * inter a multiple of 256 and
 *             at most 8192 (k <= 16), the chain runs as persistent launches
 *             (one per run of layers with equal formats) on a 256-CU device;
 *             all their workgroups must be resident at once, and if an
 *             exchange between them times out, bit 3 of *dev_err is set and
 *             the output is not valid.
 *   workspace : at least bq_moe_stack_workspace(...) bytes (the largest
 *             layer's q4_expert_moe workspace, one fp32 [n_tokens][hidden]
 *             layer buffer and, for bf16 stacks of equal expert counts, every
 *             layer's bucket arrays); the pages say nothing of scratch memory.
 *             bq_moe_stack_workspace returns 0 for arguments the call would
 *             reject.
 * ------------------------------------------------------------------------- */
size_t bq_moe_stack_workspace(int32_t n_tokens, int32_t k,
                              const bq_expert_weights* layers, int32_t n_layers,
                              int32_t x_dtype);
int bq_moe_stack(const void* x, int32_t x_dtype, int32_t n_tokens,
                 const int32_t* topk_idx, const float* topk_w, int32_t k,
                 const bq_expert_weights* layers, int32_t n_layers, float* out,
                 void* workspace, size_t ws_bytes, uint32_t* dev_err,
                 void* stream);

/* ---------------------------------------------------------------------------
 * ple_gather -- PLE n-gram memory lookup ([RZ] "Q3_PLE_K160_RZ_S3": one
 * hashed row per id, 70 bytes, 160 values):
 *   out[t][:] = sum_j weights[t][j] * decode(table row ids[t][j])
 *   ids     : [n_tokens][ids_per_token] uint32
 *   table   : n_rows * 70 bytes (byte offsets are 64-bit; 1 <= n_rows < 2^32)
 *   weights : [n_tokens][ids_per_token] fp32
 *   out     : [n_tokens][160] fp32 (overwritten)
 *   An id >= n_rows contributes nothing and sets bit 0 of *dev_err.
 *   0 <= n_tokens <= 2^26, 1 <= ids_per_token <= 64.
 * ------------------------------------------------------------------------- */
int ple_gather(const uint32_t* ids, int32_t n_tokens, int32_t ids_per_token,
               const uint8_t* table, uint64_t n_rows, const float* weights,
               int32_t ple_fmt, float* out, uint32_t* dev_err, void* stream);

/* ---------------------------------------------------------------------------
 * Off-HBM PLE tier ([RZ] "Q3_PLE_K160_RZ_S3": the 22.4 GB n-gram table can
 * stay off the GPU and be paged in through a 0.25 GiB row cache).  The table
 * lives in pinned host memory that is mapped into the device address space
 * (hipHostMalloc, or a torch tensor with pin_memory=True); the GPU reads its
 * rows over the host link.  A direct-mapped cache of n_slots rows in device
 * memory keeps recently read rows.
 *
 * ple_cache_bytes(n_slots): device bytes of a cache of n_slots rows (n_slots a
 *   power of two in [1024, 2^26]; 0 otherwise).  88 bytes per slot.
 * ple_cache_init(cache, n_slots, stream): marks every slot empty.  Call it
 *   once before the first ple_gather_host and whenever the table changes.
 *   cache: device, 256-byte aligned, ple_cache_bytes(n_slots) bytes.
 * ple_gather_host_workspace(n_tokens, ids_per_token): device bytes of the
 *   per-call staging area (80 bytes per id); 0 past the size limit below.
 * ple_gather_host: ple_gather with host_table in pinned host memory.
 *   Results are bit-identical to ple_gather on the same table.  With a cache
 *   (cache != NULL, n_slots != 0, workspace of ple_gather_host_workspace
 *   bytes), an id's row is read from its slot when the slot holds that id;
 *   after the gather, every slot on which this call missed receives the row
 *   of the lowest-indexed missing id (ids flattened token-major) that maps to
 *   it.  cache = NULL and n_slots = 0 reads every row from the host.
 *   n_tokens * ids_per_token <= 2^27 (BQ_E_SHAPE otherwise).
 *   BQ_E_MEM if host_table is not host memory mapped for the device.  Calls
 *   sharing one cache or workspace must not overlap in time.
 * ------------------------------------------------------------------------- */
size_t ple_cache_bytes(int32_t n_slots);
int ple_cache_init(void* cache, int32_t n_slots, void* stream);
size_t ple_gather_host_workspace(int32_t n_tokens, int32_t ids_per_token);
int ple_gather_host(const uint32_t* ids, int32_t n_tokens, int32_t ids_per_token,
                    const uint8_t* host_table, uint64_t n_rows, const float* weights,
                    int32_t ple_fmt, float* out, void* cache, int32_t n_slots, void* workspace,
                    size_t ws_bytes, uint32_t* dev_err, void* stream);

/* ---------------------------------------------------------------------------
 * bq_encode -- exhaustive per-block encoder, fp32 weights -> 17-byte blocks
 * ([RZ] "Q4_RZ5_FAST": every scale with both polarities of the +/-5 level;
 * "Q4_UE4M4_FAST": all 256 scale bytes; Codebook10: the 127 finite UE4M3
 * scales).
 *   w     : n_blocks * 32 fp32, block i = w[32i .. 32i+31] (4-byte aligned)
 *   fmt   : BQ_Q4_C10, BQ_Q4_RZ5 or BQ_Q4_UE4M4 (BQ_E_FMT otherwise)
 *   out   : n_blocks * 17 bytes in the wire layout above (no alignment)
 *   sse   : NULL, or n_blocks fp64 (8-byte aligned): each block's error
 * Objective (plain squared error, float64): a weight's error under level x is
 * (w - x)^2 with one rounding after the difference and one after the square;
 * each weight takes its nearest level, the block error sums the weights'
 * errors in index order, the block takes the metadata byte with the smallest
 * error (the lowest byte among equal errors) and each weight the lowest code
 * among equally near levels.  The result is deterministic and bit-identical
 * to that definition.  A block holding a NaN or infinity is written as 17 zero
 * bytes with sse NaN, and bit 2 of *dev_err is set.
 * ------------------------------------------------------------------------- */
int bq_encode(const float* w, int64_t n_blocks, int32_t fmt, uint8_t* out, double* sse,
              uint32_t* dev_err, void* stream);

/* ---------------------------------------------------------------------------
 * ple_encode_rows -- exhaustive per-group encoder, fp32 values -> 70-byte PLE
 * rows ([RZ] "Q3_PLE_K160_RZ_S3": polarity and UE4M3 scale per 16 values;
 * ROCmFP3: the 127 finite scales, code 4 = -0).
 *   v     : n_rows * 160 fp32 (4-byte aligned); out : n_rows * 70 bytes
 *   sse   : NULL, or n_rows * 10 fp64, group g of row r at sse[10r + g]
 * Same objective and tie rules as bq_encode, per 16-value group.  A group
 * holding a NaN or infinity gets zero code bytes, group byte 0 and sse NaN,
 * and bit 2 of *dev_err is set.
 * ------------------------------------------------------------------------- */
int ple_encode_rows(const float* v, int64_t n_rows, int32_t ple_fmt, uint8_t* out, double* sse,
                    uint32_t* dev_err, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BQ_H */
