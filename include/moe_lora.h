/* moe_lora.h -- C ABI of the fused MoE-LoRA layer for AMD MI355X (gfx950).
 *
 * The layer (vLLM blog "Multi-LoRA for MoE models", vllm.com.cn, 2026-02-26,
 * section "Implementing multi-LoRA inference for MoE models in vLLM",
 * Figure 1 and the equation y = xW + xAB): every token t is routed to topk
 * experts with weights w[t][j] and carries the adapter id of its request.
 * For each routed pair (t, e) with adapter l:
 *     g  = x[t] W_gu[e]  + s * (x[t] A_gu[l][e]) B_gu[l][e]      (gate_up, 2I wide)
 *     h  = silu(g[0:I]) * g[I:2I]                                 (SiLU gate)
 *     d  = h W_down[e]   + s * (h A_down[l][e]) B_down[l][e]      (down, H wide)
 *     y[t] = sum_j w[t][j] * d(t, e_j)                            (top-k combine)
 * The products with A are the LoRA "shrink" ops (h_in -> r) and the products
 * with B the "expand" ops (r -> h_out), four per expert (same section).  The
 * adapter is skipped for tokens whose id is -1.
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; `stream` is a hipStream_t (NULL = default stream).
 *   - Calls that take a stream are asynchronous: host-side checks run first
 *     and return an error code WITHOUT launching anything; otherwise the work
 *     is enqueued and the call returns MOE_LORA_OK.  Nothing allocates device
 *     memory; all scratch lives in the caller's workspace.
 *   - The caller owns every buffer and must keep it alive until the stream
 *     has passed the call.  Two calls that share a workspace must be ordered
 *     on one stream.
 *   - bf16 tensors are passed as uint16_t bit patterns.  Weights are stored
 *     with the reduction index contiguous, i.e. as the transposes of the
 *     pages' h_in x h_out matrices:
 *         W_gu   [E][2I][H]    rows 0..I-1 = gate, rows I..2I-1 = up
 *         W_down [E][H][I]
 *         A_gu   [L][E][r][H]      B_gu   [L][E][2I][r]
 *         A_down [L][E][r][I]      B_down [L][E][H][r]
 *   - H, I and r must be multiples of 8 and every tensor pointer 16-byte
 *     aligned (whole 16-byte vector loads).
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_LORA_OK 0
#define MOE_LORA_EINVAL (-1)       /* null pointer, negative or zero size, topk > E, bad block_m */
                                   /* or kernel configuration field                              */
#define MOE_LORA_EALIGN (-2)       /* pointer not 16-byte aligned, H or I not a multiple of 8    */
#define MOE_LORA_EWORKSPACE (-3)   /* workspace smaller than moe_lora_workspace_bytes()          */
#define MOE_LORA_EUNSUPPORTED (-4) /* r not a multiple of 8 or r > 128; E*(L+1) > 14336; x or the  */
                                   /* intermediate h ((T*topk + E*255) x I bf16) of 2 GiB or more;  */
                                   /* one expert's gate_up weights of 2^32 elements or more         */
#define MOE_LORA_EHIP (-5)         /* a HIP runtime call or kernel launch failed                 */

/* Layer sizes.  T may be 0 (every call is then a no-op). */
typedef struct moe_lora_shape {
  int32_t T;        /* tokens                                                     */
  int32_t H;        /* hidden size: h_in of gate_up, h_out of down                */
  int32_t I;        /* per-expert intermediate size; gate_up produces 2I values   */
  int32_t E;        /* experts                                                    */
  int32_t topk;     /* experts per token, 1 <= topk <= E                          */
  int32_t L;        /* adapters resident in the A/B stacks (>= 1)                 */
  int32_t r;        /* adapter rank                                               */
  int32_t block_m;  /* rows per block shared by every op of the layer: one of     */
                    /* 16, 32, 64, 128, 192, 256, or 0 to choose it from shape    */
  float lora_scale; /* s above                                                    */
  /* Kernel configuration; 0 in any field = the library's choice for the shape.
   * moe_lora_tune_apply fills them from a tuning table (an offline sweep).    */
  int32_t shrink_splits;  /* K splits of both shrinks, 1..64 (several: partial   */
                          /* sums added with fp32 atomics)                       */
  int32_t shrink_zblocks; /* work items per shrink tile across the r columns:    */
                          /* 1 (all r), or 2..r/8 dividing r into multiples of 8 */
  int32_t down_splits;    /* K splits of the streaming down GEMM (the one that   */
                          /* runs for block_m <= 32 or I >= 4096), 1..64 (at     */
                          /* most I / 128 are used)                              */
  int32_t tile_order;     /* workgroup order of the LDS-tiled GEMMs: 1 = row     */
                          /* tile-major; 2 = each row tile's column tiles on one */
                          /* XCD, row tiles interleaved over the 8 XCDs;         */
                          /* 0 = 1 for gate_up and 2 for down                    */
  int32_t expand_mode;    /* LoRA expand of the LDS-tiled GEMMs (block_m >= 64): */
                          /* 2 = as extra K stages through the LDS ring over the */
                          /* (expert, adapter) segments meeting a row tile (64   */
                          /* ranks of one segment per stage, or 8/(r/8) segments */
                          /* side by side when r < 64), taken where L <= 64 and  */
                          /* the GEMM's K is a multiple of 64 (the register form */
                          /* runs elsewhere); 1 = masked MFMAs on the            */
                          /* accumulators from z and B in registers; 0 = 2 where */
                          /* r >= 32 and 2 is taken, else 1                      */
} moe_lora_shape;

/* Device pointers into a workspace (see moe_lora_workspace_view). */
typedef struct moe_lora_views {
  int32_t* sorted_ids;   /* [cap_rows] pair id p = t*topk + j per row; sentinel P = T*topk   */
  int32_t* expert_off;   /* [E+1] first row of each expert's run (runs padded to block_m)    */
  int32_t* seg_start;    /* [E*(L+1)] first row of (expert e, slot s) at e*(L+1)+s; slot = l  */
  int32_t* seg_cnt;      /* [E*(L+1)] pairs in that segment; slot L = tokens without adapter */
  int32_t* block_expert; /* [cap_blocks] expert of each block_m-row block, -1 when unused    */
  int32_t* pos_of_pair;  /* [T*topk] row of each pair, -1 when its expert id is invalid      */
  int32_t* num_padded;   /* [1] rows in use = expert_off[E]                                  */
  int32_t* err_count;    /* [1] invalid expert ids (per pair) + invalid adapter ids (per token) */
  float* z_gu;           /* [cap_rows][r] gate_up shrink result per row (adapter rows only)  */
  float* z_down;         /* [cap_rows][r] down shrink result per row (adapter rows only)     */
  uint16_t* h;           /* [cap_rows][I] bf16 SiLU-gate output per row                      */
  float* d;              /* [d_splits][cap_rows][H] down output per row, already times       */
                         /* w[t][j]; with several K splits the row's output is the sum of  */
                         /* its slabs (the combine adds them in slab order)                */
  int64_t cap_rows;      /* T*topk + E*(block_m-1)                                           */
  int64_t cap_blocks;    /* ceil(cap_rows / block_m)                                         */
  int32_t block_m;       /* block size in effect (resolved when the shape says 0)           */
  int32_t d_splits;      /* K splits of the down GEMM (1 unless few experts, wide weights)  */
  uint16_t* h_lo;        /* [cap_rows][I] bf16 remainder h - rne(h) when I >= 4096, else NULL */
} moe_lora_views;

/* Device pointers to the align outputs inside a workspace (see
 * moe_lora_align_view); the same regions as the first eight moe_lora_views
 * fields, read-only. */
typedef struct moe_lora_align_ptrs {
  const int32_t* sorted_ids;   /* [cap_rows]                                              */
  const int32_t* expert_off;   /* [E+1]                                                   */
  const int32_t* seg_start;    /* [E*(L+1)]                                               */
  const int32_t* seg_cnt;      /* [E*(L+1)]                                               */
  const int32_t* block_expert; /* [cap_blocks]                                            */
  const int32_t* pos_of_pair;  /* [T*topk]                                                */
  const int32_t* num_padded;   /* [1]                                                     */
  const int32_t* err_count;    /* [1]                                                     */
} moe_lora_align_ptrs;

/* Opaque stage-timing recorder owned by the caller (moe_lora_profiler_create). */
typedef struct moe_lora_profiler moe_lora_profiler;

/* block_m used for this shape (the shape's own value when non-zero), or a
 * negative status when the shape is invalid.  Host only, pure. */
int moe_lora_resolve_block_m(const moe_lora_shape* shape);

/* One entry of a tile-configuration table, the result of an offline sweep
 * (the pages' tuned kernel configurations per shape: "Multi-LoRA for MoE
 * models", section "Tuning kernel configurations for Amazon SageMaker AI and
 * Amazon Bedrock").  Key: the shape class, with
 * rows_per_expert = ceil(T*topk / min(E, T*topk)) of the swept shape; value:
 * the block_m measured fastest for it. */
typedef struct {
  int32_t rows_per_expert, H, I, E, r, L; /* key */
  int32_t block_m;                        /* value: 16, 32, 64, 128, 192 or 256 */
  int32_t shrink_splits, shrink_zblocks, down_splits, tile_order; /* value: as in    */
                                          /* moe_lora_shape (0 = the library's choice) */
  int32_t expand_mode;                    /* likewise                                  */
} moe_lora_tune_entry;

/* block_m for `shape` chosen from a tuning table: the shape's own block_m
 * when it is non-zero; otherwise the block_m of the nearest entry, where the
 * distance is the sum over the key fields of |log2(shape value / entry
 * value)|, rows_per_expert counted four times (ties: the earlier entry),
 * provided that distance is at most max_dist (max_dist <= 0: no limit) and
 * the shape's workspace layout is valid with that block_m; otherwise the
 * built-in choice (moe_lora_resolve_block_m).  Entries with a block_m
 * outside {16, 32, 64, 128, 192, 256} or a non-positive key field are
 * skipped.
 * table may be NULL when n == 0.  Returns a negative status when the shape
 * is invalid.  Host only, pure: the table is read, not kept. */
int moe_lora_tune_block_m(const moe_lora_shape* shape, const moe_lora_tune_entry* table, int32_t n,
                          float max_dist);

/* The whole configuration from a tuning table: *out = *shape with block_m and
 * the five knobs taken from the entry moe_lora_tune_block_m would pick (same
 * distance, limit and validity rules; the shape's own non-zero fields win
 * field by field).  With no entry in range *out = *shape.  Returns the
 * block_m in effect, or a negative status (invalid shape, null out).  Host
 * only, pure. */
int moe_lora_tune_apply(const moe_lora_shape* shape, const moe_lora_tune_entry* table, int32_t n,
                        float max_dist, moe_lora_shape* out);

/* Bytes of device workspace that moe_lora_align / moe_lora_forward need for
 * this shape, or 0 when the shape is invalid.  Host only, pure. */
size_t moe_lora_workspace_bytes(const moe_lora_shape* shape);

/* (expert, adapter) align: a stable counting sort of the T*topk (token, slot)
 * pairs by key (expert, adapter slot), slot = adapter id or L for "no
 * adapter".  Each expert's pairs form one run, adapter groups within it are
 * contiguous segments in adapter order (no-adapter last), pairs keep
 * ascending p = t*topk + j inside a segment, and each run is padded to a
 * multiple of block_m with the sentinel T*topk.  One block size is shared by
 * every op of the layer (vLLM blog, section "Tuning kernel configurations for
 * Amazon SageMaker AI and Amazon Bedrock": the four LoRA ops share
 * BLOCK_SIZE_M).  The adapter dimension of the sort is the pages' extra grid
 * dimension over active adapters (section "Implementing multi-LoRA ...").
 *
 *   topk_ids  device [T][topk] int32 expert ids; ids outside [0,E) drop the pair
 *   lora_ids  device [T] int32 adapter ids; -1 = none; ids outside [-1,L) are
 *             treated as none
 *   workspace device, ws_bytes >= moe_lora_workspace_bytes(shape)
 * Writes the align outputs into the workspace (bit-exact, deterministic) and
 * clears the shrink accumulators.  Invalid ids are counted (see
 * moe_lora_device_errors), never fatal. */
int moe_lora_align(const moe_lora_shape* shape, const int32_t* topk_ids, const int32_t* lora_ids,
                   void* workspace, size_t ws_bytes, void* stream);

/* Router: each token's top-k experts and their weights from fp32 logits.
 * The router sends each token to its top-k experts and the layer aggregates
 * their outputs (vLLM blog, section "Implementing multi-LoRA inference for MoE
 * models in vLLM"); the pages fix neither tie order nor weight formula.  This
 * library: experts by descending logit, equal logits by ascending expert index
 * (slot j = j-th choice, bit-exact); weights = softmax over the k chosen
 * logits (fp32), i.e. the full softmax's top-k probabilities renormalised.
 *
 *   logits        device [T][E] fp32.  A non-finite logit (NaN, +inf, -inf)
 *                 is never chosen; a slot left without a finite logit gets
 *                 expert -1 and weight 0 (the align counts and drops it) and
 *                 the chosen experts share the weight.
 *   topk_ids      device [T][topk] int32, written
 *   topk_weights  device [T][topk] fp32, written
 * shape->topk must be at most 64 (MOE_LORA_EUNSUPPORTED otherwise).  Async on
 * stream; the outputs feed moe_lora_align / moe_lora_forward. */
int moe_lora_route(const moe_lora_shape* shape, const float* logits, int32_t* topk_ids,
                   float* topk_weights, void* stream);

/* moe_lora_route followed by moe_lora_align on the routed ids, fused into a
 * single kernel when T*topk <= 256 (decode batches) and the align's tables
 * fit in LDS; otherwise the router kernel runs first.  Arguments as in the two
 * calls; topk_ids and topk_weights are written and the workspace receives the
 * align outputs. */
int moe_lora_route_align(const moe_lora_shape* shape, const float* logits, const int32_t* lora_ids,
                         int32_t* topk_ids, float* topk_weights, void* workspace, size_t ws_bytes,
                         void* stream);

/* Typed device pointers into `workspace` for this shape (host only, no GPU
 * work).  For tests and tools that inspect the align or intermediates. */
int moe_lora_workspace_view(const moe_lora_shape* shape, void* workspace, moe_lora_views* out);

/* Device pointers to the align outputs in `workspace` for this shape (host
 * only, no GPU work, nothing is read): sorted_ids, expert_off, seg_start,
 * seg_cnt, block_expert, pos_of_pair, num_padded, err_count as written by
 * moe_lora_align (layouts in moe_lora_views).  MOE_LORA_EINVAL for a null
 * workspace or out, or an invalid shape's status. */
int moe_lora_align_view(const moe_lora_shape* shape, const void* workspace, moe_lora_align_ptrs* out);

/* The layer forward.  Requires a preceding moe_lora_align with the same
 * shape, ids and workspace on the same stream, and each forward needs an
 * align of its own: the align clears the shrink accumulators in the
 * workspace, and a forward whose shrinks split K adds into them, so a second
 * forward after the same align would add the adapters' shrink results twice.
 *   x            device [T][H] bf16
 *   topk_ids     device [T][topk] int32 (as given to the align)
 *   topk_weights device [T][topk] float
 *   lora_ids     device [T] int32 (as given to the align)
 *   W_gu, W_down, A_gu, B_gu, A_down, B_down   device bf16, layouts above
 *   y            device [T][H] bf16 output, overwritten (round to nearest even)
 * Accumulation is fp32 everywhere; the gate_up result stays fp32 through the
 * SiLU; h is stored bf16, and from I = 4096 on also as its bf16 remainder
 * (h - rne(h)), which the down GEMM multiplies too (a down GEMM that deep
 * then runs on 16- or 32-row tiles whatever block_m is).  With split-K
 * shrinks the fp32 sums are added with atomics, so y may differ between runs
 * in the last bits. */
int moe_lora_forward(const moe_lora_shape* shape, const uint16_t* x, const int32_t* topk_ids,
                     const float* topk_weights, const int32_t* lora_ids, const uint16_t* W_gu,
                     const uint16_t* W_down, const uint16_t* A_gu, const uint16_t* B_gu,
                     const uint16_t* A_down, const uint16_t* B_down, void* workspace,
                     size_t ws_bytes, uint16_t* y, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): align +
 * forward in one call, with the workspace in a static device array of
 * MOE_LORA_NOALLOC_WORKSPACE_BYTES that the library holds on each GPU it
 * runs on until the process ends.  Arguments as in moe_lora_forward (the
 * caller still owns x, the ids, the weights and y); the same kernels and
 * results as moe_lora_align + moe_lora_forward.  Returns
 * MOE_LORA_EWORKSPACE, without launching anything, when the shape's
 * workspace (moe_lora_workspace_bytes) exceeds that size -- decode batches
 * and the GPT-OSS-20B-like layer fit, a 2048-token prefill does not.  Calls
 * no allocating routine.  Every call on one GPU uses that GPU's one array:
 * calls that overlap on a GPU (two streams, two host threads) race and give
 * wrong results; order them on one stream.  The invalid-id count of these
 * calls is not exposed (moe_lora_device_errors needs a caller workspace). */
#define MOE_LORA_NOALLOC_WORKSPACE_BYTES (64u << 20)
int moe_lora_forward_noalloc(const moe_lora_shape* shape, const uint16_t* x, const int32_t* topk_ids,
                             const float* topk_weights, const int32_t* lora_ids, const uint16_t* W_gu,
                             const uint16_t* W_down, const uint16_t* A_gu, const uint16_t* B_gu,
                             const uint16_t* A_down, const uint16_t* B_down, uint16_t* y,
                             void* stream);

/* Number of invalid ids the last align on `workspace` met.  Synchronises
 * `stream` (the only call here that waits for the GPU). */
int moe_lora_device_errors(const moe_lora_shape* shape, const void* workspace,
                           int32_t* host_count, void* stream);

/* Human-readable name of a status code (static string). */
const char* moe_lora_status_str(int status);

/* Stage timing with HIP events, for benchmarks and tools.  The recorder is
 * the caller's object: moe_lora_profiler_create makes one for up to
 * max_calls align+forward calls, recording the stages whose bit is set in
 * stage_mask (bit s = stage s of moe_lora_stage_name; 0xffffffff for all).
 * The *_timed variants of align, route_align and forward take it as their
 * last argument (NULL: nothing is recorded, exactly the plain call) and
 * record two events around each selected stage's launches on the call's
 * stream; a call counts once its forward is enqueued, and calls past
 * max_calls are not recorded.  moe_lora_profiler_read waits for the recorded
 * events and writes each stage's summed milliseconds to stage_ms[0..n)
 * (n <= moe_lora_stage_count()) and the recorded calls to *calls.
 * A recorder is used by one host thread at a time; the library itself keeps
 * no state between calls. */
int moe_lora_stage_count(void);
const char* moe_lora_stage_name(int stage);
int moe_lora_profiler_create(int max_calls, uint32_t stage_mask, moe_lora_profiler** out);
int moe_lora_profiler_read(moe_lora_profiler* prof, float* stage_ms, int n, int* calls);
void moe_lora_profiler_destroy(moe_lora_profiler* prof);
int moe_lora_align_timed(const moe_lora_shape* shape, const int32_t* topk_ids,
                         const int32_t* lora_ids, void* workspace, size_t ws_bytes, void* stream,
                         moe_lora_profiler* prof);
int moe_lora_route_align_timed(const moe_lora_shape* shape, const float* logits,
                               const int32_t* lora_ids, int32_t* topk_ids, float* topk_weights,
                               void* workspace, size_t ws_bytes, void* stream,
                               moe_lora_profiler* prof);
int moe_lora_forward_timed(const moe_lora_shape* shape, const uint16_t* x, const int32_t* topk_ids,
                           const float* topk_weights, const int32_t* lora_ids,
                           const uint16_t* W_gu, const uint16_t* W_down, const uint16_t* A_gu,
                           const uint16_t* B_gu, const uint16_t* A_down, const uint16_t* B_down,
                           void* workspace, size_t ws_bytes, uint16_t* y, void* stream,
                           moe_lora_profiler* prof);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LORA_H */
