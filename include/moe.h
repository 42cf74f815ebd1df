/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts layer.
 *
 * The layer follows the decomposition of vLLM's modular fused-MoE kernel
 * (page "vllm/model_executor/layers/fused_moe/modular_kernel.py", header
 * comment): [Router] -> [Quantize-Dispatch] -> [Permute-Experts-Unpermute]
 * -> [Combine].  One call exists per step, plus moe_forward for the whole
 * layer (FusedMoEModularKernel.forward on the same page) and
 * moe_shared_expert for the always-on shared expert (page "SharedExperts",
 * vllm fused_moe/runner/shared_experts).
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees, synchronises the host, or reads device data on
 *    the host.  Work is enqueued on the caller's stream(s) only, so every call
 *    can be captured into a hipGraph.
 *  - Tensors are dense and row-major.  Index tensors are int32.
 *  - Return codes come from host-side checks only (and from hipGetLastError
 *    after each launch).  Problems that only the device can see (an expert id
 *    out of range, a batched expert receiving more rows than its capacity)
 *    set bits of a sticky int32 status word inside the workspace
 *    (moe_ws_layout.status); the caller may read it after the stream has
 *    synchronised.  moe_prepare / moe_forward clear it.
 *  - M == 0 is valid: nothing is launched and MOE_OK is returned (the pages'
 *    empty-input case in FusedMoEModularKernel.forward).
 *  - One workspace belongs to one layer invocation at a time: moe_prepare,
 *    moe_experts and moe_finalize of the same step must be given the same
 *    workspace, and two steps in flight at once need two workspaces.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shapes   */
  MOE_ERR_UNSUPPORTED = 2, /* valid request this library does not implement */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size()    */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed     */
} moe_status;

/* FusedMoEActivationFormat (modular_kernel.py page):
 *  STANDARD          activations are (num_tokens, hidden);
 *  BATCHED_EXPERTS   activations are (num experts, max tokens per expert,
 *                    hidden): the padded "worst-tokens" layout whose masked
 *                    grouped GEMM reads per-expert counts from a device int32
 *                    tensor (page "EP: CUDA-graph-safe HT internode
 *                    dispatch+combine (worst-tokens mode)"). */
enum { MOE_FORMAT_STANDARD = 0, MOE_FORMAT_BATCHED_EXPERTS = 1 };

/* Element types.  FP8_E4M3 is OCP e4m3fn (max 448).  fp8 weights carry one
 * fp32 scale per 128x128 block; fp8 activations one fp32 scale per token and
 * group of 128 channels. */
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1, MOE_DTYPE_FP8_E4M3 = 2 };
enum { MOE_QUANT_NONE = 0, MOE_QUANT_FP8_TOKEN_GROUP_128 = 1 };
enum { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1 };
/* FusedMoEPermuteExpertsUnpermute.activation (modular_kernel.py page):
 * silu_and_mul, or gelu_and_mul with the exact GELU g * Phi(g)
 * = 0.5 g (1 + erf(g / sqrt 2)). */
enum { MOE_ACTIVATION_SILU = 0, MOE_ACTIVATION_GELU = 1 };

/* Weight layouts.  ROW_MAJOR is w1 [E, N, K] / w2 [E, K, N/2] as above.
 * PACKED is the same bytes reordered by moe_pack_weights so that each
 * wavefront of the weight-streaming GEMM reads one contiguous 4 KB block per
 * K-step (128 bytes of 16 rows, in MFMA fragment order).  The packed layout
 * is internal to this library version (moe_version) and needs (N/2) % 128 == 0. */
enum { MOE_WEIGHTS_ROW_MAJOR = 0, MOE_WEIGHTS_PACKED = 1 };

/* Bits of the device status word. */
enum { MOE_DEVICE_BAD_EXPERT_ID = 1, MOE_DEVICE_CAPACITY_OVERFLOW = 2 };

/* The problem, as _moe_problem_size (modular_kernel.py page) extracts it:
 * E experts, M tokens, N = rows of w1 per expert, K = hidden size, topk.
 * N = 2*I: w1 holds the gate rows [0, I) then the up rows [I, 2I) (the page
 * fixes only that the activation halves the width).
 * Unlike the page's 3-D case, M always counts tokens; the batched capacity
 * is max_tokens_per_expert.
 *
 * Expert-parallel shard (the page's expert_map / global_num_experts /
 * local_num_experts): E counts this GPU's local experts (weights, counts);
 * the router picks among global_E experts (logits [M, global_E], topk_ids in
 * [0, global_E)); expert_map (device int32[global_E]) gives each global expert
 * its local index or -1 when another shard holds it.  Picks of other shards
 * are neither counted nor computed and add nothing to this call's output, so
 * the shards' outputs sum to the unsharded layer's.  expert_map NULL and
 * global_E 0 (or E) is the plain one-shard layer.
 *
 * Activation chunking (the page's _maybe_chunk_fused_experts): with
 * 0 < chunk_tokens < M, moe_forward routes and prepares the whole batch, then
 * runs the experts step chunk by chunk (per-chunk recount, permutation, tile
 * plan and GEMMs) into slices of the full (M, topk, K) expert output, and
 * combines once.  The workspace then holds one chunk's intermediates.  The
 * STANDARD format only; the stage calls moe_prepare / moe_experts need an
 * unchunked problem.  Each token's result is the same as unchunked.
 *
 * apply_router_weight_on_input (topk == 1 only; FusedMoEModularKernel.forward
 * on the page): prepare multiplies each token's input row by its router
 * weight, rounded to act_dtype, before any quantisation, and the combine adds
 * the expert output unweighted. */
typedef struct moe_problem {
  int64_t E;
  int64_t M;
  int64_t N;
  int64_t K;
  int64_t topk;
  int64_t max_tokens_per_expert; /* BATCHED_EXPERTS: rows per expert buffer  */
  int64_t align;                 /* STANDARD: pad expert segments to this (0 = 1) */
  int64_t shared_N;              /* rows of the shared expert's w1 (2*I_s); 0 = none */
  int64_t global_E;              /* router width (experts in the global space); 0 = E */
  int64_t chunk_tokens;          /* moe_forward: experts step in chunks of this many tokens (0 = all) */
  int32_t format;                /* MOE_FORMAT_*                               */
  int32_t act_dtype;             /* x, out, fused_out: F32 or BF16            */
  int32_t w_dtype;               /* F32, BF16 or FP8_E4M3                      */
  int32_t act_quant;             /* MOE_QUANT_*; FP8 requires w_dtype FP8      */
  int32_t scoring;               /* MOE_SCORING_*                              */
  int32_t renormalize;           /* divide the k weights by their sum          */
  int32_t activation;            /* MOE_ACTIVATION_* (routed and shared experts) */
  int32_t apply_router_weight_on_input; /* 0 or 1 (1 needs topk == 1)        */
  int32_t weight_layout;         /* MOE_WEIGHTS_* of the expert weights        */
  int32_t reserved;              /* must be 0                                  */
  const int32_t *expert_map;     /* device int32[global_E] or NULL (identity)  */
} moe_problem;

/* Expert weights.  w1 [E, N, K], w2 [E, K, N/2] in w_dtype; for FP8_E4M3
 * w1_scale [E, N/128, K/128] and w2_scale [E, K/128, N/256] (fp32), else NULL. */
typedef struct moe_weights {
  const void *w1;
  const float *w1_scale;
  const void *w2;
  const float *w2_scale;
} moe_weights;

/* The shared expert and the streams it overlaps on (SharedExperts page,
 * maybe_forward_async / wait): input_ready is recorded on the main stream
 * (moe_forward: once the routed gated GEMM is queued, so the expert overlaps
 * the down GEMM; at the start when the experts step is chunked), the aux
 * stream waits on it and runs the expert,
 * output_ready is recorded on the aux stream and the main stream waits on it
 * before moe_forward returns.
 * w1 [shared_N, K], w2 [K, shared_N/2] in act_dtype; out [M, K] in act_dtype. */
typedef struct moe_shared {
  const void *w1;
  const void *w2;
  void *out;
  hipStream_t aux_stream;
  hipEvent_t input_ready;
  hipEvent_t output_ready;
} moe_shared;

/* Optional events recorded on the main stream between the kernels of
 * moe_forward, for timing: [0] start, [1] after route, [2] after prepare and
 * the grouped-GEMM tile plan, [3] after the gated grouped GEMM (w1, SiLU-and-
 * mul), [4] after the down grouped GEMM (w2; with fp8, after the
 * re-quantisation that precedes it), [5] after combine.  Any entry may be
 * NULL. */
#define MOE_NUM_STAGE_EVENTS 6
typedef struct moe_stage_events {
  hipEvent_t ev[MOE_NUM_STAGE_EVENTS];
} moe_stage_events;

/* Byte offsets of the workspace regions (for tests and inspection). */
typedef struct moe_ws_layout {
  size_t total_bytes;
  size_t status;      /* int32                                           */
  size_t counts;      /* int32[E]: tokens routed to each expert          */
  size_t offsets;     /* int32[E+1]: STANDARD segment starts (padded)    */
  size_t chunk_hist;  /* int32[n_chunks * E]                             */
  size_t tiles;       /* int32[max_tiles * 4] + int32 count              */
  size_t perm;        /* int32[perm_len]: slot -> pair m*topk+j, -1 pad  */
  size_t inv;         /* int32[M*topk]: pair -> slot (-1: dropped)       */
  size_t act;         /* first GEMM output [rows, N/2]                   */
  size_t act_q;       /* fp8: re-quantised act codes                     */
  size_t act_scale;   /* fp8: its scales                                 */
  size_t topk_weights;/* moe_forward: float[M*topk]                      */
  size_t topk_ids;    /* moe_forward: int32[M*topk]                      */
  size_t a_q;         /* moe_forward: prepared activations               */
  size_t a_scale;     /* moe_forward: their fp8 scales                   */
  size_t fused_out;   /* moe_forward: expert output (unweighted)         */
  size_t shared_act;  /* shared expert's intermediate [M, shared_N/2]    */
  int64_t perm_len;   /* M*topk + E*(align-1)                            */
  int64_t n_chunks;
  int64_t chunk;
  int64_t max_tiles;
  int64_t tile_rows;  /* rows per grouped-GEMM tile                      */
  int64_t act_rows;   /* rows of act (perm_len or E*capacity)            */
  size_t down_partial;/* fp32[down_split][perm_len][K]: K-split partial   */
                      /* sums of the down GEMM (empty when not split)     */
  int64_t down_split; /* K splits of the down GEMM (1: none)              */
} moe_ws_layout;

const char *moe_status_str(moe_status s);
/* ABI version, raised whenever a struct or a call changes: 5 (3: moe_ws_layout
 * gained down_partial and down_split; 4: moe_forward_noalloc; 5: the
 * asynchronous prepare / finalize calls and moe_forward_dbo). */
int moe_version(void);

/* Host-side check of a problem description (the asserts of
 * _moe_problem_size, FusedMoEPermuteExpertsUnpermute.activation and
 * FusedMoEModularKernel.__init__ on the modular_kernel.py page, plus this
 * library's own limits: E <= global_E <= 1024, topk <= min(global_E, 64),
 * K % 128 == 0, (N/2) % 64 == 0, fp8 needs (N/2) % 128 == 0, M*topk and
 * E*capacity < 2^31; expert_map NULL needs global_E 0 or E). */
moe_status moe_validate(const moe_problem *p);

/* Workspace needed by any call on this problem (workspace_shapes on the
 * modular_kernel.py page; one region per intermediate, none shared). */
moe_status moe_workspace_size(const moe_problem *p, size_t *bytes);
moe_status moe_workspace_layout(const moe_problem *p, moe_ws_layout *out);

/* One-time reordering of row-major expert weights into MOE_WEIGHTS_PACKED
 * (done once when weights are loaded, not per step).  src holds row-major
 * w1 / w2 (the problem's weight_layout is ignored); w1_packed and w2_packed
 * receive the same number of bytes each.  Scales are not reordered.  The
 * buffers must not overlap their sources. */
moe_status moe_pack_weights(const moe_problem *p, const moe_weights *src, void *w1_packed,
                            void *w2_packed, hipStream_t stream);

/* [Router]: logits [M, global_E] fp32 -> topk_weights [M, topk] fp32 and
 * topk_ids [M, topk] int32 global ids (the topk_weights / topk_ids that
 * FusedMoEModularKernel.forward consumes).  The topk experts with the largest
 * logits, in descending order, ties to the lower index; weights are the
 * softmax over all global_E logits or the sigmoid of each, optionally divided
 * by their sum.  NaN logits give unspecified (but in-range) ids. */
moe_status moe_route(const moe_problem *p, const float *logits, float *topk_weights,
                     int32_t *topk_ids, hipStream_t stream);

/* [Quantize-Dispatch] (FusedMoEPrepareAndFinalize.prepare): counts the pairs
 * routed to each local expert into expert_num_tokens [E] (ExpertTokensMetadata;
 * device only, no host copy) and lays the pairs out:
 *  STANDARD: a stable counting sort of the M*topk pairs by expert into the
 *    workspace permutation; a_out / a_scale_out receive x quantised per token
 *    group of 128 when act_quant is FP8 ([M, K] codes, [M, K/128] scales), or
 *    with the router weight on the input w*x in act_dtype ([M, K]), and must
 *    be NULL otherwise (the experts then read x directly).
 *  BATCHED_EXPERTS: row m of x goes to a_out[e, r, :] for each of its experts
 *    e, r its rank among e's pairs (ascending token); a_out is
 *    [E, max_tokens_per_expert, K] in act_dtype, or fp8 codes with a_scale_out
 *    [E, max_tokens_per_expert, K/128] when act_quant is FP8.  Rows past the
 *    counts are left untouched.  Pairs whose rank reaches the capacity are
 *    dropped and flag MOE_DEVICE_CAPACITY_OVERFLOW.
 * topk_weights [M, topk] is read only with apply_router_weight_on_input (else
 * it may be NULL).  topk_ids with an id outside [0, global_E), or mapped to an
 * entry outside [-1, E), flag MOE_DEVICE_BAD_EXPERT_ID and that pair is
 * ignored; picks mapped to -1 belong to other shards and are skipped. */
moe_status moe_prepare(const moe_problem *p, const void *x, const int32_t *topk_ids,
                       const float *topk_weights, void *a_out, float *a_scale_out,
                       int32_t *expert_num_tokens, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* [Permute-Experts-Unpermute] (FusedMoEPermuteExpertsUnpermute.apply): for
 * each expert, its rows times w1 (gate|up), act(gate) * up, [fp8:
 * re-quantised per token group], times w2.  `a` is what moe_prepare produced
 * (STANDARD without quantisation: x itself).  expert_num_tokens [E] is read on
 * the device (the masked grouped GEMM of the worst-tokens page).  fused_out
 * receives the unweighted, unreduced expert output in act_dtype:
 * STANDARD (M, topk, K); BATCHED_EXPERTS [E, max_tokens_per_expert, K] (rows
 * past each count untouched).  STANDARD also reads the permutation moe_prepare
 * left in the same workspace. */
moe_status moe_experts(const moe_problem *p, const void *a, const float *a_scale,
                       const moe_weights *w, const int32_t *expert_num_tokens, void *fused_out,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* [Combine] (FusedMoEPrepareAndFinalize.finalize with a TopKWeightAndReduce):
 * out[m, :] = sum_j topk_weights[m, j] * fused_out[pair (m, j), :], summed in
 * fp32 in j order, written in act_dtype; out [M, K] is fully overwritten.
 * It reads the pair -> row map moe_prepare left in the same workspace (so
 * moe_prepare of this step must have run on it): pairs with a bad expert id,
 * dropped batched pairs and other shards' picks contribute nothing, and their
 * fused_out rows are never read.  With apply_router_weight_on_input the
 * weights are not applied again (topk_weights may be NULL). */
moe_status moe_finalize(const moe_problem *p, const void *fused_out, const float *topk_weights,
                        void *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The shared expert alone (SharedExperts page): out [M, K] = the gated MLP
 * with w1 [shared_N, K], w2 [K, shared_N/2] applied to every token of x,
 * all in act_dtype (F32 or BF16), on `stream`. */
moe_status moe_shared_expert(const moe_problem *p, const void *x, const void *w1, const void *w2,
                             void *out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* The whole layer (FusedMoEModularKernel.forward): route, prepare, experts,
 * finalize on `stream`, all intermediates in the workspace; out [M, K] in
 * act_dtype.  With `shared` non-NULL (problem shared_N > 0) the shared expert
 * runs on shared->aux_stream concurrently and its output is ready when the
 * main stream passes the end of this call's work.  out may alias x only when
 * there is no shared expert.  `events` may be NULL. */
moe_status moe_forward(const moe_problem *p, const float *logits, const void *x,
                       const moe_weights *w, void *out, const moe_shared *shared,
                       void *workspace, size_t workspace_bytes, hipStream_t stream,
                       const moe_stage_events *events);

/* ---------------------------------------------------------------------
 * Asynchronous prepare / finalize and the two-microbatch schedule
 * (modular_kernel.py page: FusedMoEPrepareAndFinalize.prepare_async and
 * finalize_async, whose result is a hook / receiver pair equivalent to
 * prepare / finalize; FusedMoEModularKernel.shared_buffers, one set of
 * buffers per DBO microbatch; the supports_async() branch of
 * FusedMoEModularKernel.forward; page "DBO HT without cudagraph").  On one
 * GPU the dispatch and combine are local kernels, so what the overlap can
 * hide is their latency-bound chain (router, counting, scan, ranking), not
 * communication.
 */

/* moe_prepare enqueued on `stream` (the dispatch stream), then `done`
 * recorded there; returns at once.  The outputs are valid on any stream once
 * it has passed moe_receive(that stream, done) (or done has completed); until
 * then they must not be read.  Same arguments and errors as moe_prepare;
 * `done` must be a valid event. */
moe_status moe_prepare_async(const moe_problem *p, const void *x, const int32_t *topk_ids,
                             const float *topk_weights, void *a_out, float *a_scale_out,
                             int32_t *expert_num_tokens, void *workspace, size_t workspace_bytes,
                             hipStream_t stream, hipEvent_t done);

/* moe_finalize enqueued on `stream`, then `done` recorded there; out is valid
 * after moe_receive(consumer, done).  Same arguments and errors as
 * moe_finalize. */
moe_status moe_finalize_async(const moe_problem *p, const void *fused_out, const float *topk_weights,
                              void *out, void *workspace, size_t workspace_bytes, hipStream_t stream,
                              hipEvent_t done);

/* The receiver: `stream` waits (on the device, the host returns at once) for
 * the work `done` marks.  hipEventQuery(done) is the non-blocking check. */
moe_status moe_receive(hipStream_t stream, hipEvent_t done);

/* Events of moe_forward_dbo, created by the caller (any flags). */
typedef struct moe_dbo_events {
  hipEvent_t prepared[2];   /* dispatch stream: microbatch u routed and prepared */
  hipEvent_t computed[2];   /* compute stream: microbatch u's expert GEMMs done  */
  hipEvent_t finalized[2];  /* dispatch stream: microbatch u combined            */
} moe_dbo_events;

/* The layer in two microbatches (tokens [0, (M+1)/2) and [(M+1)/2, M)), each
 * with its own workspace, on two streams:
 *   dispatch stream: route + prepare of microbatch 0, then of microbatch 1
 *                    (beside microbatch 0's expert GEMMs), then each
 *                    microbatch's combine once its experts are done (the
 *                    combine of 0 beside the experts of 1);
 *   compute stream:  the expert GEMMs of microbatch 0, then of microbatch 1.
 * The dispatch stream starts from the compute stream's position at the call
 * and the compute stream joins it at the end, so to the caller this is one
 * call on compute_stream, like moe_forward; out [M, K] is fully written.
 * Each token's result equals moe_forward's whenever both pick the same GEMM
 * kernels (the microbatches are half as large, which can change the choice).
 *  - workspace0 / workspace1: distinct, each at least moe_workspace_size() of
 *    the problem with M replaced by (M + 1) / 2.
 *  - shared: NULL, or an array of two moe_shared, one per microbatch (its
 *    rows of the shared output and its own event pair, as the SharedExperts
 *    page keeps one pair per microbatch).
 *  - MOE_ERR_UNSUPPORTED with chunk_tokens > 0 (chunk the microbatches
 *    instead). */
moe_status moe_forward_dbo(const moe_problem *p, const float *logits, const void *x, const moe_weights *w,
                           void *out, const moe_shared *shared, void *workspace0, void *workspace1,
                           size_t workspace_bytes, hipStream_t compute_stream, hipStream_t comm_stream,
                           const moe_dbo_events *ev);

/* For callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward
 * with the workspace held by the library itself, a static device array of
 * MOE_STATIC_SCRATCH_BYTES on each GPU the library runs on (kept until the
 * process ends), instead of a caller buffer.  Arguments as moe_forward; the
 * caller still owns every input and output.  stream must belong to the
 * current device; the first call on each device looks up that device's copy
 * of the array (outside graph capture: make one eager call first).
 *  - MOE_ERR_WORKSPACE when moe_workspace_size() of the problem exceeds
 *    MOE_STATIC_SCRATCH_BYTES (nothing is launched).
 *  - status_out (device int32, may be NULL) receives the device status word
 *    of this call once the stream reaches the end of its work (untouched when
 *    M == 0).
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (other streams, other host threads) race and give undefined results;
 *    calls in one stream order are safe.  Nothing is carried from one call to
 *    the next (the kernels reset what must start at zero).
 *  - Allocates nothing: no hipMalloc, hipFree or allocating library call. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_problem *p, const float *logits, const void *x,
                               const moe_weights *w, void *out, const moe_shared *shared,
                               hipStream_t stream, const moe_stage_events *events, int32_t *status_out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
