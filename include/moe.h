/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward.
 *
 * One MoE layer on one GPU, every expert resident in HBM:
 *   route     : linear gate -> softmax/sigmoid scores -> (group limit) -> top-k
 *               -> gates                               (moe_route)
 *   dispatch  : per-expert histogram -> exclusive scan -> stable permutation of
 *               the T*k assignments into expert-contiguous rows -> row gather
 *                                                      (moe_dispatch)
 *   expert FFN: per-expert SwiGLU as a grouped GEMM over the ragged segments
 *                                                      (moe_grouped_ffn)
 *   combine   : gate-weighted sum of each token's k expert rows, back in token
 *               order, plus the shared expert          (moe_combine)
 *   the whole chain                                    (moe_layer_forward)
 *
 * The dataflow is the per-token routing path of "Expert-Parallel MoE
 * Inference: Serving Sparse Models at Scale" (section "Deeper Analysis:
 * Routing, Balance, and a Capacity Worked Example", Figure 2) and the
 * router -> top-k -> dispatch -> expert FFN -> combine chain of "MoE Expert
 * Parallelism in Practice" (section "Core Principles", item 1).  The
 * expert-contiguous buffer is the layout the dispatch exchange ships ("Expert-
 * Parallel MoE Inference", section "The all-to-all dispatch and combine, step
 * by step", Figure 3); experts run as grouped GEMMs and combine is a weighted
 * sum ("Tensor vs Expert vs Data Parallelism for MoE Serving", section
 * "Deeper Analysis", Figure 2).  Dispatch is drop-free: every assignment is
 * processed (section "Capacity factor and token dropping" of the first page).
 *
 * Conventions (all entry points)
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer; the library allocates nothing and keeps no state.
 *   - Row-major, contiguous.  Weights are stored out x in (K contiguous):
 *       w_router [E][d], w1/w3 [E][f][d], w2 [E][d][f],
 *       shared w1/w3 [f_shared][d], shared w2 [d][f_shared].
 *   - Every device pointer must be 16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     with no host synchronisation, so a call can be captured in a HIP graph.
 *     Outputs are valid once the stream reaches the end of the call.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a bad argument returns a negative moe_status and enqueues
 *     nothing.  A launch failure returns MOE_ERR_DEVICE.  Faults inside a
 *     kernel surface at the caller's next synchronisation.  Nothing is printed
 *     and nothing aborts.  A workspace smaller than the size the matching
 *     moe_workspace_size query returns gives MOE_ERR_WORKSPACE: the library
 *     never drops tokens to fit a buffer (fixed buffers fail loudly, as the
 *     low-latency dispatch of "Tensor vs Expert vs Data Parallelism", section
 *     "Two kernel modes for two phases", does).
 *   - Entry points are reentrant; calls that share output or workspace
 *     buffers must be ordered by the caller (same stream or events).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* null/misaligned pointer, inconsistent sizes   */
  MOE_ERR_UNSUPPORTED = -2,  /* shape or dtype combination not implemented    */
  MOE_ERR_WORKSPACE = -3,    /* workspace smaller than the size query returns */
  MOE_ERR_DEVICE = -4        /* a HIP call or kernel launch failed            */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;
typedef enum {
  MOE_STAGE_ROUTE = 0, MOE_STAGE_DISPATCH = 1, MOE_STAGE_FFN = 2, MOE_STAGE_LAYER = 3
} moe_stage;

/* Host struct describing one layer, passed by pointer. */
typedef struct {
  int32_t T;          /* tokens, >= 0 (0: only counts/offsets are written, as 0)  */
  int32_t d;          /* hidden size, multiple of 128                             */
  int32_t f;          /* routed-expert FFN width, multiple of 128                 */
  int32_t E;          /* routed experts, 1..512                                   */
  int32_t k;          /* experts per token, 1..min(E, 16)                         */
  int32_t score;      /* moe_score                                                */
  int32_t renorm;     /* 1: gates divided by their sum over the chosen k          */
  int32_t n_group;    /* 0 = no group limit; else divides E, E/n_group >= 2       */
  int32_t topk_group; /* groups kept (1..n_group), topk_group*E/n_group >= k      */
  int32_t f_shared;   /* 0 = no shared expert; else multiple of 128               */
  int32_t act;        /* moe_dtype of activations: MOE_F32 or MOE_BF16            */
  int32_t wdtype;     /* moe_dtype of routed weights: act, or MOE_FP8_E4M3 when
                         act is MOE_BF16 (per-output-channel fp32 scales)         */
  int32_t capacity;   /* 0 = dropless; else slots per expert (>= 1), e.g. from
                         moe_capacity_slots (capacity_factor * T * k / E,
                         rounded up).  Assignments claim slots in increasing
                         a = t*k + j; one that finds its expert full is dropped
                         (contributes 0)                                     */
  int32_t overflow;   /* with a capacity: MOE_OVERFLOW_DROP (0) drops an
                         assignment that finds its expert full;
                         MOE_OVERFLOW_REROUTE (1) first offers it the token's
                         next-best expert (see "Capacity overflow" below;
                         moe_layer_forward only)                              */
  int32_t dispatch_fp8; /* 0: the dispatched rows are x itself (act dtype);
                         1: they are the block-scaled E4M3 payload of x (act
                         must be MOE_BF16; see "fp8 dispatch payload" below).
                         The router and the shared expert always read x.    */
  int32_t w_layout;   /* moe_w_layout of the routed w1, w3, w2 (see "Weight
                         layout" below); the router's and the shared expert's
                         weights are always row-major                        */
} moe_desc;

typedef enum { MOE_OVERFLOW_DROP = 0, MOE_OVERFLOW_REROUTE = 1 } moe_overflow;
typedef enum { MOE_W_ROWMAJOR = 0, MOE_W_KBLOCKED = 1 } moe_w_layout;

/* Weight layout.  Each routed expert matrix has N output rows and K input
 * columns (w1, w3: N = f, K = d; w2: N = d, K = f).
 *   MOE_W_ROWMAJOR: element (n, c) at n*K + c, K contiguous.
 *   MOE_W_KBLOCKED: K/32 planes of [N][32]; element (n, c) at
 *     (c/32)*N*32 + n*32 + c%32, so a tile's 32-column slice of consecutive
 *     rows is one contiguous run (whole cache lines for the direct-to-LDS
 *     loads of the MFMA kernels).  Requires wdtype MOE_BF16 or MOE_FP8_E4M3;
 *     moe_pack_weights converts once, e.g. at load time.
 * Experts stay consecutive ([E][...]) and the fp8 scales keep their layout. */

/* Capacity overflow rerouted (capacity > 0, overflow = MOE_OVERFLOW_REROUTE).
 * "Expert-Parallel MoE Inference", section "Capacity factor and token
 * dropping": overflow tokens are dropped or rerouted to their next-best
 * expert.  Two passes over the assignments a = t*k + j:
 *   1. each claims a slot of its own expert in increasing a (as dropping);
 *   2. the m-th assignment of a token that found its expert full (counting in
 *      increasing j) is offered the token's candidate m -- its eligible
 *      expert of rank k + m in the router's order (score descending, id
 *      ascending) -- and the offers claim the slots left after pass 1, in
 *      increasing a.  An offer with no slot, or an overflow with no
 *      candidate, is dropped.
 * A rerouted copy carries its new expert's gate: the expert's score, divided
 * by the sum of the token's top-k scores when renorm = 1.  Rows of an expert
 * are its pass-1 rows, then its pass-2 rows, each in increasing a.  counts
 * stay the demand of the top-k; topk_idx and topk_w stay the router's top-k.
 * moe_layer_forward runs it whole; as stages, moe_route_candidates returns
 * the candidates and moe_dispatch_reroute dispatches with them (moe_dispatch
 * returns MOE_ERR_UNSUPPORTED for this mode). */

/* fp8 dispatch payload (dispatch_fp8 = 1).  Each row of x is cut into blocks
 * of 32 elements; a block with largest magnitude amax gets the scale 2^s, s
 * the smallest integer with amax <= 448 * 2^s (so nothing saturates), clamped
 * to [-127, 127], and s = 0 for an all-zero block; its elements become OCP
 * E4M3 codes of x / 2^s rounded to nearest, ties to even (a value that rounds
 * to zero is +0).  The experts see code value * 2^s.  DeepSeek's serving
 * system dispatches FP8 token copies and combines in BF16 ("Tensor vs Expert
 * vs Data Parallelism for MoE Serving", section "Deeper Analysis", Figure 2);
 * the 32-element power-of-two scale is the block the gfx950 block-scaled MFMA
 * consumes.  A payload of R rows is one buffer of
 *   MOE_FP8_PAYLOAD_BYTES(R, d) bytes:
 *   codes  uint8 [R][d]                at byte 0
 *   scales uint8 [R][MOE_FP8_SCALE_STRIDE(d)], E8M0 (byte = s + 127), at
 *          byte MOE_FP8_SCALES_OFFSET(R, d); block b of row r at r*stride + b. */
#define MOE_FP8_SCALE_STRIDE(d) ((((size_t)(d) / 32) + 15) / 16 * 16)
#define MOE_FP8_SCALES_OFFSET(R, d) (((size_t)(R) * (size_t)(d) + 255) / 256 * 256)
#define MOE_FP8_PAYLOAD_BYTES(R, d) \
  (MOE_FP8_SCALES_OFFSET(R, d) + (size_t)(R) * MOE_FP8_SCALE_STRIDE(d))

/* Number of hipEvents moe_layer_forward records when given a trace array. */
#define MOE_TRACE_EVENTS 7

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status s);

/* Validates `desc` (host) without touching the GPU.  MOE_OK if supported. */
moe_status moe_validate(const moe_desc* desc);

/* Expert capacity in slots: a capacity factor times the average load T*k/E,
 * rounded up to whole slots, the static per-expert buffer size of "Expert-
 * Parallel MoE Inference" (section "Capacity factor and token dropping").
 * The factor is the exact ratio factor_num / factor_den (1.25 is 5/4):
 *   *slots (host) = ceil(factor_num * T * k / (factor_den * E)),
 * computed exactly in integers; 0 (dropless, no limit) when factor_num <= 0.
 * Host only, touches no GPU.  MOE_ERR_INVALID when slots is NULL,
 * factor_den <= 0, T < 0, k < 1, E < 1 or the result exceeds INT32_MAX. */
moe_status moe_capacity_slots(int64_t factor_num, int64_t factor_den, int32_t T, int32_t k, int32_t E,
                              int32_t* slots);

/* Workspace bytes needed by moe_route, moe_dispatch, moe_grouped_ffn or
 * moe_layer_forward for `desc`; written to *bytes (host). */
moe_status moe_workspace_size(const moe_desc* desc, moe_stage stage, size_t* bytes);

/* Router.  Scores every expert for every token with the linear gate
 *   z[t,e] = sum_i x[t,i] * w_router[e][i] + bias[e]   (fp32 accumulate)
 * then s = softmax(z) over the E experts or s = sigmoid(z); with n_group > 0
 * only the experts of the topk_group groups with the largest group score
 * (sum of the group's two largest s) are eligible; keeps the k eligible experts
 * with the largest s (ties: lower id first) in descending order; gate
 * g = s (renorm = 0) or s / sum of the k chosen s (renorm = 1).
 *   x        [T][d]   act dtype
 *   w_router [E][d]   act dtype
 *   bias     [E]      fp32, nullable (no bias)
 *   topk_idx [T][k]   int32 out
 *   topk_w   [T][k]   fp32  out
 *   ws: moe_workspace_size(MOE_STAGE_ROUTE) bytes (holds the fp32 logits).
 * ("Expert-Parallel MoE Inference", section "Deeper Analysis", first
 * paragraph and Figure 2.) */
moe_status moe_route(const moe_desc* desc, const void* x, const void* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* The router plus each token's rerouting candidates (capacity overflow
 * rerouted, overflow = MOE_OVERFLOW_REROUTE; see "Capacity overflow" above):
 * moe_route's outputs, and
 *   cand_idx [T][k] int32 out: candidate m of token t is its eligible expert
 *            of rank k + m in the router's order, -1 where fewer than k + m + 1
 *            experts are eligible
 *   cand_w   [T][k] fp32  out: the candidate's gate, with the normalisation of
 *            topk_w (its score over the sum of the top-k scores when renorm)
 *   ws: moe_workspace_size(MOE_STAGE_ROUTE) bytes.
 * For moe_dispatch_reroute; any overflow mode of desc is accepted. */
moe_status moe_route_candidates(const moe_desc* desc, const void* x, const void* w_router, const float* bias,
                                int32_t* topk_idx, float* topk_w, int32_t* cand_idx, float* cand_w, void* ws,
                                size_t ws_bytes, void* stream);

/* Dispatch.  For the T*k assignments a = t*k + j (expert topk_idx[t][j]):
 *   counts[e]      = number of assignments to expert e          int32 [E]
 *   kept[e]        = counts[e], or min(counts[e], capacity) with a capacity
 *   offsets[e]     = sum of kept[e'] for e' < e; offsets[E] = sum of kept
 *                    (T*k when dropless)                          int32 [E+1]
 *   inv_pos[a]     = row of assignment a: offsets[e] + number of earlier
 *                    assignments (smaller a) to the same expert, or -1 when
 *                    that number reaches the capacity (dropped)   int32 [T*k]
 *   perm_token[p]  = token of row p (so perm_token[inv_pos[a]] = a / k),
 *                    for p < offsets[E]                            [T*k]
 *   x_perm[p][:]   = x[perm_token[p]][:], p < offsets[E]  act dtype [T*k][d];
 *                    with dispatch_fp8 the payload of those rows, R = T*k
 *                    (MOE_FP8_PAYLOAD_BYTES(T*k, d) bytes)
 * Rows of one expert are contiguous and in increasing token order; the result
 * is deterministic.  topk_idx entries must lie in [0, E).  The capacity slots
 * are those of "Expert-Parallel MoE Inference", section "Capacity factor and
 * token dropping": each routed token takes a free slot of its expert or is
 * dropped.
 * ws: device workspace of moe_workspace_size(MOE_STAGE_DISPATCH) bytes. */
moe_status moe_dispatch(const moe_desc* desc, const int32_t* topk_idx, const void* x,
                        int32_t* counts, int32_t* offsets, int32_t* perm_token,
                        int32_t* inv_pos, void* x_perm, void* ws, size_t ws_bytes,
                        void* stream);

/* moe_dispatch with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (less ws, ws_bytes) and the same
 * outputs as moe_dispatch, bit for bit; allocates nothing and calls no
 * allocating routine.
 * Its scratch (the per-chunk expert counts) is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library, one copy per GPU, held until the
 * process ends.  A desc whose dispatch workspace (moe_workspace_size with
 * MOE_STAGE_DISPATCH: ceil(T*k/256) * E * 4 bytes) exceeds it gives
 * MOE_ERR_WORKSPACE: T*k up to 2^28 / E assignments fit (2^20 at E = 256).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * Nothing in the array needs clearing: each call writes every entry it reads.
 * The buffers and the stream must belong to the current device; the first
 * call on a device looks up its copy of the array (MOE_ERR_DEVICE if that
 * fails).  overflow = MOE_OVERFLOW_REROUTE gives MOE_ERR_UNSUPPORTED. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
moe_status moe_dispatch_noalloc(const moe_desc* desc, const int32_t* topk_idx, const void* x, int32_t* counts,
                                int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, void* x_perm,
                                void* stream);

/* Dispatch with capacity overflow rerouted (desc: capacity > 0 and overflow =
 * MOE_OVERFLOW_REROUTE, else MOE_ERR_INVALID): the two passes of "Capacity
 * overflow" above, from moe_route_candidates' outputs.  Outputs as
 * moe_dispatch -- inv_pos[a] is the row of the copy that serves assignment a
 * (its own expert's, or its candidate's when rerouted), or -1 when dropped;
 * an expert's rows are its pass-1 rows, then its pass-2 rows -- and
 *   gates [T*k] fp32 out: the gate of the copy serving assignment a (topk_w,
 *         or the candidate's cand_w when rerouted), to pass to moe_combine in
 *         place of topk_w; unspecified where inv_pos[a] = -1.
 * ws: moe_workspace_size(MOE_STAGE_DISPATCH) bytes for this desc. */
moe_status moe_dispatch_reroute(const moe_desc* desc, const int32_t* topk_idx, const float* topk_w,
                                const int32_t* cand_idx, const float* cand_w, const void* x, int32_t* counts,
                                int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, float* gates,
                                void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* Row-major [mats][rows][cols] -> K-blocked [mats][cols/32][rows][32]
 * (MOE_W_KBLOCKED with N = rows, K = cols), elem_bytes 1 (E4M3) or 2 (bf16).
 * src and dst: device, 16-byte aligned, not overlapping; cols a multiple of
 * 32; mats * rows * cols * elem_bytes at most 2^40.  One kernel on `stream`.
 * MOE_ERR_INVALID for bad arguments.  A storage layout of the same values
 * (see "Weight layout"), not a step of the method: no page defines it. */
moe_status moe_pack_weights(const void* src, int64_t mats, int32_t rows, int32_t cols, int32_t elem_bytes,
                            void* dst, void* stream);

/* Grouped expert FFN over the expert-contiguous rows.  Expert e transforms
 * rows [offsets[e], offsets[e+1]) of x_perm (act dtype [T*k][d], or with
 * dispatch_fp8 the payload of T*k rows as moe_dispatch writes it):
 *   u = x W1_e^T, v = x W3_e^T (fp32 accumulate, times s1/s3 for fp8),
 *   h = silu(u) * v   stored in the act dtype                    [T*k][f]
 *   y = h W2_e^T      (times s2 for fp8) stored in the act dtype [T*k][d]
 * SwiGLU, silu(u) = u / (1 + exp(-u)).
 *   offsets  [E+1] int32 (device), as produced by moe_dispatch; offsets[E]
 *            <= T*k (rows past it are not touched)
 *   w1, w3   [E][f][d], w2 [E][d][f] in wdtype, laid out per w_layout
 *   s1, s3   [E][f], s2 [E][d] fp32 per-output-channel scales when wdtype is
 *            MOE_FP8_E4M3, else NULL
 *   h, y_perm outputs; ws: moe_workspace_size(MOE_STAGE_FFN) bytes.
 * Each expert transforms only the rows routed to it; all experts' segments
 * run as one grouped GEMM ("Tensor vs Expert vs Data Parallelism for MoE
 * Serving", section "Deeper Analysis", Figure 2; the expert's FFN step of the
 * per-token path in "Expert-Parallel MoE Inference", section "Deeper
 * Analysis", Figure 2).  The SwiGLU form and the fp8 weights with per-channel
 * scales are this layer's definition; the pages name neither. */
moe_status moe_grouped_ffn(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                           const void* w1, const void* w3, const void* w2,
                           const float* s1, const float* s3, const float* s2,
                           void* h, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* Combine.  out[t][:] = sum_{j<k} topk_w[t][j] * y_perm[inv_pos[t*k+j]][:]
 *                       (+ shared_y[t][:]), fp32 accumulation in that order,
 * stored in the act dtype; terms with inv_pos = -1 (dropped) are skipped.
 * No atomics: each token reads its own k rows.
 *   shared_y [T][d] act dtype, nullable.
 * The expert outputs come back to their tokens' original order and are
 * summed weighted by the gates ("Expert-Parallel MoE Inference", section
 * "Deeper Analysis", Figure 2, and the combine step of section "The all-to-
 * all dispatch and combine, step by step", Figure 3; the weighted-sum combine
 * of "Tensor vs Expert vs Data Parallelism", section "Deeper Analysis",
 * Figure 2).  The always-on shared expert is added with coefficient 1
 * (DeepSeek-V3's shared expert, same page, section "Context and Background"). */
moe_status moe_combine(const moe_desc* desc, const void* y_perm, const int32_t* inv_pos,
                       const float* topk_w, const void* shared_y, void* out, void* stream);

/* The whole layer: route, dispatch, grouped FFN, shared expert (when
 * f_shared > 0: the SwiGLU expert of every token with gate 1, weights in the
 * act dtype), combine.  Intermediates (perm_token, inv_pos, offsets, x_perm,
 * h, y_perm, shared h and y) live in ws (moe_workspace_size(MOE_STAGE_LAYER))
 * in layouts of the library's choosing.
 *   w1, w3, w2, s1, s3, s2 as for moe_grouped_ffn (w_layout applies).
 *   out [T][d] act dtype; topk_idx [T][k], topk_w [T][k], counts [E] outputs.
 *   sw1, sw3, sw2: shared expert, NULL when f_shared == 0.
 *   trace: NULL, or MOE_TRACE_EVENTS hipEvent_t (host array of handles)
 *          recorded on `stream` before the router and after the router,
 *          dispatch (with the GEMM tile table), routed gate-up GEMM, routed
 *          down GEMM, shared expert and combine, for per-stage timing.
 * The chain router -> top-k -> dispatch -> expert FFN -> combine -> original
 * token order of "MoE Expert Parallelism in Practice" (section "Core
 * Principles", item 1) and of the per-token path in "Expert-Parallel MoE
 * Inference", section "Deeper Analysis", Figure 2, on one GPU: the
 * expert-contiguous rows the dispatch exchange would ship stay local. */
moe_status moe_layer_forward(const moe_desc* desc, const void* x, const void* w_router,
                             const float* bias, const void* w1, const void* w3, const void* w2,
                             const float* s1, const float* s3, const float* s2,
                             const void* sw1, const void* sw3, const void* sw2,
                             void* out, int32_t* topk_idx, float* topk_w, int32_t* counts,
                             void* ws, size_t ws_bytes, void* stream, void* const* trace);

/* Rows each expert processed in the last moe_layer_forward enqueued with this
 * workspace (same desc, same stream, before this call):
 *   rows[e] = offsets[e+1] - offsets[e]                       int32 [E], device
 * The demand (counts) less the assignments dropped, plus, when rerouting,
 * those rerouted to e: the capacity's drop-rate metric ("Expert-Parallel MoE
 * Inference", section "Capacity factor and token dropping").  Enqueued on
 * `stream`; ws and ws_bytes as given to moe_layer_forward. */
moe_status moe_layer_rows(const moe_desc* desc, const void* ws, size_t ws_bytes, int32_t* rows,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
