/*
 * libmoe_gfx950 -- one GPU's mixture-of-experts layer on AMD Instinct MI355X
 * (gfx950), forward and backward, as a C ABI.
 *
 * The layer is y = sum over the top-k experts of g(x)_i * E_i(x) ("Scalable
 * Training of Mixture-of-Experts Models with Megatron Core", summary page,
 * "Problem Definition"), run in the stage order Router -> Dispatcher ->
 * Experts -> Combiner (same page, "Pipeline Flow"; thelatestinai.com page,
 * Figure 1).  On one GPU, dispatch and combine become a permutation of token
 * rows into expert-contiguous order and its inverse.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is DEVICE memory unless stated otherwise; the
 *   caller owns and allocates all of it (inputs, outputs, workspace).  The
 *   library never allocates, frees or synchronises, never copies anything to
 *   the host and only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *   default stream).  Calls are asynchronous: device-side faults surface at the
 *   caller's next synchronisation.
 * - Matrices are row-major and contiguous.  "storage" means the element type
 *   named by moe_cfg.dtype: float (MOE_F32) or bfloat16 (MOE_BF16 and
 *   MOE_MXFP8, stored as uint16_t bit patterns).  fp32 tensors (logits, gates, d_gates, d_logits,
 *   dx_partial) are float in every mode.  Indices are int32.
 * - Weights use the nn.Linear orientation [out, in]: w_router [E, d];
 *   w13 [E, 2f, d] with rows 0..f-1 the gate projection and f..2f-1 the up
 *   projection; w2 [E, d, f]; the shared expert ws13 [2 f_shared, d] and
 *   ws2 [d, f_shared].
 * - Rows of the permuted buffers ([T*k, .]) are expert-major: expert e owns rows
 *   expert_offsets[e] .. expert_offsets[e+1]-1, tokens in ascending order inside
 *   an expert.  Routing is dropless: exactly T*k rows, no capacity, no padding.
 * - Every argument is validated on the host before anything is launched
 *   (null pointers, shape limits, 16-byte alignment of storage matrices).  On
 *   failure nothing is enqueued and a status is returned; moe_last_error() then
 *   names the offending argument.  Indices produced by these calls are trusted:
 *   out-of-range expert ids or row ids passed in by a caller are undefined.
 * - Results are deterministic: no floating-point atomics, fixed reduction order.
 *   topk_idx, expert_counts, expert_offsets, row_id_map and src_token are
 *   bit-identical to any correct implementation of the rules below given the
 *   same fp32 router logits.
 * - Limits: 1 <= k <= E <= 256, d and f multiples of 8 (f_shared too; multiples
 *   of 64 for calls that run bf16 GEMMs: router with x, experts, backward), T*k and
 *   every matrix dimension below 2^31 elements per row index.
 */
#ifndef MOE_GFX950_H
#define MOE_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad shape, misalignment    */
  MOE_ERR_UNSUPPORTED = 2,        /* not a gfx950 device, dtype not built     */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_DEVICE = 4              /* a HIP call or kernel launch failed       */
} moe_status;

/* MOE_MXFP8: bf16 storage everywhere, expert GEMMs (routed and shared) on fp8
 * e4m3 operands with e8m0 block scales -- see moe_quantize_mxfp8.
 * MOE_MXFP4: the same with fp4 e2m1 operands -- see moe_quantize_mxfp4. */
typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2, MOE_MXFP4 = 3 } moe_dtype;

typedef enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* Layer modes (moe_cfg.flags, any combination).
 *
 * MOE_FLAG_FORCE_BALANCED: the benchmark condition of the pages' throughput
 *   runs (thelatestinai.com page, Table 11 caption: force-balanced routing).
 *   moe_router_topk still computes logits and scores, but choice j of token t
 *   is expert (t*k + j) mod E instead of the top-k: every expert receives
 *   T*k/E rows when E divides T*k.  Gates follow the usual rule on the
 *   assigned experts' logits or scores; group limits and the bias play no part.
 *
 * MOE_FLAG_FOLD_GATES: gate folding, a reading of the memory-efficient
 *   permutation (figures page, Figure 7 and Table 6).  Each permuted row's
 *   gate multiplies its SwiGLU output before the down projection (which is
 *   linear), act[r] = storage(g_r silu(H) U), so y_perm rows already carry
 *   their gates and the combine sums them unweighted.  The backward then needs
 *   neither a saved y_perm nor a gate-weighted dy_perm: dy_perm rows are
 *   copies of dy, and the gate gradient d_gates[t,j] = <dA, silu(H) U> of the
 *   row is formed inside the grouped-GEMM backward (dA = dy_perm w2[e], fp32).
 *   The calls then take row_gates / row_id_map / d_gates as described below.
 *
 * MOE_FLAG_RECOMPUTE_ACT: SwiGLU recomputation (figures page, Figure 8
 *   "Selective Recomputation"; Table 4, "Activation Function (SwiGLU)").  The
 *   forward forms act from the stored (rounded) H and U, and the backward
 *   forms it again from hu_save (and hu_shared_save) into its workspace, so act
 *   (and act_shared) are not read by the backward and need not be kept after
 *   the forward; the re-formed act is bit-identical to the forward's. */
typedef enum moe_flags {
  MOE_FLAG_FORCE_BALANCED = 1,
  MOE_FLAG_FOLD_GATES = 2,
  MOE_FLAG_RECOMPUTE_ACT = 4
} moe_flags;

/* Shape and routing rule of one MoE layer (host memory). */
typedef struct moe_cfg {
  int64_t T;          /* tokens (batch x sequence, flattened)                */
  int64_t d;          /* hidden size                                          */
  int64_t E;          /* routed experts                                       */
  int64_t k;          /* experts per token                                    */
  int64_t f;          /* routed expert FFN width                              */
  int64_t f_shared;   /* shared-expert FFN width, 0 = no shared expert        */
  int32_t score;      /* moe_score                                            */
  int32_t n_group;    /* expert groups for group-limited routing (1 = off)    */
  int32_t topk_group; /* groups kept per token                                */
  int32_t renorm;     /* 1: gates renormalised over the selected experts      */
  float scale;        /* gate multiplier applied after renormalisation        */
  float aux_coeff;    /* load-balancing loss coefficient (0 = off; softmax)   */
  int32_t dtype;      /* moe_dtype of activations and weights                 */
  int32_t flags;      /* moe_flags bits (0: plain top-k, gated combine, act kept) */
} moe_cfg;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* Message describing the last failure of a call made on this host thread
 * ("" if the last call succeeded).  Valid until the next call on the thread. */
const char* moe_last_error(void);

/* Checks that `device` is a gfx950 GPU and caches its properties.  Optional:
 * every call performs the same check lazily on the current device. */
moe_status moe_init(int device);

/* Bytes of device workspace every call below needs for `cfg` (the same size
 * serves all of them).  0 on an invalid cfg (see moe_last_error). */
size_t moe_workspace_size(const moe_cfg* cfg);

/* ---------------------------------------------------------------------------
 * Router ("System Modules: Router": a learned linear layer producing a
 * probability distribution and a top-k choice per token; Figure 2: linear
 * projection, score function, top-k selection, load balancing).
 *
 *   logits[t,e] = sum_i x[t,i] w_router[e,i]     fp32 accumulation, stored fp32
 *   softmax: selection key = the logit; p = softmax over all E (fp32)
 *   sigmoid: s = fp32(1/(1+exp(-(double)l))); key = fp32(s + bias[e]); the
 *            bias only steers selection
 *   n_group > 1: experts split into n_group contiguous groups of E/n_group;
 *            group score = fp32 sum of its two largest keys (its only key for
 *            one-expert groups); the topk_group best groups (ties -> lower
 *            group id) are eligible, the rest are not
 *   topk_idx[t,:] = the k eligible experts by key descending, equal keys ->
 *            lower expert id, in that order
 *   gates:   softmax+renorm: softmax over the selected logits; softmax without
 *            renorm: p of the selected experts; sigmoid: s_j / sum of selected s
 *            (if renorm) -- all multiplied by cfg.scale
 *   expert_counts[e] = number of (t, j) with topk_idx[t,j] == e
 *   aux_loss (only if cfg.aux_coeff != 0; softmax only):
 *            aux_coeff * E * sum_e (counts[e] / (T k)) * (sum_t p[t,e] / T)
 *
 * x [T,d] storage, w_router [E,d] storage, bias [E] fp32 or NULL;
 * logits [T,E] fp32 written -- or, if x and w_router are both NULL, READ as
 * precomputed router logits; topk_idx [T,k] int32, topk_gates [T,k] fp32,
 * expert_counts [E] int32 written; aux_loss [1] fp32 written when aux is on,
 * may be NULL otherwise.  T = 0 writes zero counts (and aux 0).
 * ------------------------------------------------------------------------- */
moe_status moe_router_topk(const moe_cfg* cfg, const void* x, const void* w_router,
                           const float* bias, float* logits, int32_t* topk_idx,
                           float* topk_gates, int32_t* expert_counts, float* aux_loss,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Selection-bias update without an auxiliary loss (figures page, Figure 39,
 * load-balancing strategies; the pages name the strategy, not its rule: the
 * plainest reading is taken).  After a step, each expert's selection bias
 * moves one fixed step toward balance: up if it received fewer than the mean
 * T*k/E assignments, down if more, unchanged at exactly the mean:
 *
 *   bias[e] = fp32( bias[e] + rate * sign(T*k - E*expert_counts[e]) )
 *
 * (the sign is taken on the integers, the add is one fp32 round-to-nearest).
 * expert_counts [E] int32 (moe_router_topk's output), bias [E] fp32 updated
 * in place.  Only meaningful for the sigmoid score, whose selection the bias
 * steers; accepted for any cfg.
 * ------------------------------------------------------------------------- */
moe_status moe_router_bias_update(const moe_cfg* cfg, const int32_t* expert_counts, float rate,
                                  float* bias, void* stream);

/* ---------------------------------------------------------------------------
 * Permute ("System Modules: Dispatcher" on one GPU; memory-efficient
 * permutation, Figure 7): a stable counting sort of the (token, choice) pairs
 * by expert, then each token row is copied to its k permuted rows (read once,
 * written k times).
 *
 *   expert_offsets[e] = number of assignments to experts < e  ([E+1] int32,
 *                       expert_offsets[E] = T*k)
 *   row_id_map[t,j]   = expert_offsets[e] + #{t' < t : e in topk_idx[t',:]},
 *                       e = topk_idx[t,j]                          ([T,k] int32)
 *   src_token[row]    = the token of that row                     ([T*k] int32)
 *   x_perm[row,:]     = x[src_token[row],:]                       ([T*k,d] storage)
 *   row_gates[row_id_map[t,j]] = topk_gates[t,j]                  ([T*k] fp32)
 *
 * x [T,d] storage, topk_idx [T,k] int32 (each row k distinct ids in [0,E)).
 * topk_gates [T,k] fp32 and row_gates: both or neither (the gate of each
 * permuted row; required with MOE_FLAG_FOLD_GATES, where the grouped GEMMs
 * apply it).  x_perm is the only permuted copy of the activations kept by the
 * layer.
 * ------------------------------------------------------------------------- */
moe_status moe_permute(const moe_cfg* cfg, const void* x, const int32_t* topk_idx,
                       const float* topk_gates, int32_t* expert_offsets, int32_t* row_id_map,
                       int32_t* src_token, float* row_gates, void* x_perm, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Experts ("System Modules: Experts": FFNs run as a grouped GEMM over uneven
 * expert sizes, "Key Terms: Grouped GEMM"; SwiGLU activation, Table 4; shared
 * expert processing every token, Table 1 and Figure 40).
 *
 * For each expert e over its rows r in [off[e], off[e+1]) (empty experts
 * skipped):
 *   H = x_perm[r] w13[e][0:f]^T, U = x_perm[r] w13[e][f:2f]^T   (fp32 accumulate)
 *   act[r]    = storage(g_r silu(H) * U), silu(h) = h / (1 + exp(-h)),
 *               g_r = row_gates[r] with MOE_FLAG_FOLD_GATES, else 1; with
 *               MOE_FLAG_RECOMPUTE_ACT, H and U enter as storage(H), storage(U)
 *   y_perm[r] = storage(act[r] w2[e]^T)
 *   hu_save[r] = (storage(H) | storage(U))       [T*k, 2f], if non-NULL
 * Shared expert (cfg.f_shared > 0): the same FFN with ws13/ws2 on every token
 * of x, writing act_shared [T,fs], y_shared [T,d], hu_shared_save [T,2fs].
 *
 * x_perm [T*k,d], expert_offsets [E+1] (from moe_permute), w13, w2 storage;
 * row_gates [T*k] fp32 (moe_permute's) required with MOE_FLAG_FOLD_GATES,
 * else ignored; act [T*k,f] and y_perm [T*k,d] required; hu_save optional
 * (needed by the backward call).  x, ws13, ws2, act_shared, y_shared required
 * iff f_shared > 0; hu_shared_save optional.  The shared expert's act is never
 * gated.
 * ------------------------------------------------------------------------- */
moe_status moe_grouped_gemm_swiglu(const moe_cfg* cfg, const void* x_perm,
                                   const int32_t* expert_offsets, const float* row_gates,
                                   const void* w13, const void* w2, void* hu_save, void* act,
                                   void* y_perm,
                                   const void* x, const void* ws13, const void* ws2,
                                   void* hu_shared_save, void* act_shared, void* y_shared,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* moe_grouped_gemm_swiglu for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and results (bit-identical), with
 * no workspace argument.  Its scratch (the tile prefix, E + 2 ints) lives in a
 * static device array of 4 KiB inside the library, one per GPU, held until
 * the process ends; the call allocates nothing.  cfg.dtype MOE_F32 or MOE_BF16
 * (MOE_MXFP8 -> MOE_ERR_UNSUPPORTED); E + 2 above the array's 1024 ints ->
 * MOE_ERR_INVALID_ARGUMENT (unreachable while E <= 256).  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on different streams
 * without ordering between them) race. */
moe_status moe_grouped_gemm_swiglu_noalloc(const moe_cfg* cfg, const void* x_perm,
                                           const int32_t* expert_offsets, const float* row_gates,
                                           const void* w13, const void* w2, void* hu_save, void* act,
                                           void* y_perm, const void* x, const void* ws13, const void* ws2,
                                           void* hu_shared_save, void* act_shared, void* y_shared,
                                           void* stream);

/* ---------------------------------------------------------------------------
 * Unpermute-combine ("System Modules: Combiner": tokens go back to their
 * original position and the gate-weighted sum is formed).
 *   y[t] = storage( sum_{j=0}^{k-1} gates[t,j] * y_perm[row_id_map[t,j]]
 *                   + y_shared[t] )        fp32 sum in j order, one rounding
 * With MOE_FLAG_FOLD_GATES the rows carry their gates: the sum is unweighted
 * and topk_gates is ignored (may be NULL).
 * y_perm [T*k,d], row_id_map [T,k], topk_gates [T,k] fp32, y_shared [T,d] or
 * NULL, y [T,d].
 * ------------------------------------------------------------------------- */
moe_status moe_unpermute_combine(const moe_cfg* cfg, const void* y_perm,
                                 const int32_t* row_id_map, const float* topk_gates,
                                 const void* y_shared, void* y, void* stream);

/* ===========================================================================
 * Backward.  Gradients of <y, dy> (+ d_aux * aux_loss).  Routing is held
 * fixed (top-k is piecewise constant; the selection bias gets no gradient).
 * Call order: combine_bwd -> grouped_gemm_swiglu_bwd -> router_topk_bwd ->
 * permute_bwd.
 * ========================================================================= */

/* dy_perm[row_id_map[t,j]] = storage(gates[t,j] * dy[t])          [T*k,d]
 * d_gates[t,j] = sum_i dy[t,i] * y_perm[row_id_map[t,j], i]      [T,k] fp32
 * With MOE_FLAG_FOLD_GATES: dy_perm[row_id_map[t,j]] = dy[t] (a copy: the gate
 * is inside the expert), and y_perm, topk_gates, d_gates are not used (may be
 * NULL); moe_grouped_gemm_swiglu_bwd writes d_gates. */
moe_status moe_unpermute_combine_bwd(const moe_cfg* cfg, const void* dy,
                                     const void* y_perm, const int32_t* row_id_map,
                                     const float* topk_gates, void* dy_perm,
                                     float* d_gates, void* stream);

/* Per expert e over its rows (weights of empty experts get exact zeros):
 *   dA  = dy_perm w2[e]                      (fp32, never stored)
 *   dH  = dA * U * sig(H) * (1 + H (1 - sig(H))),  dU = dA * silu(H)
 *         (H, U read from hu_save) -> dhu [T*k, 2f] = (dH | dU), storage
 *   dw2[e]  = dy_perm[rows]^T act[rows]                  [d, f]   storage
 *   dx_perm = dhu w13[e]                                 [T*k, d] storage
 *   dw13[e] = dhu[rows]^T x_perm[rows]                   [2f, d]  storage
 * MOE_FLAG_FOLD_GATES (dy_perm holds copies of dy, act carries the gates):
 *   dH, dU as above with g_r dA in place of dA, g_r = row_gates[r], and the
 *   gate gradient d_gates[t,j] = sum_c dA[r,c] silu(H[r,c]) U[r,c] of row
 *   r = row_id_map[t,j] (fp32; per row, partial sums over 64-column blocks
 *   added in order); row_gates [T*k], row_id_map [T,k], d_gates [T,k]
 *   required, else ignored.
 * MOE_FLAG_RECOMPUTE_ACT: act (and act_shared) are not read (may be NULL): the
 *   dA product forms act = storage(g_r silu(H) U) again from hu_save into the
 *   workspace, bit-identical to the forward's, and dw2 uses that.
 * Shared expert (f_shared > 0), on all tokens with upstream gradient dy:
 *   the same with ws13/ws2, hu_shared_save, act_shared, x -> dhu_shared,
 *   dws13, dws2, and its input gradient dhu_shared ws13 written in fp32 to
 *   dx_partial [T,d].  Without a shared expert dx_partial is zero-filled.
 * dx_partial is consumed by moe_router_topk_bwd (accumulates) and
 * moe_permute_bwd (reads). */
moe_status moe_grouped_gemm_swiglu_bwd(const moe_cfg* cfg, const void* dy_perm,
                                       const void* x_perm, const int32_t* expert_offsets,
                                       const float* row_gates, const int32_t* row_id_map,
                                       const void* hu_save, const void* act,
                                       const void* w13, const void* w2, void* dhu,
                                       void* dx_perm, void* dw13, void* dw2, float* d_gates,
                                       const void* dy, const void* x,
                                       const void* hu_shared_save, const void* act_shared,
                                       const void* ws13, const void* ws2, void* dhu_shared,
                                       float* dx_partial, void* dws13, void* dws2,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Router backward, from d_gates [T,k] fp32 (moe_unpermute_combine_bwd) and the
 * scalar d_aux (host value; ignored when aux is off):
 *   softmax+renorm: dl_m = scale q_m (dg_m - sum_j q_j dg_j) on the selection,
 *                   q = gates / scale (the renormalised probabilities)
 *   softmax, no renorm: dl = scale p (dg_full - sum_e p_e dg_full_e), dg_full
 *                   the d_gates scattered to their experts (0 elsewhere)
 *   aux:            dl[t,e] += d_aux p[t,e] (a_e - sum_e' p[t,e'] a_e'),
 *                   a_e = aux_coeff E counts[e] / (T k T)
 *   sigmoid:        ds_m = (scale/S)(dg_m - sum_j dg_j s_j / S), S = sum s_sel
 *                   (renorm) or scale dg_m; dl = ds s (1 - s)
 *   d_logits [T,E] fp32 written; dw_router [E,d] = d_logits^T x (storage);
 *   dx_partial [T,d] fp32 += d_logits w_router.
 * In bf16 mode the two router GEMMs consume d_logits rounded to bf16.
 * logits/topk_idx/topk_gates/expert_counts are the forward call's outputs. */
moe_status moe_router_topk_bwd(const moe_cfg* cfg, const void* x, const void* w_router,
                               const float* logits, const int32_t* topk_idx,
                               const float* topk_gates, const int32_t* expert_counts,
                               const float* d_gates, float d_aux, float* d_logits,
                               void* dw_router, float* dx_partial, void* workspace,
                               size_t workspace_bytes, void* stream);

/* dx[t] = storage( dx_partial[t] + sum_{j=0}^{k-1} dx_perm[row_id_map[t,j]] )
 * (fp32 sum, j in order, one rounding).  dx_partial may be NULL (zeros). */
moe_status moe_permute_bwd(const moe_cfg* cfg, const void* dx_perm,
                           const int32_t* row_id_map, const float* dx_partial, void* dx,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timing trace (a profiling aid; no computation depends on it).
 * moe_trace_begin(capacity) starts a trace on the calling host thread: every
 * kernel the library enqueues afterwards is bracketed by two HIP events
 * recorded on that kernel's stream, for up to `capacity` kernels (later ones
 * are not traced).  It creates 2*capacity events (no device memory).
 * moe_trace_end(names, ms, capacity) stops the trace, waits for the recorded
 * events, writes up to `capacity` kernel names (static strings) and durations
 * in milliseconds, destroys the events and returns the number of kernels
 * traced (or -1 on a HIP error).  Do not trace inside a hipGraph capture.
 * ------------------------------------------------------------------------- */
moe_status moe_trace_begin(int capacity);
int moe_trace_end(const char** names, float* ms, int capacity);

/* ---------------------------------------------------------------------------
 * MXFP8 ("microscaling FP8": thelatestinai.com page, Figure 30, FP8 training
 * recipes, and Table 11, Dtype column; Figure 31 on quantisation granularity
 * and the tensor layouts each GEMM needs; Table 8, quantisation kernel
 * overhead).  A tensor becomes fp8 e4m3fn codes (one byte per value) plus one
 * e8m0 scale byte per 32 consecutive values along a chosen dimension:
 *
 *   scale byte = e + 127, e the smallest integer with 448 * 2^e >= the block's
 *                largest magnitude, clamped to [-127, 127] (an all-zero block
 *                gives byte 0 and zero codes)
 *   code       = the e4m3fn value nearest to v / 2^e, ties to the even code,
 *                saturating at +-448;   value = decode(code) * 2^(byte - 127)
 *
 * A GEMM contracts each operand along its blocked dimension, so the expert
 * weights are needed in both orientations (quantised once per weight update,
 * outside the layer calls); activations are quantised inside the layer calls.
 * ------------------------------------------------------------------------- */
typedef enum moe_mx_orientation {
  MOE_MX_ROWS = 0,  /* blocks along the contiguous dimension: codes [B][R][C],
                       scales [B][R][C/32]; C % 32 == 0                        */
  MOE_MX_COLS = 1,  /* transposed copy, blocks along R: codes [B][C][R],
                       scales [B][C][R/32]; R % 32 == 0, C % 8 == 0            */
  MOE_MX_GROUPED = 2 /* flag (OR-ed into the orientation, or the `flags` of the
                       _both calls): scales in the grouped layout below       */
} moe_mx_orientation;

/* Grouped scale layout.  For a quantised matrix of R' rows (R for
 * MOE_MX_ROWS, C for MOE_MX_COLS) with nb blocks of 32 per row (nb a multiple
 * of 4: the blocked dimension a multiple of 128), the four scales of blocks
 * 4q .. 4q+3 of row r form one 4-byte word, and word (q, r) is at index
 * q * R' + r: the scale of block b of row r is byte 4 (floor(b/4) R' + r) +
 * b % 4 of the matrix's R' nb bytes (a batch's matrices follow each other as
 * in the plain layout).  Codes are unchanged.  The microscaled layer calls
 * read the expert weights' scales in this layout: a slice of 128 fp8 (256
 * fp4) values along K is one (two) word(s) per row, and a tile's rows then
 * fetch adjacent words. */

/* Quantises `batch` row-major bf16 matrices src [batch][rows][cols] in the
 * given orientation.  codes 16-byte aligned; rows * cols < 2^31; batch <=
 * 65535.  Deterministic and bit-exact to the rule above. */
moe_status moe_quantize_mxfp8(const void* src, int64_t batch, int64_t rows, int64_t cols,
                              int32_t orientation, uint8_t* codes, uint8_t* scales, void* stream);

/* Both orientations of the same matrices in one pass, each bf16 value read
 * once: codes_rows / scales_rows exactly as MOE_MX_ROWS | flags, codes_cols /
 * scales_cols exactly as MOE_MX_COLS | flags would give them.  flags: 0 or
 * MOE_MX_GROUPED (then rows and cols multiples of 128).  rows and cols
 * multiples of 32; other limits and errors as moe_quantize_mxfp8.  For the
 * callers that quantise expert weights (both forms, once per update). */
moe_status moe_quantize_mxfp8_both(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                   uint8_t* codes_rows, uint8_t* scales_rows, uint8_t* codes_cols,
                                   uint8_t* scales_cols, int32_t flags, void* stream);

/* One quantised operand (device memory): codes 16-byte, scales 4-byte aligned. */
typedef struct moe_mx_tensor {
  const uint8_t* codes;
  const uint8_t* scales;
} moe_mx_tensor;

/* Expert weights for the MXFP8 calls, each in the orientation its GEMM
 * contracts (MOE_MX_ROWS of the tensor named, or of its per-expert transpose),
 * scales in the grouped layout (MOE_MX_GROUPED):
 *   w13   codes [E][2f][d]  scales [E][2f][d/32]   forward gate/up (along d)
 *   w2    codes [E][d][f]   scales [E][d][f/32]    forward down (along f)
 *   w13_t codes [E][d][2f]  scales [E][d][2f/32]   dX = dHU W13 (along 2f)
 *   w2_t  codes [E][f][d]   scales [E][f][d/32]    dA = dY W2 (along d)
 *   ws13, ws2, ws13_t, ws2_t: the shared expert's, same layouts without [E]
 *                                        (ignored when f_shared = 0)
 * w13 and w13_t are moe_quantize_mxfp8_both(w13, E, 2f, d, ..., MOE_MX_GROUPED)
 * (w13_t alone: moe_quantize_mxfp8(w13, E, 2f, d, MOE_MX_COLS | MOE_MX_GROUPED)). */
typedef struct moe_mx_weights {
  moe_mx_tensor w13, w2, w13_t, w2_t;
  moe_mx_tensor ws13, ws2, ws13_t, ws2_t;
} moe_mx_weights;

/* moe_grouped_gemm_swiglu with MXFP8 expert GEMMs (cfg.dtype = MOE_MXFP8;
 * d, f, f_shared multiples of 128).  Same tensors and semantics, except that
 * x_perm (and x for the shared expert) is quantised along d before GEMM1 and
 * the bf16 act along f before GEMM2; weights come quantised in `weights`
 * (host pointer to the struct; its members are device pointers).  fp32
 * accumulation, bf16 outputs. */
moe_status moe_grouped_gemm_swiglu_mxfp8(const moe_cfg* cfg, const void* x_perm,
                                         const int32_t* expert_offsets, const float* row_gates,
                                         const moe_mx_weights* weights, void* hu_save, void* act,
                                         void* y_perm, const void* x, void* hu_shared_save,
                                         void* act_shared, void* y_shared, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* moe_grouped_gemm_swiglu_bwd with MXFP8 GEMMs.  Every GEMM quantises its two
 * operands along the dimension it contracts: dY_perm along d (dA = dY W2,
 * with weights->w2_t), dHU along 2f (dX = dHU W13, with weights->w13_t), and
 * for the weight gradients dY_perm, act, dHU and x_perm along their rows, in
 * blocks of 32 rows that restart at each expert's first row (rows past the
 * expert's end count as zeros); the shared expert likewise over all T rows.
 * The weight gradients multiply those quantised values widened to bf16 (every
 * e4m3 or e2m1 value times its power-of-two scale is a bf16 value, blocks
 * scaled at the clamp 2^-127 aside): the same products, accumulated in fp32.
 * Same outputs as the bf16 call (dx_partial written, not accumulated). */
moe_status moe_grouped_gemm_swiglu_bwd_mxfp8(const moe_cfg* cfg, const void* dy_perm,
                                             const void* x_perm, const int32_t* expert_offsets,
                                             const float* row_gates, const int32_t* row_id_map,
                                             const void* hu_save, const void* act,
                                             const moe_mx_weights* weights, void* dhu, void* dx_perm,
                                             void* dw13, void* dw2, float* d_gates, const void* dy,
                                             const void* x,
                                             const void* hu_shared_save, const void* act_shared,
                                             void* dhu_shared, float* dx_partial, void* dws13,
                                             void* dws2, void* workspace, size_t workspace_bytes,
                                             void* stream);

/* ---------------------------------------------------------------------------
 * MXFP4 (the gfx950 counterpart of the NVFP4 format the pages' system trains
 * with: papers.lunadong.com summary, "Technical Details" and "Key Terms";
 * thelatestinai.com page, Table 8 on FP4 activation memory).  The MXFP8 block
 * structure with fp4 e2m1 elements -- one sign bit, two exponent bits (bias 1),
 * one mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6:
 *
 *   scale byte = e + 127, e the smallest integer with 6 * 2^e >= the block's
 *                largest magnitude, clamped to [-127, 127] (all-zero block:
 *                byte 0, zero codes)
 *   code       = the e2m1 value nearest to v / 2^e, ties to the even code,
 *                saturating at +-6
 *
 * Codes are stored two per byte along the blocked dimension, element 2i in the
 * low nibble: MOE_MX_ROWS gives codes [B][R][C/2] and scales [B][R][C/32],
 * MOE_MX_COLS codes [B][C][R/2] and scales [B][C][R/32] (same size rules as
 * moe_quantize_mxfp8).
 * ------------------------------------------------------------------------- */
moe_status moe_quantize_mxfp4(const void* src, int64_t batch, int64_t rows, int64_t cols, int32_t orientation,
                              uint8_t* codes, uint8_t* scales, void* stream);
/* moe_quantize_mxfp8_both with e2m1 codes (two per byte) */
moe_status moe_quantize_mxfp4_both(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                   uint8_t* codes_rows, uint8_t* scales_rows, uint8_t* codes_cols,
                                   uint8_t* scales_cols, int32_t flags, void* stream);

/* moe_grouped_gemm_swiglu_mxfp8 and moe_grouped_gemm_swiglu_bwd_mxfp8 with
 * MXFP4 operands (cfg.dtype = MOE_MXFP4; d, f, f_shared multiples of 256, one
 * 128-byte code slice per row).  `weights` holds moe_quantize_mxfp4 forms in
 * the moe_mx_weights layouts (code widths halved: w13 codes [E][2f][d/2],
 * w13_t [E][d][f], ...); the same seven expert products are quantised along
 * their contractions inside the calls; the weight gradients' 32-row blocks
 * restart at each expert's first row as in MXFP8.  Same outputs, workspace
 * (moe_workspace_size of the MOE_MXFP4 cfg) and errors. */
moe_status moe_grouped_gemm_swiglu_mxfp4(const moe_cfg* cfg, const void* x_perm,
                                         const int32_t* expert_offsets, const float* row_gates,
                                         const moe_mx_weights* weights, void* hu_save, void* act,
                                         void* y_perm, const void* x, void* hu_shared_save,
                                         void* act_shared, void* y_shared, void* workspace,
                                         size_t workspace_bytes, void* stream);
moe_status moe_grouped_gemm_swiglu_bwd_mxfp4(const moe_cfg* cfg, const void* dy_perm,
                                             const void* x_perm, const int32_t* expert_offsets,
                                             const float* row_gates, const int32_t* row_id_map,
                                             const void* hu_save, const void* act,
                                             const moe_mx_weights* weights, void* dhu, void* dx_perm,
                                             void* dw13, void* dw2, float* d_gates, const void* dy,
                                             const void* x,
                                             const void* hu_shared_save, const void* act_shared,
                                             void* dhu_shared, float* dx_partial, void* dws13,
                                             void* dws2, void* workspace, size_t workspace_bytes,
                                             void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_GFX950_H */
