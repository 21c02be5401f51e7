/*
 * moe.h -- C ABI of libmoe.so, the MI355X (gfx950) sparse mixture-of-experts
 * feed-forward layer (Mixtral: E = 8 experts, top-2 routing, SwiGLU experts).
 *
 * The layer, per token x (a row of length d):
 *   l = x W_g^T (+ b)               8 router scores, one per expert
 *   (a, b) = the two largest scores, larger first, ties to the lower index;
 *            every other score becomes -inf
 *   g = softmax over the surviving pair  (g_a = 1/(1+exp(l_b-l_a)), g_b = 1-g_a)
 *   o_e = (SiLU(x w1_e^T) * (x w3_e^T)) w2_e^T   for e in {a, b}
 *   y = g_a o_a + g_b o_b           (dropless: every token gets both experts)
 * Sources: "Mixtral of Experts" (azimuth.plus), router paragraph (linear map
 * x W_g to 8 scores, top-2 kept, others -inf, softmax over the survivors)
 * and architecture paragraph (SwiGLU experts with their own weights);
 * "Mixtral > Architecture Overview" (mbrenndoerfer.com), hyperparameter list
 * (d = 4096, f = 14336, 8 experts, 2 active) and parameter-count paragraph
 * (gate, up and down projections); "Mixtral & Sparse MoE (2024) > The
 * Solution" (mbrenndoerfer.com), routing paragraph (outputs combined by the
 * routing scores, each token routed on its own).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensor pointers are DEVICE pointers to row-major, contiguous arrays,
 *   16-byte aligned.  Scalars and the dims struct are host memory.
 * - Layouts: x [T, d]; w_gate [E, d] (one row per expert: the transpose of
 *   the d x E map the router multiplies by); w1 (gate) and w3 (up) [E, f, d];
 *   w2 (down) [E, d, f]; logit_bias [E] fp32 or NULL.
 * - dtype MOE_BF16: x, weights, h and y are bf16; accumulation, router
 *   scores, gates and y_rows are fp32; h and y are rounded to nearest even.
 *   dtype MOE_F32: everything fp32.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   work is enqueued on it; calls return right after enqueueing and never
 *   synchronise, allocate, free, or keep a pointer after returning.
 * - Errors: every argument is checked on the host before anything is
 *   enqueued; on error nothing is enqueued and outputs are untouched.
 *   NULL required pointer, T < 0, misaligned pointer -> MOE_ERR_INVALID_ARGUMENT;
 *   E != 8, k != 2, d or f not a multiple of 128, unknown dtype/variant/gating,
 *   or a size above a stated limit -> MOE_ERR_UNSUPPORTED;
 *   T == 0 -> MOE_OK with nothing enqueued.  A failed launch -> MOE_ERR_HIP
 *   (outputs unspecified).  Device faults surface at the caller's next sync.
 * - Calls on one stream are ordered; the library holds no mutable state
 *   besides a lazily filled, lock-protected per-device property cache.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Kernel family for the expert GEMMs.  AUTO picks DECODE (weight streaming,
 * token groups of 16 on MFMA) when T <= 128 and PREFILL (LDS-tiled grouped
 * GEMM) otherwise; DECODE forced streams up to T = 128 (more rows per expert
 * use register-direct kernels).  Both compute the same function; the choice only affects
 * speed.  PREFILL needs d >= 256, f >= 256 and x below 4 GiB (T * d < 2^31);
 * other bf16 layers always run DECODE.  MOE_F32 always uses its own fp32
 * kernels. */
typedef enum { MOE_VARIANT_AUTO = 0, MOE_VARIANT_DECODE = 1, MOE_VARIANT_PREFILL = 2 } moe_variant;

/* Expert capacity (moe_dims.capacity = C > 0): each expert keeps its first C
 * slots in slot order (slot s = t*k + j: earlier tokens first, a token's
 * larger score before its smaller) and drops the rest; a dropped slot adds
 * nothing to its token's output and the token's other gate is not
 * renormalised (a token with both slots dropped outputs zero).  Reading of
 * "Mixtral & Sparse MoE (2024) > The Solution" (mbrenndoerfer.com),
 * load-balancing paragraph: capacity constraints limit the tokens routed to
 * each expert (the page gives no rule for which; this is the plainest). */

/* Gates of the two kept experts.  PAIR (Mixtral, the default): softmax over
 * the kept pair with every other score at -inf, g_a = 1/(1+exp(l_b-l_a)),
 * g_b = 1 - g_a ("Mixtral of Experts", azimuth.plus, router paragraph).
 * FULL: softmax over all E scores first, then the two largest
 * probabilities as they stand, g_e = exp(l_e) / sum_j exp(l_j), which sum to
 * less than 1 ("Mixtral & Sparse MoE (2024) > The Solution",
 * mbrenndoerfer.com, routing paragraph, read literally).  Both select the
 * same experts; the outputs differ by the factor g_a + g_b. */
typedef enum { MOE_GATING_PAIR = 0, MOE_GATING_FULL = 1 } moe_gating;

typedef struct {
  int64_t T;        /* tokens, >= 0; T * k must fit in int32 */
  int32_t d;        /* hidden size, multiple of 128 */
  int32_t f;        /* expert FFN width, multiple of 128 */
  int32_t E;        /* experts, must be 8 */
  int32_t k;        /* experts per token, must be 2 */
  int32_t dtype;    /* moe_dtype */
  int32_t variant;  /* moe_variant */
  int32_t gating;   /* moe_gating (0 = PAIR) */
  int32_t capacity; /* slots each expert keeps, >= 0; 0 = no limit (dropless, Mixtral) */
} moe_dims;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* Library version, e.g. "1.0.0" (static string). */
const char* moe_version(void);

/*
 * Router: scores, top-2 selection and the softmax over the kept pair.
 * "Mixtral of Experts" (azimuth.plus), router paragraph.
 *   x [T, d] (dtype), w_gate [E, d] (dtype), logit_bias [E] fp32 or NULL
 *   (added to every token's scores; a workload device, not part of Mixtral).
 *   Outputs: topk_idx [T, 2] int32 (slot 0 = larger score, ties to the lower
 *   index), topk_w [T, 2] fp32 (>= 0; sum 1 with MOE_GATING_PAIR, below 1
 *   with MOE_GATING_FULL), logits [T, E] fp32 or NULL.
 *   Scores are accumulated in fp32.  Limit: E * d * elem_size <= 128 KiB
 *   (the router matrix is staged in LDS), i.e. d <= 8192 for bf16.
 */
moe_status moe_router_topk(const moe_dims* dims, const void* x, const void* w_gate,
                           const float* logit_bias, int32_t* topk_idx, float* topk_w,
                           float* logits, void* stream);

/*
 * Expert-major permutation of the token slots (slot s = t * k + j is token
 * t's j-th expert).  It groups each expert's tokens so the expert GEMMs read
 * them contiguously; it changes no value ("Mixtral & Sparse MoE (2024) > The
 * Solution", routing paragraph: each token is routed on its own).
 *   topk_idx [T, k] int32 (an id outside [0, E) gets no row: its slot is
 *   treated like a dropped one, slot_rows = -1).
 *   Outputs: expert_offsets [E + 1] int32 (exclusive prefix sum of the per-
 *   expert rows; offsets[E] = T * k without a capacity), sorted_slots
 *   [T * k] int32 (slots of expert 0 in increasing slot id, then expert 1,
 *   ...: a stable order; entries past offsets[E] are left as they were),
 *   slot_rows [T * k] int32 (inverse: position of slot s in sorted_slots, or
 *   -1 for a slot dropped by dims->capacity).
 *   workspace: caller-owned device memory, 16-byte aligned, for per-group
 *   counts (ceil(T/16) * E int32 when 512 < T <= 65536; at least 256 bytes
 *   otherwise); workspace == NULL is a size query as in moe_ffn_forward.
 *   Deterministic (no atomics).  Up to 512 tokens one workgroup; up to 65536
 *   tokens one launch counts each 16-token group's slots per expert and a
 *   second places them, one wave per group; beyond, one workgroup.
 */
moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_offsets,
                       int32_t* sorted_slots, int32_t* slot_rows, void* workspace, size_t* workspace_bytes,
                       void* stream);

/*
 * Both expert projections for every slot, in expert-major order:
 *   h[r, :]      = SiLU(x[tok] w1_e^T) * (x[tok] w3_e^T)   (dtype)
 *   y_rows[r, :] = h[r, :] w2_e^T                          (fp32)
 * for r in [offsets[e], offsets[e+1]), tok = sorted_slots[r] / k.
 * "Mixtral of Experts" (azimuth.plus), architecture paragraph (SwiGLU
 * experts); "Mixtral > Architecture Overview" (mbrenndoerfer.com),
 * parameter-count paragraph (gate, up and down projections).
 *   expert_offsets [E + 1], sorted_slots [T * k] as produced by moe_permute
 *   (device memory; the host never reads them).  h [T * k, f] and
 *   y_rows [T * k, d] are caller-owned outputs.
 */
moe_status moe_grouped_swiglu(const moe_dims* dims, const void* x, const int32_t* expert_offsets,
                              const int32_t* sorted_slots, const void* w1, const void* w3,
                              const void* w2, void* h, float* y_rows, void* stream);

/*
 * The two halves of moe_grouped_swiglu as separate calls (same kernels), so
 * that each projection can be timed or checked on its own:
 *   moe_expert_up:   h[r, :] = SiLU(x[tok] w1_e^T) * (x[tok] w3_e^T)   (dtype)
 *   moe_expert_down: y_rows[r, :] = h[r, :] w2_e^T                     (fp32)
 * Arguments, layouts and sources as for moe_grouped_swiglu.
 */
moe_status moe_expert_up(const moe_dims* dims, const void* x, const int32_t* expert_offsets,
                         const int32_t* sorted_slots, const void* w1, const void* w3, void* h, void* stream);
moe_status moe_expert_down(const moe_dims* dims, const void* h, const int32_t* expert_offsets, const void* w2,
                           float* y_rows, void* stream);

/*
 * Gate-weighted combine: y[t, :] = topk_w[t, 0] * y_rows[slot_rows[2t], :]
 *                                 + topk_w[t, 1] * y_rows[slot_rows[2t+1], :]
 * added in that order in fp32, then rounded once to dtype.
 * "Mixtral & Sparse MoE (2024) > The Solution" (mbrenndoerfer.com), routing
 * paragraph; "Mixtral of Experts" (azimuth.plus), router paragraph (the
 * gates set how much each expert's output contributes).
 *   y_rows [T * k, d] fp32, slot_rows [T * k] int32, topk_w [T, k] fp32,
 *   y [T, d] (dtype, output).
 */
moe_status moe_combine(const moe_dims* dims, const float* y_rows, const int32_t* slot_rows,
                       const float* topk_w, void* y, void* stream);

/*
 * The whole layer: router -> permute -> grouped SwiGLU experts -> combine.
 *   x, w_gate, logit_bias, w1, w3, w2 as above; y [T, d] (dtype) output.
 *   Optional outputs (NULL to skip): topk_idx_out [T, 2] int32,
 *   topk_w_out [T, 2] fp32, expert_counts_out [E] int32.
 *   workspace: caller-owned device memory, 256-byte aligned.  With
 *   workspace == NULL the call only writes the required size to
 *   *workspace_bytes and returns MOE_OK (nothing enqueued).  Otherwise
 *   *workspace_bytes is its size; too small -> MOE_ERR_WORKSPACE_TOO_SMALL.
 *   The workspace holds the routing, permutation, h [T*k, f] and
 *   y_rows [T*k, d]; its contents after the call are unspecified.
 */
moe_status moe_ffn_forward(const moe_dims* dims, const void* x, const void* w_gate,
                           const float* logit_bias, const void* w1, const void* w3, const void* w2,
                           void* y, int32_t* topk_idx_out, float* topk_w_out,
                           int32_t* expert_counts_out, void* workspace, size_t* workspace_bytes,
                           void* stream);

/*
 * moe_ffn_forward with its stages timed, for measurement: the same launches
 * on the same stream, with an event recorded at each stage boundary.
 *   stage_events: 8 hipEvent_t handles (passed as void*), created by the
 *   caller; event i is recorded before stage i and event i+1 after it, for
 *   the stages router, permute, up GEMM, up remainder fixup and expert
 *   tails, down GEMM, down tails and fixup, combine.  A
 *   stage the chosen kernels do not have gets two back-to-back events.
 *   up_gemm_clock: NULL, or int64 [4 * G] in device memory with G the
 *   CU count rounded down to a multiple of 8 (256 on MI355X); when the layer
 *   runs the prefill up GEMM, its clock-recording twin (same kernel, plus
 *   two counter reads) stores per workgroup b the shader clock counter at
 *   start and end and the constant 100 MHz reference counter at start and
 *   end in [4b .. 4b+3]; otherwise the buffer is left as it was.
 * The sum of the seven stages is the layer: moe_ffn_forward's output and
 * routing are computed exactly as by moe_ffn_forward.  Other arguments,
 * errors and workspace as moe_ffn_forward (a NULL stage_events array or
 * event -> MOE_ERR_INVALID_ARGUMENT).  The events' timing is the caller's.
 */
moe_status moe_ffn_forward_timed(const moe_dims* dims, const void* x, const void* w_gate,
                                 const float* logit_bias, const void* w1, const void* w3,
                                 const void* w2, void* y, int32_t* topk_idx_out, float* topk_w_out,
                                 int32_t* expert_counts_out, void* workspace, size_t* workspace_bytes,
                                 void* stream, void* const* stage_events, int64_t* up_gemm_clock);

/*
 * Measurement: the bf16 matrix-core ceiling of this GPU under its power
 * limit.  Runs the prefill GEMM's MFMA pattern alone (each wave issues the
 * 64 v_mfma_f32_16x16x32_bf16 of its 128 x 128 tile per 32-deep step,
 * `iters` times, on distinct fragments of the caller's data; one wave per
 * SIMD on G workgroups, G = the CU count rounded down to a multiple of 8)
 * and stores per workgroup b the shader clock counter and the constant
 * 100 MHz reference counter at the loop's start and end in
 * clock_out[4b .. 4b+3].  Flops = G * 4 * 64 * iters * 16384.
 *   operands: 32768 bf16 in device memory (64 fragments of 64 lanes x 8),
 *   16-byte aligned; sink: G * 256 fp32 (written, keeps the work live).
 *   NULL pointer, misalignment or iters < 1 -> MOE_ERR_INVALID_ARGUMENT.
 */
moe_status moe_mfma_ceiling(const void* operands, int64_t* clock_out, float* sink, int32_t iters,
                            void* stream);

/*
 * The whole layer from a routing computed elsewhere (by
 * moe_rmsnorm_residual_route, or any top-2 pairs and gates): permutation,
 * both expert projections and the combine, as moe_ffn_forward without its
 * router.  topk_idx [T, 2] int32 (an id outside [0, E) adds nothing), topk_w [T, 2] fp32, as
 * moe_router_topk writes them; dims->capacity applies; dims->gating is not
 * used.  Workspace as moe_ffn_forward (same size query).
 */
moe_status moe_ffn_forward_routed(const moe_dims* dims, const void* x, const int32_t* topk_idx,
                                  const float* topk_w, const void* w1, const void* w3, const void* w2,
                                  void* y, int32_t* expert_counts_out, void* workspace,
                                  size_t* workspace_bytes, void* stream);

/*
 * moe_ffn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the workspace is a fixed device array
 * inside the library, 32 MiB (33554432 bytes) per GPU, held from the first
 * call on that GPU until the process ends.  The call allocates nothing.
 *   Arguments, outputs and errors as moe_ffn_forward; a layer whose
 *   workspace (moe_ffn_forward's size query) exceeds 32 MiB is rejected with
 *   MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (at d = 4096,
 *   f = 14336: up to 272 tokens with the kernels AUTO picks, 372 with the
 *   decode kernels forced).  All calls on one GPU share its array and it keeps the last
 *   call's contents (the layer writes every region before reading it, so
 *   nothing needs clearing): calls that overlap on one GPU -- on different
 *   streams or from different threads without ordering -- race and give
 *   undefined results.  Calls on one stream are ordered and safe.
 */
moe_status moe_ffn_forward_noalloc(const moe_dims* dims, const void* x, const void* w_gate,
                                   const float* logit_bias, const void* w1, const void* w3,
                                   const void* w2, void* y, int32_t* topk_idx_out, float* topk_w_out,
                                   int32_t* expert_counts_out, void* stream);

/*
 * One stacked block's MoE half with the combine fused into the glue that
 * follows it: moe_ffn_forward_routed on x (the layer's input u_l) and its
 * routing, except that the gate-weighted pair of each token's expert rows is
 * added straight into the fp32 residual instead of being written as y, then
 * u_out = resid / sqrt(mean(resid^2) + eps) and, when w_gate_next is given,
 * the next layer's pair and gates from the rounded u_out, as
 * moe_rmsnorm_residual_route computes them.  The added row is the layer's
 * output y rounded to dtype exactly as moe_combine rounds it, so the result
 * equals moe_ffn_forward_routed followed by moe_rmsnorm_residual_route bit
 * for bit, without y's round trip through memory.  ("Mixtral & Sparse MoE
 * (2024) > The Solution", routing paragraph: outputs combined by the routing
 * scores; "Mixtral > Architecture Overview", layer-components list: the
 * blocks are stacked on a residual stream.)
 *   resid [T, d] fp32 in/out, u_out [T, d] (dtype) output; u_out may be x
 *   and topk_idx_next / topk_w_next may be topk_idx / topk_w (each is read
 *   before it is overwritten).  w_gate_next [E, d], logit_bias_next [E] or
 *   NULL; with w_gate_next NULL no routing is computed (after the last
 *   layer).  Limits: d <= 8192, and E * d * elem_size <= 128 KiB when
 *   routing.  Workspace and its size query as moe_ffn_forward.
 */
moe_status moe_ffn_forward_routed_residual(const moe_dims* dims, const void* x, const int32_t* topk_idx,
                                           const float* topk_w, const void* w1, const void* w3,
                                           const void* w2, float* resid, void* u_out, float eps,
                                           const void* w_gate_next, const float* logit_bias_next,
                                           int32_t* topk_idx_next, float* topk_w_next,
                                           int32_t* expert_counts_out, void* workspace,
                                           size_t* workspace_bytes, void* stream);

/*
 * Auxiliary load-balancing loss, loss[0] = E * sum_e f_e * P_e, with f_e the
 * fraction of the T * k slots whose router choice is expert e (before any
 * capacity) and P_e the mean over tokens of the softmax over all E scores at
 * e: 1 for an even router, up to E when the work collapses onto one expert.
 * "Mixtral & Sparse MoE (2024) > The Solution", load-balancing paragraph
 * (auxiliary losses push towards an even spread of work; the page gives no
 * formula, this is the usual product form).
 *   logits [T, E] fp32 (moe_router_topk's optional output), topk_idx [T, k]
 *   int32, loss: one fp32 in device memory.  One workgroup, deterministic
 *   (fixed reduction order).  T == 0: nothing is enqueued (loss untouched).
 */
moe_status moe_load_balance_loss(const moe_dims* dims, const float* logits, const int32_t* topk_idx,
                                 float* loss, void* stream);

/*
 * Glue between stacked layers (not part of the MoE layer itself; the
 * pages' decoder blocks are stacked with a residual stream, "Mixtral >
 * Architecture Overview", layer-components list):
 *   resid[t, :] += y_add[t, :]            (if y_add != NULL; fp32 residual)
 *   u[t, :] = resid[t, :] / sqrt(mean(resid[t, :]^2) + eps)   (unit gain)
 *   resid [T, d] fp32 in/out, y_add [T, d] (dtype) or NULL, u_out [T, d]
 *   (dtype) output.  d must be a multiple of 128 and at most 16384.
 */
moe_status moe_rmsnorm_residual(int64_t T, int32_t d, float* resid, const void* y_add, void* u_out,
                                float eps, int32_t dtype, void* stream);

/*
 * moe_rmsnorm_residual fused with the router of the layer that follows:
 * resid += y_add (if given), u = resid / sqrt(mean(resid^2) + eps) in
 * dims->dtype, then that layer's top-2 pair and gates from the rounded u
 * exactly as moe_router_topk computes them (dims->gating; w_gate [E, d],
 * logit_bias [E] or NULL), written to topk_idx [T, 2] and topk_w [T, 2].
 * One read of the residual row serves both steps (the stacked-layer glue
 * and "Mixtral of Experts", azimuth.plus, router paragraph).  Limits: d <=
 * 8192 and E * d * elem_size <= 128 KiB.
 */
moe_status moe_rmsnorm_residual_route(const moe_dims* dims, float* resid, const void* y_add, void* u_out,
                                      float eps, const void* w_gate, const float* logit_bias,
                                      int32_t* topk_idx, float* topk_w, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
