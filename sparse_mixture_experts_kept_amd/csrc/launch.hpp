// Internal launchers of libmoe (host side).  Each enqueues its kernels on
// `s` and returns the launch status; argument validation happens in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// Gating of the kept pair (values of moe_dims.gating).
constexpr int kGatingPair = 0;  // softmax over the kept pair (weights sum to 1)
constexpr int kGatingFull = 1;  // softmax over all scores, pair not renormalised

// group_counts (bf16 only, may be null): [ceil(T/16), 8] int32, the slots of
// each 16-token group per expert, for launch_permute_groups.
hipError_t launch_router(int dtype, const void* x, const void* wg, const float* bias, int32_t* idx, float* w,
                         float* logits, int64_t T, int d, int gating, int n_cu, hipStream_t s,
                         int32_t* group_counts = nullptr);

// Slot counts up to this take the one-workgroup ballot form (one slot per thread).
constexpr int64_t kPermuteSmallSlots = 1024;
// capacity > 0: each expert keeps its first `capacity` slots (slot order);
// dropped slots get slot_rows = -1.
hipError_t launch_permute(const int32_t* idx, int32_t n_slots, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_rows, int32_t* counts_out, int capacity, hipStream_t s);
// The same permutation from the router's per-group counts: one wave per
// 16-token group.  n_tokens <= kMaxGroupPermuteTokens.
constexpr int64_t kMaxGroupPermuteTokens = 65536;
hipError_t launch_permute_groups(const int32_t* idx, int32_t n_tokens, const int32_t* group_counts, int32_t* offsets,
                                 int32_t* sorted_slots, int32_t* slot_rows, int32_t* counts_out, int capacity,
                                 hipStream_t s);
// The same from the ids alone: a first launch counts each group's slots
// per expert into group_counts [ceil(n_tokens/16), 8] int32.
hipError_t launch_permute_counted(const int32_t* idx, int32_t n_tokens, int32_t* group_counts, int32_t* offsets,
                                  int32_t* sorted_slots, int32_t* slot_rows, int32_t* counts_out, int capacity,
                                  hipStream_t s);
// loss[0] = E * sum_e f_e * P_e from the scores [T, E] and the pairs [T, k].
hipError_t launch_load_balance_loss(const float* logits, const int32_t* idx, int64_t T, float* loss, hipStream_t s);

// Expert projections.  up: h = SiLU(x w1^T) * (x w3^T) over the gathered
// rows; down: y_rows = h w2^T.  n_slots = T * k.
hipError_t launch_up_f32(const float* x, const int32_t* offs, const int32_t* sorted_slots, const float* w1,
                         const float* w3, float* h, int64_t n_slots, int d, int f, hipStream_t s);
hipError_t launch_down_f32(const float* h, const int32_t* offs, const float* w2, float* y_rows, int64_t n_slots,
                           int d, int f, hipStream_t s);

// Split down-projection tails (launch_down_tail_stream with a buffer): the
// first kTailPartHeader floats hold an int, the part count P the launch
// chose (1: it wrote y_rows itself), then P x 8 experts x kTailPartRows rows
// x d fp32 partial sums, row m of expert e's tail at ((p*8 + e)*32 + m)*d.
constexpr int kTailPartHeader = 64;
constexpr int kTailPartRows = 32;
constexpr int kMaxTailParts = 8;
// Parts that fit a buffer of `bytes` (0 without a buffer).
inline int tail_part_capacity(const float* p, int64_t bytes, int d) {
  if (!p || bytes <= kTailPartHeader * 4) return 0;
  const int64_t n = (bytes - kTailPartHeader * 4) / (int64_t{8} * kTailPartRows * d * 4);
  return n > kMaxTailParts ? kMaxTailParts : static_cast<int>(n);
}

// The prefill kernels handle the layer: d, f multiples of 128 and >= 256,
// and x (T x d bf16) smaller than 4 GiB.
bool prefill_fits(int64_t T, int d, int f);
// thin_elsewhere: skip the rows of each expert's last 256-row tile when it
// holds at most 32 of them and the expert has more than 256 rows (the tail
// launchers below compute exactly those rows).
// partials (may be null): an fp32 buffer of partial_bytes for the remainder
// split of the work units (the up projection's, then the down projection's:
// both launches are stream-ordered); it adds a fixup launch.
// clk (may be null): launch the clock-recording twin of the up GEMM, which
// stores per workgroup {shader cycles at start, at end, 100 MHz reference
// ticks at start, at end} in clk[4 * prefill_grid(n_cu)] int64.
// after_gemm (may be null): recorded on s right after the GEMM launch
// (before the remainder fixup).
int prefill_grid(int n_cu);
hipError_t launch_up_prefill(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                             const bf16_t* w3, bf16_t* h, int d, int f, int n_cu, bool thin_elsewhere,
                             float* partials, int64_t partial_bytes, hipStream_t s, long long* clk = nullptr,
                             hipEvent_t after_gemm = nullptr);
// split == 2: two partial sums over the two halves of f, the second at
// y_rows + split_stride; otherwise one full sum in y_rows, and with
// partials the remainder units' rows are completed by
// launch_down_prefill_fixup (after the tail launch, whose split partial sums
// it also adds when tail_part is given).
hipError_t launch_down_prefill(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int d, int f,
                               int n_cu, int split, int64_t split_stride, bool thin_elsewhere, float* partials,
                               int64_t partial_bytes, hipStream_t s);
hipError_t launch_down_prefill_fixup(const int32_t* offs, const float* partials, int64_t partial_bytes,
                                     const float* tail_part, float* y_rows, int d, int f, int n_cu,
                                     bool thin_elsewhere, hipStream_t s);
// The rows the prefill launches skip with thin_elsewhere, on the streaming
// kernels (full reduction: with split == 2 the tail rows' second partial
// must be zero).  Need 2T * f * 2 and T * d * 2 below 2^31.
hipError_t launch_up_tail_stream(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                                 const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, int n_cu, hipStream_t s);
// tail_part (may be null): buffer for split tails (layout above).
hipError_t launch_down_tail_stream(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T,
                                   int d, int f, int n_cu, float* tail_part, int64_t tail_part_bytes, hipStream_t s);

// Decode (few rows per expert).  T bounds the rows per expert of a top-2
// routing (any routing stays correct, more rows only take more passes).
hipError_t launch_up_decode(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                            const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, hipStream_t s);
// split == 2 (f a multiple of 256): two partial sums, the second at
// y_rows + split_stride; otherwise one full sum in y_rows.
hipError_t launch_down_decode(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T, int d,
                              int f, int split, int64_t split_stride, hipStream_t s);

// Decode batches of at most kStreamMaxTokens tokens: the weight streams of
// the touched experts through per-wave LDS rings, 2 * n_cu single-wave
// workgroups, token groups of 16 (up to 1, 2 or 4 per pass for T <= 32, 64,
// 128; an expert with more rows takes more passes).  Returns
// hipErrorInvalidValue above kStreamMaxTokens.
constexpr int64_t kStreamMaxTokens = 128;
hipError_t launch_up_decode_stream(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots,
                                   const bf16_t* w1, const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, int n_cu,
                                   hipStream_t s);
hipError_t launch_down_decode_stream(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T,
                                     int d, int f, int n_cu, hipStream_t s);

// Small batches (T <= 64): routing + permutation.  bf16: the router's
// d-slices on one workgroup each, then one workgroup adds them, routes and
// permutes; partials: route_partials_bytes(T) of device scratch.  fp32: one
// workgroup (partials unused).
constexpr int kRouteSlices = 16;           // d-slices of the bf16 small-batch router (at most)
constexpr int64_t kRouteSplitMaxTokens = 64;
inline size_t route_partials_bytes(int64_t T) {
  return static_cast<size_t>(kRouteSlices) * static_cast<size_t>((T + 15) / 16) * 64 * 16;
}
hipError_t launch_route_permute(int dtype, const void* x, const void* wg, const float* bias, int32_t* idx, float* w,
                                int32_t T, int d, int gating, int capacity, int32_t* offsets, int32_t* sorted_slots,
                                int32_t* slot_rows, int32_t* counts_out, float* partials, hipStream_t s);

// y_rows2 (optional): a second partial-sum buffer added to y_rows first.
hipError_t launch_combine(int dtype, const float* y_rows, const float* y_rows2, const int32_t* slot_rows,
                          const float* topk_w, void* y, int64_t T, int d, int n_cu, hipStream_t s);

// The bf16 MFMA ceiling probe: operands [64 x 64] bf16x8 (64 KiB), clk
// [4 * prefill_grid(n_cu)] int64, sink [prefill_grid(n_cu) * 256] fp32.
hipError_t launch_mfma_ceiling(const bf16_t* operands, long long* clk, float* sink, int iters, int n_cu,
                               hipStream_t s);

hipError_t launch_rmsnorm_residual(int dtype, float* resid, const void* y_add, void* u, int64_t T, int d, float eps,
                                   hipStream_t s);
// The same glue with the next layer's router fused in (idx [T, 2], w [T, 2]);
// d <= kMaxNormRouteD and W_g within the router's LDS limit.
constexpr int kMaxNormRouteD = 8192;
hipError_t launch_rmsnorm_route(int dtype, float* resid, const void* y_add, void* u, const void* wg,
                                const float* bias, int32_t* idx, float* w, int64_t T, int d, float eps, int gating,
                                int n_cu, hipStream_t s);
// The same glue with the layer's combine fused in: resid += the gate-weighted
// pair of y_rows rows (plus y_rows2, the second partial, if given) of each
// token, rounded to dtype exactly as launch_combine rounds y; then RMSNorm
// and (wg != nullptr) the next layer's routing.  y is never written.
hipError_t launch_combine_rmsnorm_route(int dtype, const float* y_rows, const float* y_rows2, const int32_t* slot_rows,
                                        const float* gates, float* resid, void* u, const void* wg, const float* bias,
                                        int32_t* idx, float* w, int64_t T, int d, float eps, int gating, int n_cu,
                                        hipStream_t s);

}  // namespace moe
