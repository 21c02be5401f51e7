// extern "C" entry points of libmoe: host-side validation, workspace
// carve-up, kernel-family choice and launch sequencing on the caller's
// stream.  The declarations, with the passages of the pages each entry point
// realises, are in include/moe.h.
#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "launch.hpp"

namespace {

using moe::bf16_t;

// AUTO takes the streaming kernels up to here: measured on the full-size
// layer (d = 4096, f = 14336), they are 2-4% faster than the grouped GEMM up
// to T = 128 (T = 80-128: 495-511 us against 510-523 us); beyond, experts
// with more than 64 rows take further passes over their weights.
constexpr int64_t kDecodeMaxTokens = 128;
// Small batches: routing and permutation by launch_route_permute (bf16: a
// workgroup per d-slice of the router, then one that routes and permutes).
constexpr int64_t kRoutePermuteMaxTokens = 64;
static_assert(kRoutePermuteMaxTokens <= moe::kRouteSplitMaxTokens, "small-batch router");
constexpr size_t kRouterLdsLimit = 128 * 1024;
constexpr int kMaxDevices = 64;

int g_cu_count[kMaxDevices];
std::mutex g_cu_mutex;

// Compute units of the current device (cached per device).
moe_status cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return MOE_ERR_HIP;
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int dtype) { return dtype == moe::kDtypeBF16 ? 2 : 4; }

// Shape checks shared by every entry point that takes dims.
moe_status check_dims(const moe_dims* dims) {
  if (!dims) return MOE_ERR_INVALID_ARGUMENT;
  if (dims->T < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (dims->E != 8 || dims->k != 2) return MOE_ERR_UNSUPPORTED;
  if (dims->d <= 0 || dims->f <= 0 || dims->d % 128 != 0 || dims->f % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (dims->dtype != MOE_F32 && dims->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (dims->variant < MOE_VARIANT_AUTO || dims->variant > MOE_VARIANT_PREFILL) return MOE_ERR_UNSUPPORTED;
  if (dims->gating != MOE_GATING_PAIR && dims->gating != MOE_GATING_FULL) return MOE_ERR_UNSUPPORTED;
  if (dims->capacity < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (dims->T > (int64_t{1} << 30) / dims->k) return MOE_ERR_UNSUPPORTED;  // slot ids are int32
  // Largest row offset of h / y_rows must fit comfortably in int64 (always true) and
  // element offsets r*f, r*d are formed in int64 on the device.
  return MOE_OK;
}

// The prefill kernels pipeline the reduction in 64-wide stages (d, f >= 256)
// and address gathered token rows with 32-bit offsets (x below 4 GiB); other
// layers use the decode kernels.
bool use_decode(const moe_dims* dims) {
  if (!moe::prefill_fits(dims->T, dims->d, dims->f)) return true;
  if (dims->variant == MOE_VARIANT_DECODE) return true;
  if (dims->variant == MOE_VARIANT_PREFILL) return false;
  return dims->T <= kDecodeMaxTokens;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Stage boundaries of the layer (moe_ffn_forward_timed): an event is
// recorded on the layer's stream after each stage (the up GEMM's own, event
// 3, right after the GEMM launch), and the up GEMM may run as its
// clock-recording twin.  Null marks record nothing.
constexpr int kStageEvents = 8;
struct StageMarks {
  void* const* ev = nullptr;  // kStageEvents hipEvent_t
  long long* clk = nullptr;   // 4 int64 per workgroup of the up GEMM
};
moe_status mark(const StageMarks* m, int i, hipStream_t s) {
  if (!m || !m->ev) return MOE_OK;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(m->ev[i]), s));
}
long long* up_clock(const StageMarks* m) { return m ? m->clk : nullptr; }

// Prefill projections hand the short expert tails (the rows past an expert's
// last full 256-row tile, when at most 32) to the streaming kernels, which
// spread each tail's weight stream over the whole chip; inside the prefill
// GEMM such a tile is bound by one CU's load latency (a down-projection tail
// tile costs 0.58 of a full tile there).  The streaming kernels address x and
// h with 31-bit byte offsets.
constexpr bool kUpTailsStreamed = true;
bool tails_streamable(const moe_dims* dims) {
  const int64_t limit = int64_t{1} << 31;
  return dims->T * dims->k * dims->f * 2 < limit && dims->T * dims->d * 2 < limit;
}

// partials (may be null): a scratch buffer of partial_bytes for the GEMMs'
// remainder split (the work units past the last whole round of the grid are
// cut along the reduction and their partial tiles summed by a fixup launch).
moe_status up_prefill(const moe_dims* dims, const bf16_t* x, const int32_t* offs, const int32_t* sorted,
                      const bf16_t* w1, const bf16_t* w3, bf16_t* h, int n_cu, float* partials,
                      int64_t partial_bytes, hipStream_t s, const StageMarks* marks = nullptr) {
  const bool tails = kUpTailsStreamed && tails_streamable(dims);
  moe_status st = hip_status(moe::launch_up_prefill(x, offs, sorted, w1, w3, h, dims->d, dims->f, n_cu, tails,
                                                    partials, partial_bytes, s, up_clock(marks),
                                                    marks && marks->ev ? static_cast<hipEvent_t>(marks->ev[3])
                                                                       : nullptr));
  if (st != MOE_OK || !tails) return st;
  return hip_status(moe::launch_up_tail_stream(x, offs, sorted, w1, w3, h, dims->T, dims->d, dims->f, n_cu, s));
}

// split == 2 keeps the tails in the GEMM (their second partial sum must exist).
// With partials (split == 1 only): the first n_cu planes of 256 x 256 fp32
// serve the GEMM's remainder split, the rest the split tails; one fixup
// launch after the tails completes both.
moe_status down_prefill(const moe_dims* dims, const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows,
                        int n_cu, int split, int64_t split_stride, float* partials, int64_t partial_bytes,
                        hipStream_t s, const StageMarks* marks = nullptr) {
  const bool tails = split == 1 && tails_streamable(dims);
  const int64_t plane_bytes = std::min<int64_t>(partial_bytes, int64_t{n_cu} * 256 * 256 * 4);
  float* tail_part = partials && partial_bytes > plane_bytes ? partials + plane_bytes / 4 : nullptr;
  const int64_t tail_bytes = tail_part ? partial_bytes - plane_bytes : 0;
  moe_status st = hip_status(moe::launch_down_prefill(h, offs, w2, y_rows, dims->d, dims->f, n_cu, split,
                                                      split_stride, tails, partials, plane_bytes, s));
  if (st == MOE_OK) st = mark(marks, 5, s);
  if (st != MOE_OK) return st;
  if (tails) {
    st = hip_status(moe::launch_down_tail_stream(h, offs, w2, y_rows, dims->T, dims->d, dims->f, n_cu, tail_part,
                                                 tail_bytes, s));
    if (st != MOE_OK) return st;
  }
  if (!partials || split != 1) return MOE_OK;
  const bool split_tails = tails && moe::tail_part_capacity(tail_part, tail_bytes, dims->d) >= 2;
  return hip_status(moe::launch_down_prefill_fixup(offs, partials, plane_bytes, split_tails ? tail_part : nullptr,
                                                   y_rows, dims->d, dims->f, n_cu, tails, s));
}

size_t align256(size_t v) { return (v + 255) & ~size_t{255}; }

struct Workspace {
  size_t idx, w, offsets, sorted, rows, gcounts, rpart, h, y_rows, y_rows2, total;
};

Workspace plan_workspace(const moe_dims* dims) {
  const size_t slots = static_cast<size_t>(dims->T) * dims->k;
  Workspace ws;
  size_t o = 0;
  ws.idx = o; o += align256(slots * 4);
  ws.w = o; o += align256(slots * 4);
  ws.offsets = o; o += align256((dims->E + 1) * 4);
  ws.sorted = o; o += align256(slots * 4);
  ws.rows = o; o += align256(slots * 4);
  ws.gcounts = o; o += align256(static_cast<size_t>((dims->T + 15) / 16) * dims->E * 4);  // router group counts
  // partial scores of the bf16 small-batch router (one workgroup per d-slice)
  ws.rpart = o;
  if (dims->dtype == MOE_BF16 && dims->T <= kRoutePermuteMaxTokens) o += align256(moe::route_partials_bytes(dims->T));
  ws.h = o; o += align256(slots * dims->f * elem_size(dims->dtype));
  ws.y_rows = o; o += align256(slots * dims->d * 4);
  // Second partial of the split down projection (and the prefill GEMMs'
  // partial tiles): only the bf16 prefill kernels use it.
  ws.y_rows2 = o;
  if (dims->dtype == MOE_BF16 && !use_decode(dims)) o += align256(slots * dims->d * 4);
  ws.total = o;
  return ws;
}

moe_status run_router(const moe_dims* dims, const void* x, const void* w_gate, const float* bias, int32_t* idx,
                      float* w, float* logits, hipStream_t s, int32_t* group_counts = nullptr) {
  int n_cu = 0;
  moe_status st = cu_count(&n_cu);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_router(dims->dtype, x, w_gate, bias, idx, w, logits, dims->T, dims->d, dims->gating,
                                      n_cu, s, group_counts));
}

// The permutation's form for T tokens: per-group counts then one wave per
// 16-token group when the slots exceed one workgroup's ballot form and the
// group counts fit; otherwise one workgroup.
bool permute_by_groups(const moe_dims* dims) {
  return dims->T * dims->k > moe::kPermuteSmallSlots && dims->T <= moe::kMaxGroupPermuteTokens;
}

// Permutation of the pairs in idx; group_counts [ceil(T/16), 8] int32 is
// scratch for the multi-workgroup form.
moe_status permute_slots(const moe_dims* dims, const int32_t* idx, int32_t* group_counts, int32_t* offs,
                         int32_t* sorted, int32_t* rows, int32_t* counts_out, hipStream_t s) {
  if (permute_by_groups(dims))
    return hip_status(moe::launch_permute_counted(idx, static_cast<int32_t>(dims->T), group_counts, offs, sorted,
                                                  rows, counts_out, dims->capacity, s));
  return hip_status(moe::launch_permute(idx, static_cast<int32_t>(dims->T * dims->k), offs, sorted, rows,
                                        counts_out, dims->capacity, s));
}

moe_status run_up(const moe_dims* dims, const void* x, const int32_t* offs, const int32_t* sorted, const void* w1,
                  const void* w3, void* h, hipStream_t s) {
  if (dims->dtype == MOE_F32)
    return hip_status(moe::launch_up_f32(static_cast<const float*>(x), offs, sorted, static_cast<const float*>(w1),
                                         static_cast<const float*>(w3), static_cast<float*>(h), dims->T * dims->k,
                                         dims->d, dims->f, s));
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* w1b = static_cast<const bf16_t*>(w1);
  const bf16_t* w3b = static_cast<const bf16_t*>(w3);
  bf16_t* hb = static_cast<bf16_t*>(h);
  int n_cu = 0;
  const moe_status st = cu_count(&n_cu);
  if (st != MOE_OK) return st;
  if (use_decode(dims)) {
    if (dims->T <= moe::kStreamMaxTokens)
      return hip_status(moe::launch_up_decode_stream(xb, offs, sorted, w1b, w3b, hb, dims->T, dims->d, dims->f, n_cu, s));
    return hip_status(moe::launch_up_decode(xb, offs, sorted, w1b, w3b, hb, dims->T, dims->d, dims->f, s));
  }
  return up_prefill(dims, xb, offs, sorted, w1b, w3b, hb, n_cu, nullptr, 0, s);
}

moe_status run_down(const moe_dims* dims, const void* h, const int32_t* offs, const void* w2, float* y_rows,
                    hipStream_t s) {
  if (dims->dtype == MOE_F32)
    return hip_status(moe::launch_down_f32(static_cast<const float*>(h), offs, static_cast<const float*>(w2), y_rows,
                                           dims->T * dims->k, dims->d, dims->f, s));
  const bf16_t* hb = static_cast<const bf16_t*>(h);
  const bf16_t* w2b = static_cast<const bf16_t*>(w2);
  int n_cu = 0;
  const moe_status st = cu_count(&n_cu);
  if (st != MOE_OK) return st;
  if (use_decode(dims)) {
    if (dims->T <= moe::kStreamMaxTokens)
      return hip_status(moe::launch_down_decode_stream(hb, offs, w2b, y_rows, dims->T, dims->d, dims->f, n_cu, s));
    return hip_status(moe::launch_down_decode(hb, offs, w2b, y_rows, dims->T, dims->d, dims->f, 1, 0, s));
  }
  return down_prefill(dims, hb, offs, w2b, y_rows, n_cu, 1, 0, nullptr, 0, s);
}

moe_status run_experts(const moe_dims* dims, const void* x, const int32_t* offs, const int32_t* sorted,
                       const void* w1, const void* w3, const void* w2, void* h, float* y_rows, hipStream_t s,
                       const StageMarks* marks = nullptr) {
  // (the decode and fp32 paths have no separate tail stage: marks 3/4 and 5/6 coincide)
  moe_status st = run_up(dims, x, offs, sorted, w1, w3, h, s);
  if (st == MOE_OK) st = mark(marks, 3, s);
  if (st == MOE_OK) st = mark(marks, 4, s);
  if (st != MOE_OK) return st;
  st = run_down(dims, h, offs, w2, y_rows, s);
  if (st == MOE_OK) st = mark(marks, 5, s);
  if (st == MOE_OK) st = mark(marks, 6, s);
  return st;
}

moe_status run_combine(const moe_dims* dims, const float* y_rows, const int32_t* slot_rows, const float* w, void* y,
                       hipStream_t s) {
  int n_cu = 0;
  moe_status st = cu_count(&n_cu);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_combine(dims->dtype, y_rows, nullptr, slot_rows, w, y, dims->T, dims->d, n_cu, s));
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_UNKNOWN_STATUS";
}

const char* moe_version(void) { return "1.0.0"; }

moe_status moe_router_topk(const moe_dims* dims, const void* x, const void* w_gate, const float* logit_bias,
                           int32_t* topk_idx, float* topk_w, float* logits, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (static_cast<size_t>(dims->E) * dims->d * elem_size(dims->dtype) > kRouterLdsLimit) return MOE_ERR_UNSUPPORTED;
  if (dims->T == 0) return MOE_OK;
  if (!x || !w_gate || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(topk_idx, 8) || !aligned(topk_w, 8) ||
      (logits && !aligned(logits, 16)) || (logit_bias && !aligned(logit_bias, 16)))
    return MOE_ERR_INVALID_ARGUMENT;
  return run_router(dims, x, w_gate, logit_bias, topk_idx, topk_w, logits, static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_slots,
                       int32_t* slot_rows, void* workspace, size_t* workspace_bytes, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!workspace_bytes) return MOE_ERR_INVALID_ARGUMENT;
  // Group counts [ceil(T/16), 8] for the multi-workgroup form (a token
  // count the one-workgroup forms handle still asks for a minimal workspace).
  const bool groups = permute_by_groups(dims);
  const size_t need = groups ? align256(static_cast<size_t>((dims->T + 15) / 16) * dims->E * 4) : 256;
  if (!workspace) {
    *workspace_bytes = need;
    return MOE_OK;
  }
  if (dims->T == 0) return MOE_OK;
  if (*workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!expert_offsets || !topk_idx || !sorted_slots || !slot_rows) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(topk_idx, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_slots, 4) || !aligned(slot_rows, 4) ||
      !aligned(workspace, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  return permute_slots(dims, topk_idx, static_cast<int32_t*>(workspace), expert_offsets, sorted_slots, slot_rows,
                       nullptr, static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_swiglu(const moe_dims* dims, const void* x, const int32_t* expert_offsets,
                              const int32_t* sorted_slots, const void* w1, const void* w3, const void* w2, void* h,
                              float* y_rows, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (!x || !expert_offsets || !sorted_slots || !w1 || !w3 || !w2 || !h || !y_rows) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w3, 16) || !aligned(w2, 16) || !aligned(h, 16) ||
      !aligned(y_rows, 16) || !aligned(expert_offsets, 4) || !aligned(sorted_slots, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return run_experts(dims, x, expert_offsets, sorted_slots, w1, w3, w2, h, y_rows, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_up(const moe_dims* dims, const void* x, const int32_t* expert_offsets,
                         const int32_t* sorted_slots, const void* w1, const void* w3, void* h, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (!x || !expert_offsets || !sorted_slots || !w1 || !w3 || !h) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w3, 16) || !aligned(h, 16) || !aligned(expert_offsets, 4) ||
      !aligned(sorted_slots, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return run_up(dims, x, expert_offsets, sorted_slots, w1, w3, h, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_down(const moe_dims* dims, const void* h, const int32_t* expert_offsets, const void* w2,
                           float* y_rows, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (!h || !expert_offsets || !w2 || !y_rows) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(h, 16) || !aligned(w2, 16) || !aligned(y_rows, 16) || !aligned(expert_offsets, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return run_down(dims, h, expert_offsets, w2, y_rows, static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_dims* dims, const float* y_rows, const int32_t* slot_rows, const float* topk_w,
                       void* y, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (!y_rows || !slot_rows || !topk_w || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(y_rows, 16) || !aligned(y, 16) || !aligned(slot_rows, 8) || !aligned(topk_w, 8))
    return MOE_ERR_INVALID_ARGUMENT;
  return run_combine(dims, y_rows, slot_rows, topk_w, y, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Allocation-free form of moe_ffn_forward: its workspace is this file-scope
// device array (one copy per GPU, held until the process ends).  In host
// code `scratch` only names the symbol; its device address on the current
// GPU comes from hipGetSymbolAddress, looked up once per device on the
// first call there and kept in g_scratch.  The layer's kernels need nothing
// in it zeroed: every region is written before it is read within a call.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

moe_status scratch_on_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

// The glue that takes the place of the combine in
// moe_ffn_forward_routed_residual (null: the combine writes y).
struct ResidualGlue {
  float* resid;
  void* u;
  float eps;
  const void* wg;
  const float* bias;
  int32_t* idx;
  float* w;
};

moe_status combine_or_glue(const moe_dims* dims, const float* y_rows, const float* y_rows2, const int32_t* rows,
                           const float* gate, void* y, const ResidualGlue* glue, int n_cu, hipStream_t s) {
  if (!glue)
    return hip_status(moe::launch_combine(dims->dtype, y_rows, y_rows2, rows, gate, y, dims->T, dims->d, n_cu, s));
  return hip_status(moe::launch_combine_rmsnorm_route(dims->dtype, y_rows, y_rows2, rows, gate, glue->resid, glue->u,
                                                      glue->wg, glue->bias, glue->idx, glue->w, dims->T, dims->d,
                                                      glue->eps, dims->gating, n_cu, s));
}

// The whole layer.  routed_idx / routed_w given: the routing was computed by
// the caller (e.g. by moe_rmsnorm_residual_route) and the router is skipped.
moe_status ffn_forward_impl(const moe_dims* dims, const void* x, const void* w_gate, const float* logit_bias,
                            const int32_t* routed_idx, const float* routed_w, const void* w1, const void* w3,
                            const void* w2, void* y, int32_t* topk_idx_out, float* topk_w_out,
                            int32_t* expert_counts_out, void* workspace, size_t* workspace_bytes, void* stream,
                            bool use_scratch = false, const StageMarks* marks = nullptr,
                            const ResidualGlue* glue = nullptr) {
  const bool routed = routed_idx != nullptr;
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!workspace_bytes) return MOE_ERR_INVALID_ARGUMENT;
  if (!routed && static_cast<size_t>(dims->E) * dims->d * elem_size(dims->dtype) > kRouterLdsLimit)
    return MOE_ERR_UNSUPPORTED;
  const Workspace plan = plan_workspace(dims);
  // The allocation-free form's workspace is the device array `scratch`,
  // looked up below once the arguments have been checked.
  if (use_scratch && plan.total > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!use_scratch && !workspace) {
    *workspace_bytes = plan.total;
    return MOE_OK;
  }
  if (dims->T == 0) return MOE_OK;
  if (!use_scratch && *workspace_bytes < plan.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!x || (!routed && !w_gate) || (routed && !routed_w) || !w1 || !w3 || !w2 || (!glue && !y))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((!use_scratch && !aligned(workspace, 256)) || !aligned(x, 16) || (w_gate && !aligned(w_gate, 16)) ||
      !aligned(w1, 16) || !aligned(w3, 16) || !aligned(w2, 16) || (y && !aligned(y, 16)) ||
      (logit_bias && !aligned(logit_bias, 16)) ||
      (topk_idx_out && !aligned(topk_idx_out, 8)) || (topk_w_out && !aligned(topk_w_out, 8)) ||
      (routed_idx && !aligned(routed_idx, 8)) || (routed_w && !aligned(routed_w, 8)) ||
      (expert_counts_out && !aligned(expert_counts_out, 4)))
    return MOE_ERR_INVALID_ARGUMENT;

  if (use_scratch) {
    st = scratch_on_device(&workspace);
    if (st != MOE_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(ws + plan.idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + plan.w);
  const int32_t* pair = routed ? routed_idx : idx;
  const float* gate = routed ? routed_w : w;
  int32_t* offs = reinterpret_cast<int32_t*>(ws + plan.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + plan.sorted);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + plan.rows);
  void* h = ws + plan.h;
  float* y_rows = reinterpret_cast<float*>(ws + plan.y_rows);

  st = mark(marks, 0, s);
  if (st != MOE_OK) return st;
  int32_t* gcounts = reinterpret_cast<int32_t*>(ws + plan.gcounts);
  if (routed) {
    st = mark(marks, 1, s);
    if (st != MOE_OK) return st;
    st = permute_slots(dims, pair, gcounts, offs, sorted, rows, expert_counts_out, s);
    if (st != MOE_OK) return st;
  } else if (dims->T <= kRoutePermuteMaxTokens) {
    // Small batch: routing and permutation without the router's group counts.
    st = hip_status(moe::launch_route_permute(dims->dtype, x, w_gate, logit_bias, idx, w,
                                              static_cast<int32_t>(dims->T), dims->d, dims->gating,
                                              dims->capacity, offs, sorted, rows, expert_counts_out,
                                              reinterpret_cast<float*>(ws + plan.rpart), s));
    if (st != MOE_OK) return st;
    // (bf16 decode then runs the streaming up and down projections through
    // run_experts below.)
  } else if (dims->dtype == MOE_BF16 && dims->T <= moe::kMaxGroupPermuteTokens) {
    // The router counts each 16-token group's slots per expert; the
    // permutation then runs one wave per group.
    st = run_router(dims, x, w_gate, logit_bias, idx, w, nullptr, s, gcounts);
    if (st == MOE_OK) st = mark(marks, 1, s);
    if (st != MOE_OK) return st;
    st = hip_status(moe::launch_permute_groups(idx, static_cast<int32_t>(dims->T), gcounts, offs, sorted, rows,
                                               expert_counts_out, dims->capacity, s));
    if (st != MOE_OK) return st;
  } else {
    st = run_router(dims, x, w_gate, logit_bias, idx, w, nullptr, s);
    if (st == MOE_OK) st = mark(marks, 1, s);
    if (st != MOE_OK) return st;
    st = permute_slots(dims, idx, gcounts, offs, sorted, rows, expert_counts_out, s);
    if (st != MOE_OK) return st;
  }
  // (routing and permutation in one launch: the routing stage holds both)
  if (!routed && dims->T <= kRoutePermuteMaxTokens) st = mark(marks, 1, s);
  if (st == MOE_OK) st = mark(marks, 2, s);
  if (st != MOE_OK) return st;
  if (dims->dtype == MOE_BF16 && !use_decode(dims)) {
    // Prefill.  The down projection's reduction is split in two when the
    // layer has fewer full 256 x 256 tiles than CUs (twice the work units to
    // spread); the combine then adds the two partial sums in a fixed order.
    // From one full round on, the unsplit GEMM hands its short tails to the
    // streaming kernel instead of running them as thin tiles on a few XCDs.
    int n_cu = 0;
    st = cu_count(&n_cu);
    if (st != MOE_OK) return st;
    // The second partial's region is idle until the split down projection
    // writes it: the remainder splits use it as their partial buffer.
    float* second = reinterpret_cast<float*>(ws + plan.y_rows2);
    const int64_t second_bytes = static_cast<int64_t>(plan.total - plan.y_rows2);
    st = up_prefill(dims, static_cast<const bf16_t*>(x), offs, sorted, static_cast<const bf16_t*>(w1),
                    static_cast<const bf16_t*>(w3), static_cast<bf16_t*>(h), n_cu, second, second_bytes, s, marks);
    if (st == MOE_OK) st = mark(marks, 4, s);
    if (st != MOE_OK) return st;
    const int64_t full_units = (dims->T * dims->k / 256) * (dims->d / 256);
    const int split = full_units >= n_cu ? 1 : 2;
    float* y_rows2 = split == 2 ? second : nullptr;
    st = down_prefill(dims, static_cast<const bf16_t*>(h), offs, static_cast<const bf16_t*>(w2), y_rows, n_cu, split,
                      split == 2 ? y_rows2 - y_rows : 0, split == 2 ? nullptr : second, second_bytes, s, marks);
    if (st == MOE_OK) st = mark(marks, 6, s);
    if (st != MOE_OK) return st;
    st = combine_or_glue(dims, y_rows, y_rows2, rows, gate, y, glue, n_cu, s);
    return st == MOE_OK ? mark(marks, 7, s) : st;
  }
  st = run_experts(dims, x, offs, sorted, w1, w3, w2, h, y_rows, s, marks);
  if (st != MOE_OK) return st;
  int n_cu = 0;
  st = cu_count(&n_cu);
  if (st == MOE_OK) st = combine_or_glue(dims, y_rows, nullptr, rows, gate, y, glue, n_cu, s);
  return st == MOE_OK ? mark(marks, 7, s) : st;
}

}  // namespace

extern "C" {

moe_status moe_ffn_forward(const moe_dims* dims, const void* x, const void* w_gate, const float* logit_bias,
                           const void* w1, const void* w3, const void* w2, void* y, int32_t* topk_idx_out,
                           float* topk_w_out, int32_t* expert_counts_out, void* workspace, size_t* workspace_bytes,
                           void* stream) {
  return ffn_forward_impl(dims, x, w_gate, logit_bias, nullptr, nullptr, w1, w3, w2, y, topk_idx_out, topk_w_out,
                          expert_counts_out, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_forward_noalloc(const moe_dims* dims, const void* x, const void* w_gate, const float* logit_bias,
                                   const void* w1, const void* w3, const void* w2, void* y, int32_t* topk_idx_out,
                                   float* topk_w_out, int32_t* expert_counts_out, void* stream) {
  size_t bytes = kNoAllocScratchBytes;
  return ffn_forward_impl(dims, x, w_gate, logit_bias, nullptr, nullptr, w1, w3, w2, y, topk_idx_out, topk_w_out,
                          expert_counts_out, nullptr, &bytes, stream, /*use_scratch=*/true);
}

moe_status moe_ffn_forward_timed(const moe_dims* dims, const void* x, const void* w_gate, const float* logit_bias,
                                 const void* w1, const void* w3, const void* w2, void* y, int32_t* topk_idx_out,
                                 float* topk_w_out, int32_t* expert_counts_out, void* workspace,
                                 size_t* workspace_bytes, void* stream, void* const* stage_events,
                                 int64_t* up_gemm_clock) {
  if (!stage_events) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < kStageEvents; ++i)
    if (!stage_events[i]) return MOE_ERR_INVALID_ARGUMENT;
  if (up_gemm_clock && !aligned(up_gemm_clock, 8)) return MOE_ERR_INVALID_ARGUMENT;
  StageMarks marks;
  marks.ev = stage_events;
  marks.clk = reinterpret_cast<long long*>(up_gemm_clock);
  return ffn_forward_impl(dims, x, w_gate, logit_bias, nullptr, nullptr, w1, w3, w2, y, topk_idx_out, topk_w_out,
                          expert_counts_out, workspace, workspace_bytes, stream, false, &marks);
}

moe_status moe_ffn_forward_routed(const moe_dims* dims, const void* x, const int32_t* topk_idx, const float* topk_w,
                                  const void* w1, const void* w3, const void* w2, void* y,
                                  int32_t* expert_counts_out, void* workspace, size_t* workspace_bytes,
                                  void* stream) {
  // (a NULL topk_idx leaves no router and no routing: INVALID_ARGUMENT, except for the size query)
  return ffn_forward_impl(dims, x, nullptr, nullptr, topk_idx, topk_w, w1, w3, w2, y, nullptr, nullptr,
                          expert_counts_out, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_forward_routed_residual(const moe_dims* dims, const void* x, const int32_t* topk_idx,
                                           const float* topk_w, const void* w1, const void* w3, const void* w2,
                                           float* resid, void* u_out, float eps, const void* w_gate_next,
                                           const float* logit_bias_next, int32_t* topk_idx_next,
                                           float* topk_w_next, int32_t* expert_counts_out, void* workspace,
                                           size_t* workspace_bytes, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->d > moe::kMaxNormRouteD) return MOE_ERR_UNSUPPORTED;
  if (w_gate_next && static_cast<size_t>(dims->E) * dims->d * elem_size(dims->dtype) > kRouterLdsLimit)
    return MOE_ERR_UNSUPPORTED;
  if (workspace && dims->T > 0) {
    if (!resid || !u_out || (w_gate_next && (!topk_idx_next || !topk_w_next))) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(resid, 16) || !aligned(u_out, 16) || (w_gate_next && !aligned(w_gate_next, 16)) ||
        (logit_bias_next && !aligned(logit_bias_next, 16)) || (topk_idx_next && !aligned(topk_idx_next, 8)) ||
        (topk_w_next && !aligned(topk_w_next, 8)))
      return MOE_ERR_INVALID_ARGUMENT;
  }
  const ResidualGlue glue{resid, u_out, eps, w_gate_next, logit_bias_next, topk_idx_next, topk_w_next};
  return ffn_forward_impl(dims, x, nullptr, nullptr, topk_idx, topk_w, w1, w3, w2, nullptr, nullptr, nullptr,
                          expert_counts_out, workspace, workspace_bytes, stream, false, nullptr, &glue);
}

moe_status moe_rmsnorm_residual_route(const moe_dims* dims, float* resid, const void* y_add, void* u_out, float eps,
                                      const void* w_gate, const float* logit_bias, int32_t* topk_idx, float* topk_w,
                                      void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->d > moe::kMaxNormRouteD) return MOE_ERR_UNSUPPORTED;
  if (static_cast<size_t>(dims->E) * dims->d * elem_size(dims->dtype) > kRouterLdsLimit) return MOE_ERR_UNSUPPORTED;
  if (dims->T == 0) return MOE_OK;
  if (!resid || !u_out || !w_gate || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(resid, 16) || !aligned(u_out, 16) || (y_add && !aligned(y_add, 16)) || !aligned(w_gate, 16) ||
      (logit_bias && !aligned(logit_bias, 16)) || !aligned(topk_idx, 8) || !aligned(topk_w, 8))
    return MOE_ERR_INVALID_ARGUMENT;
  int n_cu = 0;
  st = cu_count(&n_cu);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_rmsnorm_route(dims->dtype, resid, y_add, u_out, w_gate, logit_bias, topk_idx, topk_w,
                                              dims->T, dims->d, eps, dims->gating, n_cu,
                                              static_cast<hipStream_t>(stream)));
}

moe_status moe_mfma_ceiling(const void* operands, int64_t* clock_out, float* sink, int32_t iters, void* stream) {
  if (!operands || !clock_out || !sink || iters < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(operands, 16) || !aligned(clock_out, 8) || !aligned(sink, 4)) return MOE_ERR_INVALID_ARGUMENT;
  int n_cu = 0;
  const moe_status st = cu_count(&n_cu);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_mfma_ceiling(static_cast<const bf16_t*>(operands),
                                             reinterpret_cast<long long*>(clock_out), sink, iters, n_cu,
                                             static_cast<hipStream_t>(stream)));
}

moe_status moe_load_balance_loss(const moe_dims* dims, const float* logits, const int32_t* topk_idx, float* loss,
                                 void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (!logits || !topk_idx || !loss) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(loss, 4)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_load_balance_loss(logits, topk_idx, dims->T, loss, static_cast<hipStream_t>(stream)));
}

moe_status moe_rmsnorm_residual(int64_t T, int32_t d, float* resid, const void* y_add, void* u_out, float eps,
                                int32_t dtype, void* stream) {
  if (T < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (d <= 0 || d % 128 != 0 || d > 16384) return MOE_ERR_UNSUPPORTED;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!resid || !u_out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(resid, 16) || !aligned(u_out, 16) || (y_add && !aligned(y_add, 16))) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(
      moe::launch_rmsnorm_residual(dtype, resid, y_add, u_out, T, d, eps, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
