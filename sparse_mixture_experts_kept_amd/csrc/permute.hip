// Expert-major permutation of the token slots (a counting sort by expert).
//
// Grouping each expert's slots contiguously is what lets the expert GEMMs
// read an expert's tokens as one matrix; it realises the per-token routing of
// "Mixtral & Sparse MoE (2024) > The Solution" (routing paragraph) and
// changes no value.
//
// One workgroup of 1024 threads: (1) LDS histogram of the expert ids,
// (2) exclusive scan over the 8 counts -> offsets, (3) a stable scatter: the
// slots are taken in chunks of 1024 in slot order; inside a chunk, a slot's
// rank among earlier slots of the same expert is the popcount of a wave
// ballot below its lane plus the counts of earlier waves.  No atomics decide
// an order, so the result is deterministic.
#include "common.hpp"
#include "launch.hpp"
#include "permute_dev.hpp"

namespace moe {

__global__ void __launch_bounds__(kPermThreads) permute_kernel(const int32_t* __restrict__ idx, int32_t n_slots,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_slots,
                                                               int32_t* __restrict__ slot_rows,
                                                               int32_t* __restrict__ counts_out) {
  permute_block(idx, n_slots, offsets, sorted_slots, slot_rows, counts_out);
}

hipError_t launch_permute(const int32_t* idx, int32_t n_slots, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_rows, int32_t* counts_out, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, idx, n_slots, offsets, sorted_slots,
                     slot_rows, counts_out);
  return hipGetLastError();
}

}  // namespace moe
