// Block-level expert-major permutation (device code shared by the permute
// kernel and the fused small-batch routing kernel).  See permute.hip for the
// method.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPermThreads = 1024;
static_assert(kPermThreads == kPermuteSmallSlots, "the ballot form holds one slot per thread");
constexpr int kPermWaves = kPermThreads / kWave;

// Ids outside [0, E) are skipped (never used as an index).
__device__ __forceinline__ int valid_expert(int e) { return (e >= 0 && e < kExperts) ? e : -1; }

// Rows an expert with `count` routed slots keeps under `capacity` (0: all).
__device__ __forceinline__ int kept_rows(int count, int capacity) {
  return (capacity > 0 && count > capacity) ? capacity : count;
}

// The whole permutation by one workgroup of kPermThreads threads.  idx is
// read from global memory (it may have been written by this workgroup before
// a __syncthreads()).  capacity > 0: each expert keeps its first `capacity`
// slots in slot order; the others get slot_rows = -1 and no row (offsets
// count kept rows; counts_out the routed slots).
__device__ inline void permute_block(const int32_t* __restrict__ idx, int32_t n_slots, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_rows,
                              int32_t* __restrict__ counts_out, int capacity) {
  __shared__ int32_t hist[kExperts];
  __shared__ int32_t base[kExperts];   // slots of the expert in earlier chunks (its rank so far)
  __shared__ int32_t off_s[kExperts];  // the expert's first row
  __shared__ int32_t wave_cnt[kPermWaves][kExperts];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  if (tid < kExperts) hist[tid] = 0;
  __syncthreads();

  // (1) histogram: per-wave ballots, one LDS add per wave and expert.
  for (int c = 0; c < n_slots; c += kPermThreads) {
    const int s = c + tid;
    const int e = s < n_slots ? valid_expert(idx[s]) : -1;
#pragma unroll
    for (int ee = 0; ee < kExperts; ++ee) {
      const unsigned long long m = __ballot(e == ee);
      if (lane == 0 && m) atomicAdd(&hist[ee], __popcll(m));
    }
  }
  __syncthreads();

  // (2) exclusive scan over the 8 experts.
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < kExperts; ++e) {
      offsets[e] = run;
      off_s[e] = run;
      base[e] = 0;
      if (counts_out) counts_out[e] = hist[e];
      run += kept_rows(hist[e], capacity);
    }
    offsets[kExperts] = run;
  }
  __syncthreads();

  // (3) stable scatter, chunk by chunk in slot order.
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c = 0; c < n_slots; c += kPermThreads) {
    const int s = c + tid;
    const int e = s < n_slots ? valid_expert(idx[s]) : -1;
    int rank = 0;
#pragma unroll
    for (int ee = 0; ee < kExperts; ++ee) {
      const unsigned long long m = __ballot(e == ee);
      if (e == ee) rank = __popcll(m & below);
      if (lane == 0) wave_cnt[wave][ee] = __popcll(m);
    }
    __syncthreads();
    if (e < 0 && s < n_slots) slot_rows[s] = -1;  // an id outside [0, E): no row, like a dropped slot
    if (e >= 0) {
      int r = base[e] + rank;  // the slot's rank among its expert's slots
      for (int w = 0; w < wave; ++w) r += wave_cnt[w][e];
      if (capacity > 0 && r >= capacity) {
        slot_rows[s] = -1;  // dropped
      } else {
        sorted_slots[off_s[e] + r] = s;
        slot_rows[s] = off_s[e] + r;
      }
    }
    __syncthreads();
    if (tid < kExperts) {
      int add = 0;
      for (int w = 0; w < kPermWaves; ++w) add += wave_cnt[w][tid];
      base[tid] += add;
    }
    __syncthreads();
  }
}

}  // namespace moe
