// Expert-major permutation of the token slots (a counting sort by expert).
//
// Grouping each expert's slots contiguously is what lets the expert GEMMs
// read an expert's tokens as one matrix; it realises the per-token routing of
// "Mixtral & Sparse MoE (2024) > The Solution" (routing paragraph) and
// changes no value.
//
// Up to 1024 slots: one slot per thread, wave ballots (permute_dev.hpp).
// Up to 65536 tokens (moe_permute, or the layer from the router's counts):
// per-group counts, then one wave per 16-token group places its 32 slots
// (permute_groups_kernel).  Beyond, or without a group-count buffer: one
// workgroup of 1024 threads; thread i owns 8 consecutive slots of each
// chunk of 8192.  Pass 1: per-thread counts per expert, summed over the
// workgroup -> offsets (exclusive scan over the 8 experts).  Pass 2, chunk by
// chunk in slot order: per-thread counts packed two experts per 32-bit word
// (16 bits each; at most 8192 per chunk), an exclusive scan over the lanes
// of each wave (shuffles) and over the 16 waves (LDS) gives every thread the
// number of earlier slots of each expert, and the thread places its 8 slots
// in order.  Stable (slot order within an expert) and free of atomics, so the
// result is deterministic.  With an expert capacity C > 0 a slot whose rank
// among its expert's slots is C or more is dropped: it gets no row and
// slot_rows = -1 (reading of the load-balancing paragraph of "Mixtral &
// Sparse MoE (2024) > The Solution": a capacity limits the tokens per expert).
#include "common.hpp"
#include "launch.hpp"
#include "permute_dev.hpp"

namespace moe {
namespace {

constexpr int kSlotsPerThread = 8;
constexpr int kChunk = kPermThreads * kSlotsPerThread;  // 8192 slots

// The 8 expert ids of this thread's slots s0..s0+7 (-1 past the end or invalid).
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ idx, int32_t n_slots, int s0, int* ids) {
  if (s0 + kSlotsPerThread <= n_slots) {
    const int4 a = *reinterpret_cast<const int4*>(idx + s0);
    const int4 b = *reinterpret_cast<const int4*>(idx + s0 + 4);
    ids[0] = a.x; ids[1] = a.y; ids[2] = a.z; ids[3] = a.w;
    ids[4] = b.x; ids[5] = b.y; ids[6] = b.z; ids[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) ids[i] = s0 + i < n_slots ? idx[s0 + i] : -1;
  }
#pragma unroll
  for (int i = 0; i < kSlotsPerThread; ++i) ids[i] = valid_expert(ids[i]);
}

__global__ void __launch_bounds__(kPermThreads) permute_kernel(const int32_t* __restrict__ idx, int32_t n_slots,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_slots,
                                                               int32_t* __restrict__ slot_rows,
                                                               int32_t* __restrict__ counts_out, int capacity) {
  __shared__ int32_t wave_sum[kPermWaves][kExperts];
  __shared__ uint32_t wave_pk[kPermWaves][kExperts / 2];
  __shared__ int32_t base_s[kExperts];  // the expert's slots in earlier chunks (its rank so far)
  __shared__ int32_t off_s[kExperts];   // the expert's first row
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  // Pass 1: counts per expert.
  int cnt[kExperts];
#pragma unroll
  for (int e = 0; e < kExperts; ++e) cnt[e] = 0;
  for (int c = 0; c < n_slots; c += kChunk) {
    int ids[kSlotsPerThread];
    load_ids(idx, n_slots, c + tid * kSlotsPerThread, ids);
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i)
#pragma unroll
      for (int e = 0; e < kExperts; ++e) cnt[e] += ids[i] == e ? 1 : 0;
  }
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    int v = cnt[e];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    if (lane == 0) wave_sum[wave][e] = v;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < kExperts; ++e) {
      int tot = 0;
      for (int w = 0; w < kPermWaves; ++w) tot += wave_sum[w][e];
      offsets[e] = run;
      off_s[e] = run;
      base_s[e] = 0;
      if (counts_out) counts_out[e] = tot;
      run += kept_rows(tot, capacity);
    }
    offsets[kExperts] = run;
  }
  __syncthreads();

  // Pass 2: stable scatter, chunk by chunk.
  for (int c = 0; c < n_slots; c += kChunk) {
    const int s0 = c + tid * kSlotsPerThread;
    int ids[kSlotsPerThread];
    load_ids(idx, n_slots, s0, ids);
    // packed counts: word k holds experts 2k (low half) and 2k+1 (high half)
    uint32_t pk[kExperts / 2];
#pragma unroll
    for (int k = 0; k < kExperts / 2; ++k) pk[k] = 0;
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i)
#pragma unroll
      for (int k = 0; k < kExperts / 2; ++k)
        pk[k] += (ids[i] == 2 * k ? 1u : 0u) + (ids[i] == 2 * k + 1 ? 0x10000u : 0u);
    // inclusive scan over the lanes of the wave
    uint32_t inc[kExperts / 2];
#pragma unroll
    for (int k = 0; k < kExperts / 2; ++k) {
      uint32_t v = pk[k];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
      }
      inc[k] = v;
    }
    if (lane == kWave - 1) {
#pragma unroll
      for (int k = 0; k < kExperts / 2; ++k) wave_pk[wave][k] = inc[k];
    }
    __syncthreads();
    // earlier waves' counts, and this chunk's totals
    uint32_t before[kExperts / 2], total[kExperts / 2];
#pragma unroll
    for (int k = 0; k < kExperts / 2; ++k) {
      before[k] = 0;
      total[k] = 0;
    }
    for (int w = 0; w < kPermWaves; ++w) {
#pragma unroll
      for (int k = 0; k < kExperts / 2; ++k) {
        const uint32_t v = wave_pk[w][k];
        if (w < wave) before[k] += v;
        total[k] += v;
      }
    }
    int next[kExperts];  // rank of this thread's next slot of each expert
#pragma unroll
    for (int k = 0; k < kExperts / 2; ++k) {
      const uint32_t ex = before[k] + inc[k] - pk[k];  // exclusive prefix
      next[2 * k] = base_s[2 * k] + static_cast<int>(ex & 0xFFFFu);
      next[2 * k + 1] = base_s[2 * k + 1] + static_cast<int>(ex >> 16);
    }
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      const int e = ids[i];
      if (e < 0) {  // past the end, or an id outside [0, E): no row, like a dropped slot
        if (s0 + i < n_slots) slot_rows[s0 + i] = -1;
        continue;
      }
      int r = 0, off = 0;
#pragma unroll
      for (int ee = 0; ee < kExperts; ++ee)
        if (e == ee) {
          r = next[ee]++;
          off = off_s[ee];
        }
      if (capacity > 0 && r >= capacity) {
        slot_rows[s0 + i] = -1;  // dropped
      } else {
        sorted_slots[off + r] = s0 + i;
        slot_rows[s0 + i] = off + r;
      }
    }
    __syncthreads();  // every thread has read base_s and wave_pk of this chunk
    if (tid < kExperts) {
      const uint32_t t = total[tid / 2];
      base_s[tid] += static_cast<int>((tid & 1) ? (t >> 16) : (t & 0xFFFFu));
    }
    __syncthreads();
  }
}

// Up to one slot per thread: the ballot form of permute_dev.hpp, fewer passes.
__global__ void __launch_bounds__(kPermThreads) permute_small_kernel(const int32_t* __restrict__ idx, int32_t n_slots,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted_slots,
                                                                     int32_t* __restrict__ slot_rows,
                                                                     int32_t* __restrict__ counts_out,
                                                                     int capacity) {
  permute_block(idx, n_slots, offsets, sorted_slots, slot_rows, counts_out, capacity);
}

// One wave per 16-token group (32 slots, lane s < 32 holds slot 32g + s):
// the slots of the earlier groups and of all groups per expert come from
// the router's group counts (each lane adds a strided share, then a wave
// sum), the kept offsets from the totals, and a slot's rank is its group's
// prefix plus its rank among the group's slots of that expert (ballot).
// Same stable order and capacity rule as the one-workgroup form.
__global__ void __launch_bounds__(kWave) permute_groups_kernel(const int32_t* __restrict__ idx, int32_t n_tokens,
                                                               const int32_t* __restrict__ group_counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_slots,
                                                               int32_t* __restrict__ slot_rows,
                                                               int32_t* __restrict__ counts_out, int capacity) {
  const int lane = threadIdx.x;
  const int g = blockIdx.x;
  const int n_groups = (n_tokens + 15) / 16;
  int tot[kExperts], pre[kExperts];
#pragma unroll
  for (int e = 0; e < kExperts; ++e) tot[e] = pre[e] = 0;
  for (int h = lane; h < n_groups; h += kWave) {
    const int4 a = *reinterpret_cast<const int4*>(group_counts + kExperts * h);
    const int4 b = *reinterpret_cast<const int4*>(group_counts + kExperts * h + 4);
    const int c[kExperts] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < kExperts; ++e) {
      tot[e] += c[e];
      pre[e] += h < g ? c[e] : 0;
    }
  }
  int off[kExperts];
  int run = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    tot[e] = wave_sum_int(tot[e]);
    pre[e] = wave_sum_int(pre[e]);
    off[e] = run;
    run += kept_rows(tot[e], capacity);
  }
  if (g == 0 && lane <= kExperts) {
    int v = run, c = 0;
#pragma unroll
    for (int e = 0; e < kExperts; ++e)
      if (lane == e) {
        v = off[e];
        c = tot[e];
      }
    offsets[lane] = v;
    if (counts_out && lane < kExperts) counts_out[lane] = c;
  }
  const int n_slots = n_tokens * kTopK;
  const int s = g * 32 + lane;
  const int e = (lane < 32 && s < n_slots) ? valid_expert(idx[s]) : -1;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int r = 0, o = 0;
#pragma unroll
  for (int ee = 0; ee < kExperts; ++ee) {
    const unsigned long long m = __ballot(e == ee);
    if (e == ee) {
      r = pre[ee] + __popcll(m & below);
      o = off[ee];
    }
  }
  if (lane < 32 && s < n_slots) {
    if (e < 0 || (capacity > 0 && r >= capacity)) {
      slot_rows[s] = -1;  // dropped, or an id outside [0, E)
    } else {
      sorted_slots[o + r] = s;
      slot_rows[s] = o + r;
    }
  }
}

// The valid slots of each 16-token group per expert, group_counts[8g + e]
// (what the bf16 router writes for the layer): one wave per group, four
// groups per workgroup, lane s < 32 holding slot 32g + s.
constexpr int kCountWaves = 4;
__global__ void __launch_bounds__(kCountWaves * kWave) group_counts_kernel(const int32_t* __restrict__ idx,
                                                                           int32_t n_tokens,
                                                                           int32_t* __restrict__ group_counts) {
  const int lane = threadIdx.x % kWave;
  const int g = blockIdx.x * kCountWaves + threadIdx.x / kWave;
  const int n_groups = (n_tokens + 15) / 16;
  if (g >= n_groups) return;
  const int s = g * 32 + lane;
  const int e = (lane < 32 && s < n_tokens * kTopK) ? valid_expert(idx[s]) : -1;
  int mine = 0;
#pragma unroll
  for (int ee = 0; ee < kExperts; ++ee) {
    const int c = __popcll(__ballot(e == ee));
    if (lane == ee) mine = c;
  }
  if (lane < kExperts) group_counts[kExperts * g + lane] = mine;
}

}  // namespace

hipError_t launch_permute_counted(const int32_t* idx, int32_t n_tokens, int32_t* group_counts, int32_t* offsets,
                                  int32_t* sorted_slots, int32_t* slot_rows, int32_t* counts_out, int capacity,
                                  hipStream_t s) {
  if (n_tokens > kMaxGroupPermuteTokens) return hipErrorInvalidValue;
  const int groups = (n_tokens + 15) / 16;
  hipLaunchKernelGGL(group_counts_kernel, dim3((groups + kCountWaves - 1) / kCountWaves), dim3(kCountWaves * kWave),
                     0, s, idx, n_tokens, group_counts);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_permute_groups(idx, n_tokens, group_counts, offsets, sorted_slots, slot_rows, counts_out, capacity,
                               s);
}

hipError_t launch_permute_groups(const int32_t* idx, int32_t n_tokens, const int32_t* group_counts, int32_t* offsets,
                                 int32_t* sorted_slots, int32_t* slot_rows, int32_t* counts_out, int capacity,
                                 hipStream_t s) {
  if (n_tokens > kMaxGroupPermuteTokens) return hipErrorInvalidValue;
  const int groups = (n_tokens + 15) / 16;
  hipLaunchKernelGGL(permute_groups_kernel, dim3(groups), dim3(kWave), 0, s, idx, n_tokens, group_counts, offsets,
                     sorted_slots, slot_rows, counts_out, capacity);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int32_t n_slots, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_rows, int32_t* counts_out, int capacity, hipStream_t s) {
  if (n_slots <= kPermThreads)
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kPermThreads), 0, s, idx, n_slots, offsets, sorted_slots,
                       slot_rows, counts_out, capacity);
  else
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, idx, n_slots, offsets, sorted_slots,
                       slot_rows, counts_out, capacity);
  return hipGetLastError();
}

}  // namespace moe
