// bf16 grouped expert GEMMs for decode-sized batches (few tokens per
// expert), on gfx950 MFMA.  Same functions as the prefill kernels:
//   up:   h[r, n]      = SiLU(x[tok(r)] . w1_e[n]) * (x[tok(r)] . w3_e[n])   -> bf16
//   down: y_rows[r, n] = h[r] . w2_e[n]                                      -> fp32
// ("Mixtral of Experts", azimuth.plus, architecture paragraph; "Mixtral >
// Architecture Overview", parameter-count paragraph.)
//
// With ~8 rows per expert the layer is bound by streaming the touched
// experts' weights from HBM once ("Mixtral of Experts", azimuth.plus,
// paragraph on active versus stored parameters: memory scales with the total
// parameters).  Each wavefront owns 16 weight rows (output features) of one
// expert over the whole reduction and streams them straight from HBM into
// registers as the MFMA src0 operand (16 rows x 32 k per
// v_mfma_f32_16x16x32_bf16); the expert's tokens, padded to groups of 16,
// are the src1 operand, read from L2.  Weights are never staged in LDS: no
// element is used twice by the same wave.  KU k-steps of weight loads are
// issued back to back to keep enough bytes in flight per CU.  Up to 4 token
// groups (64 rows) share one pass over the weights; more rows take more
// passes.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kDThreads = 256;
constexpr int kDMaxGroups = 4;

template <bool SWIGLU, int KU>
__global__ void __launch_bounds__(kDThreads) grouped_gemm_decode_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ gather, int k_div, const int32_t* __restrict__ offs,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, void* __restrict__ Cout, int N, int K) {
  const int lane = threadIdx.x % kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const int fgroups = N / 16;
  const int wid = blockIdx.x * (kDThreads / kWave) + threadIdx.x / kWave;
  const int e = wid / fgroups;
  if (e >= kExperts) return;
  const int fg = wid - e * fgroups;
  const int row_begin = offs[e];
  const int rows = offs[e + 1] - row_begin;
  if (rows <= 0) return;

  const int n_row = fg * 16 + l16;  // weight row this lane streams
  const bf16_t* w0 = B0 + (static_cast<int64_t>(e) * N + n_row) * K + lg * 8;
  const bf16_t* w1 = SWIGLU ? B1 + (static_cast<int64_t>(e) * N + n_row) * K + lg * 8 : nullptr;

  for (int base = 0; base < rows; base += 16 * kDMaxGroups) {
    const int ng = min(kDMaxGroups, (rows - base + 15) / 16);
    const bf16_t* a_ptr[kDMaxGroups];
#pragma unroll
    for (int g = 0; g < kDMaxGroups; ++g) {
      const int m = min(base + g * 16 + l16, rows - 1);  // clamped rows are computed, never stored
      const int64_t gr = row_begin + m;
      const int64_t arow = gather ? static_cast<int64_t>(gather[gr] / k_div) : gr;
      a_ptr[g] = A + arow * K + lg * 8;
    }
    f32x4 acc0[kDMaxGroups], acc1[kDMaxGroups];
#pragma unroll
    for (int g = 0; g < kDMaxGroups; ++g) {
      acc0[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int k0 = 0; k0 < K; k0 += 32 * KU) {
      bf16x8 wa[KU], wb[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        wa[u] = *reinterpret_cast<const bf16x8*>(w0 + k0 + u * 32);
        if constexpr (SWIGLU) wb[u] = *reinterpret_cast<const bf16x8*>(w1 + k0 + u * 32);
      }
#pragma unroll
      for (int g = 0; g < kDMaxGroups; ++g) {
        if (g < ng) {
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            const bf16x8 xa = *reinterpret_cast<const bf16x8*>(a_ptr[g] + k0 + u * 32);
            acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[u], xa, acc0[g], 0, 0, 0);
            if constexpr (SWIGLU) acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[u], xa, acc1[g], 0, 0, 0);
          }
        }
      }
    }

    // acc[g][q]: token row m = base + g*16 + l16, feature n = fg*16 + 4*lg + q.
    const int n = fg * 16 + 4 * lg;
#pragma unroll
    for (int g = 0; g < kDMaxGroups; ++g) {
      const int m = base + g * 16 + l16;
      if (g >= ng || m >= rows) continue;
      const int64_t orow = row_begin + m;
      if constexpr (SWIGLU) {
        const f32x4 a = acc0[g], b = acc1[g];
        uint2 p;
        p.x = pack_bf16x2(silu(a[0]) * b[0], silu(a[1]) * b[1]);
        p.y = pack_bf16x2(silu(a[2]) * b[2], silu(a[3]) * b[3]);
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(Cout) + orow * N + n) = p;
      } else {
        const f32x4 a = acc0[g];
        *reinterpret_cast<float4*>(static_cast<float*>(Cout) + orow * N + n) = make_float4(a[0], a[1], a[2], a[3]);
      }
    }
  }
}

// Down projection fused with the gate-weighted combine, for batches of at
// most 64 tokens (so no expert has more than 64 rows).  Workgroup b owns
// output features n0 = 16 b .. n0+15 of every expert: wave w streams w2 rows
// n0.. of expert w/2 over half w%2 of the reduction (f/2 each) with the same
// MFMA scheme as above, parks its partial sums in LDS, and after a barrier the
// workgroup forms y[t, n0+c] = g_t0 (P0 + P1)[r0] + g_t1 (P0 + P1)[r1] for
// every token in a fixed order (deterministic), rounded once to bf16.
constexpr int kDcThreads = 1024;   // 16 waves: 8 experts x 2 halves of f
constexpr int kDcMaxRows = 64;

template <int KU>
__global__ void __launch_bounds__(kDcThreads) down_combine_decode_kernel(
    const bf16_t* __restrict__ H, const int32_t* __restrict__ offs, const bf16_t* __restrict__ w2,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ slot_rows, const float* __restrict__ topk_w,
    bf16_t* __restrict__ y, int T, int d, int f) {
  __shared__ float part[kDcThreads / kWave][kDcMaxRows][16];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const int e = wave / 2, half = wave % 2;
  const int n0 = blockIdx.x * 16;
  const int row_begin = offs[e];
  const int rows = offs[e + 1] - row_begin;  // <= kDcMaxRows (T <= 64)
  const int kh = f / 2;

  if (rows > 0) {
    const bf16_t* wrow = w2 + (static_cast<int64_t>(e) * d + n0 + l16) * f + half * kh + lg * 8;
    const int ng = (rows + 15) / 16;
    const bf16_t* a_ptr[kDMaxGroups];
#pragma unroll
    for (int g = 0; g < kDMaxGroups; ++g) {
      const int m = min(g * 16 + l16, rows - 1);  // clamped rows are computed, never used
      a_ptr[g] = H + static_cast<int64_t>(row_begin + m) * f + half * kh + lg * 8;
    }
    f32x4 acc[kDMaxGroups];
#pragma unroll
    for (int g = 0; g < kDMaxGroups; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < kh; k0 += 32 * KU) {
      bf16x8 wa[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) wa[u] = *reinterpret_cast<const bf16x8*>(wrow + k0 + u * 32);
#pragma unroll
      for (int g = 0; g < kDMaxGroups; ++g) {
        if (g < ng) {
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            const bf16x8 ha = *reinterpret_cast<const bf16x8*>(a_ptr[g] + k0 + u * 32);
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[u], ha, acc[g], 0, 0, 0);
          }
        }
      }
    }
    // acc[g][q]: expert row g*16 + l16, feature 4*lg + q
#pragma unroll
    for (int g = 0; g < kDMaxGroups; ++g) {
      const int m = g * 16 + l16;
      if (g < ng && m < rows) {
#pragma unroll
        for (int q = 0; q < 4; ++q) part[wave][m][4 * lg + q] = acc[g][q];
      }
    }
  }
  __syncthreads();

  // Combine: thread (t, c) for token t < T <= 64 and feature column c < 16.
  const int t = threadIdx.x / 16, c = threadIdx.x % 16;
  if (t < T) {
    float o = 0.0f;
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const int ej = topk_idx[kTopK * t + j];
      const int r = slot_rows[kTopK * t + j] - offs[ej];
      const float v = part[2 * ej][r][c] + part[2 * ej + 1][r][c];
      o = (j == 0) ? topk_w[kTopK * t] * v : o + topk_w[kTopK * t + j] * v;
    }
    y[static_cast<int64_t>(t) * d + n0 + c] = f32_to_bf16(o);
  }
}

template <bool SWIGLU, int KU>
static hipError_t launch_one_decode(const bf16_t* A, const int32_t* gather, int k_div, const int32_t* offs,
                                    const bf16_t* B0, const bf16_t* B1, void* C, int N, int K, hipStream_t s) {
  const int waves = kExperts * (N / 16);
  const int per_block = kDThreads / kWave;
  const int blocks = (waves + per_block - 1) / per_block;
  hipLaunchKernelGGL((grouped_gemm_decode_kernel<SWIGLU, KU>), dim3(blocks), dim3(kDThreads), 0, s, A, gather, k_div,
                     offs, B0, B1, C, N, K);
  return hipGetLastError();
}

hipError_t launch_up_decode(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                            const bf16_t* w3, bf16_t* h, int d, int f, hipStream_t s) {
  // K = d; KU * 32 must divide it (d % 128 == 0, so KU = 4 always works).
  if (d % 256 == 0) return launch_one_decode<true, 8>(x, sorted_slots, kTopK, offs, w1, w3, h, f, d, s);
  return launch_one_decode<true, 4>(x, sorted_slots, kTopK, offs, w1, w3, h, f, d, s);
}

hipError_t launch_down_combine_decode(const bf16_t* h, const int32_t* offs, const bf16_t* w2, const int32_t* topk_idx,
                                      const int32_t* slot_rows, const float* topk_w, bf16_t* y, int T, int d, int f,
                                      hipStream_t s) {
  // each wave covers f/2 in steps of 32*KU
  const int kh = f / 2;
  if (kh % 512 == 0)
    hipLaunchKernelGGL(down_combine_decode_kernel<16>, dim3(d / 16), dim3(kDcThreads), 0, s, h, offs, w2, topk_idx,
                       slot_rows, topk_w, y, T, d, f);
  else
    hipLaunchKernelGGL(down_combine_decode_kernel<2>, dim3(d / 16), dim3(kDcThreads), 0, s, h, offs, w2, topk_idx,
                       slot_rows, topk_w, y, T, d, f);
  return hipGetLastError();
}

hipError_t launch_down_decode(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int d, int f,
                              hipStream_t s) {
  if (f % 512 == 0) return launch_one_decode<false, 16>(h, nullptr, 1, offs, w2, nullptr, y_rows, d, f, s);
  return launch_one_decode<false, 4>(h, nullptr, 1, offs, w2, nullptr, y_rows, d, f, s);
}

}  // namespace moe
