// fp32 grouped expert GEMMs (the MOE_F32 dtype): LDS-tiled vector-FMA
// kernels, one 64x64 output tile per workgroup, 4x4 outputs per thread.
//
// Up projection + SwiGLU ("Mixtral of Experts", azimuth.plus, architecture
// paragraph; "Mixtral > Architecture Overview", parameter-count paragraph):
//   h[r, n] = SiLU(sum_i x[tok(r), i] w1_e[n, i]) * (sum_i x[tok(r), i] w3_e[n, i])
// Down projection: y_rows[r, n] = sum_j h[r, j] w2_e[n, j].
// Rows r of expert e are [offsets[e], offsets[e+1]); tok(r) = sorted_slots[r] / k.
// The grid covers an upper bound of the m-tiles; each workgroup finds its
// expert from the device-side offsets and exits if it has no rows.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

template <bool SWIGLU>
__global__ void __launch_bounds__(256) grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                               const int32_t* __restrict__ gather, int k_div,
                                                               const int32_t* __restrict__ offs,
                                                               const float* __restrict__ B0,
                                                               const float* __restrict__ B1, float* __restrict__ C,
                                                               int N, int K, int n_tiles_n) {
  __shared__ float As[kF32BK][kF32BM + 4];
  __shared__ float Bs0[kF32BK][kF32BN + 4];
  __shared__ float Bs1[SWIGLU ? kF32BK : 1][SWIGLU ? kF32BN + 4 : 1];

  const int nt = blockIdx.x % n_tiles_n;
  const int mt = blockIdx.x / n_tiles_n;
  int m0, row_begin, rows;
  const int e = locate_m_tile(offs, mt, kF32BM, &m0, &row_begin, &rows);
  if (e < 0) return;
  const int n0 = nt * kF32BN;

  const int tid = threadIdx.x;
  // loader mapping: 64 rows x 16 k, 4 consecutive k per thread
  const int ld_row = tid / 4;
  const int ld_k = (tid % 4) * 4;
  int a_row = m0 + ld_row;
  if (a_row > rows - 1) a_row = rows - 1;  // clamp: computed, never stored
  const int64_t g = row_begin + a_row;
  const float* a_ptr = A + (gather ? static_cast<int64_t>(gather[g] / k_div) : g) * K;
  int b_row = n0 + ld_row;
  if (b_row > N - 1) b_row = N - 1;
  const float* b0_ptr = B0 + (static_cast<int64_t>(e) * N + b_row) * K;
  const float* b1_ptr = SWIGLU ? B1 + (static_cast<int64_t>(e) * N + b_row) * K : nullptr;

  const int ty = tid / 16, tx = tid % 16;
  float acc0[4][4] = {}, acc1[4][4] = {};

  for (int k0 = 0; k0 < K; k0 += kF32BK) {
    const float4 av = *reinterpret_cast<const float4*>(a_ptr + k0 + ld_k);
    const float4 bv = *reinterpret_cast<const float4*>(b0_ptr + k0 + ld_k);
    As[ld_k + 0][ld_row] = av.x; As[ld_k + 1][ld_row] = av.y; As[ld_k + 2][ld_row] = av.z; As[ld_k + 3][ld_row] = av.w;
    Bs0[ld_k + 0][ld_row] = bv.x; Bs0[ld_k + 1][ld_row] = bv.y; Bs0[ld_k + 2][ld_row] = bv.z; Bs0[ld_k + 3][ld_row] = bv.w;
    if constexpr (SWIGLU) {
      const float4 cv = *reinterpret_cast<const float4*>(b1_ptr + k0 + ld_k);
      Bs1[ld_k + 0][ld_row] = cv.x; Bs1[ld_k + 1][ld_row] = cv.y; Bs1[ld_k + 2][ld_row] = cv.z; Bs1[ld_k + 3][ld_row] = cv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32BK; ++kk) {
      float a[4], b[4], c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs0[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc0[i][j] = fmaf(a[i], b[j], acc0[i][j]);
      if constexpr (SWIGLU) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = Bs1[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc1[i][j] = fmaf(a[i], c[j], acc1[i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= rows) continue;
    float* crow = C + static_cast<int64_t>(row_begin + m) * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      crow[n] = SWIGLU ? silu(acc0[i][j]) * acc1[i][j] : acc0[i][j];
    }
  }
}

hipError_t launch_up_f32(const float* x, const int32_t* offs, const int32_t* sorted_slots, const float* w1,
                         const float* w3, float* h, int64_t n_slots, int d, int f, hipStream_t s) {
  const int64_t m_bound = (n_slots + kF32BM - 1) / kF32BM + kExperts;
  const int nt = (f + kF32BN - 1) / kF32BN;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(m_bound * nt), dim3(256), 0, s, x, sorted_slots, kTopK, offs,
                     w1, w3, h, f, d, nt);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float* h, const int32_t* offs, const float* w2, float* y_rows, int64_t n_slots,
                           int d, int f, hipStream_t s) {
  const int64_t m_bound = (n_slots + kF32BM - 1) / kF32BM + kExperts;
  const int nt = (d + kF32BN - 1) / kF32BN;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(m_bound * nt), dim3(256), 0, s, h,
                     static_cast<const int32_t*>(nullptr), 1, offs, w2, static_cast<const float*>(nullptr), y_rows, d,
                     f, nt);
  return hipGetLastError();
}

}  // namespace moe
