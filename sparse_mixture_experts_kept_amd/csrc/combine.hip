// Gate-weighted combine of the two expert outputs of every token, and the
// RMSNorm + residual glue used between stacked layers.
//
// Combine: "Mixtral & Sparse MoE (2024) > The Solution" (routing paragraph):
// the selected experts' outputs are combined with the routing scores;
// "Mixtral of Experts" (azimuth.plus), router paragraph: the gates set how
// much each expert contributes.  Gather form of the scatter-add: each token
// reads its two rows of y_rows (found through slot_rows) and adds them in
// slot order, so the result is deterministic.  A slot dropped by an expert
// capacity (slot_rows = -1) adds nothing.  HBM-bound: 2*d*4 bytes read and
// d*elem bytes written per token.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// One token row per workgroup pass: the row's slot rows and gates are read
// once (uniform), each thread takes float4 columns c = 4 * (threadIdx.x +
// 256 * j), and the column loop is unrolled so that several rows' loads are
// in flight per thread.
template <typename TO>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y_rows,
                                                      const float* __restrict__ y_rows2,
                                                      const int32_t* __restrict__ slot_rows,
                                                      const float* __restrict__ topk_w, TO* __restrict__ y,
                                                      int64_t T, int d) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int64_t s0 = slot_rows[2 * t];
    const int64_t s1 = slot_rows[2 * t + 1];
    // a dropped slot (row -1) loads row 0, whose value the selects below
    // discard: the loads stay unconditional
    const float* row0 = y_rows + (s0 >= 0 ? s0 : 0) * d;
    const float* row1 = y_rows + (s1 >= 0 ? s1 : 0) * d;
    const float* row0b = y_rows2 ? y_rows2 + (s0 >= 0 ? s0 : 0) * d : nullptr;
    const float* row1b = y_rows2 ? y_rows2 + (s1 >= 0 ? s1 : 0) * d : nullptr;
    const float g0 = topk_w[2 * t];
    const float g1 = topk_w[2 * t + 1];
    const bool k0 = s0 >= 0, k1 = s1 >= 0;
#pragma unroll 4
    for (int c = static_cast<int>(threadIdx.x) * 4; c < d; c += 4 * 256) {
      float4 a = *reinterpret_cast<const float4*>(row0 + c);
      float4 b = *reinterpret_cast<const float4*>(row1 + c);
      if (y_rows2) {  // second partial sum of a split reduction, added to the first
        const float4 a2 = *reinterpret_cast<const float4*>(row0b + c);
        const float4 b2 = *reinterpret_cast<const float4*>(row1b + c);
        a.x = __fadd_rn(a.x, a2.x); a.y = __fadd_rn(a.y, a2.y); a.z = __fadd_rn(a.z, a2.z); a.w = __fadd_rn(a.w, a2.w);
        b.x = __fadd_rn(b.x, b2.x); b.y = __fadd_rn(b.y, b2.y); b.z = __fadd_rn(b.z, b2.z); b.w = __fadd_rn(b.w, b2.w);
      }
      float o[4];
      o[0] = combine_pair(a.x, b.x, g0, g1, k0, k1);
      o[1] = combine_pair(a.y, b.y, g0, g1, k0, k1);
      o[2] = combine_pair(a.z, b.z, g0, g1, k0, k1);
      o[3] = combine_pair(a.w, b.w, g0, g1, k0, k1);
      if constexpr (sizeof(TO) == 4) {
        *reinterpret_cast<float4*>(y + t * d + c) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        uint2 p;
        p.x = pack_bf16x2(o[0], o[1]);
        p.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(y + t * d + c) = p;
      }
    }
  }
}

hipError_t launch_combine(int dtype, const float* y_rows, const float* y_rows2, const int32_t* slot_rows,
                          const float* topk_w, void* y, int64_t T, int d, int n_cu, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t cap = static_cast<int64_t>(n_cu) * 16;
  const int64_t blocks = T < cap ? T : cap;
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, y_rows, y_rows2, slot_rows, topk_w,
                       static_cast<bf16_t*>(y), T, d);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, s, y_rows, y_rows2, slot_rows, topk_w,
                       static_cast<float*>(y), T, d);
  return hipGetLastError();
}

// resid += y_add (optional); u = resid / sqrt(mean(resid^2) + eps).  One
// workgroup per token row; fp32 throughout, u rounded once.
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_residual_kernel(float* __restrict__ resid, const T* __restrict__ y_add,
                                                               T* __restrict__ u, int d, float eps) {
  __shared__ float part[256 / kWave];
  const int64_t t = blockIdx.x;
  float* r = resid + t * d;
  constexpr int kMaxPerThread = 64;  // d <= 16384 with 256 threads
  float v[kMaxPerThread];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int i = threadIdx.x + j * 256;
    v[j] = 0.0f;
    if (i < d) {
      float a = r[i];
      if (y_add) a += to_f32<T>(y_add[t * d + i]);
      v[j] = a;
      ss += a * a;
    }
  }
  ss = wave_sum(ss);
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int i = threadIdx.x + j * 256;
    if (i < d) {
      if (y_add) r[i] = v[j];
      u[t * d + i] = from_f32<T>(v[j] * inv);
    }
  }
}

hipError_t launch_rmsnorm_residual(int dtype, float* resid, const void* y_add, void* u, int64_t T, int d, float eps,
                                   hipStream_t s) {
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(rmsnorm_residual_kernel<bf16_t>, dim3(T), dim3(256), 0, s, resid,
                       static_cast<const bf16_t*>(y_add), static_cast<bf16_t*>(u), d, eps);
  else
    hipLaunchKernelGGL(rmsnorm_residual_kernel<float>, dim3(T), dim3(256), 0, s, resid,
                       static_cast<const float*>(y_add), static_cast<float*>(u), d, eps);
  return hipGetLastError();
}

}  // namespace moe
