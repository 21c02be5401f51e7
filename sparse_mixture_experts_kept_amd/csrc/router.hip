// Router: scores x W_g^T, top-2 selection and the softmax over the kept pair.
// "Mixtral of Experts" (azimuth.plus), router paragraph: one linear map to 8
// scores, keep the two largest, all others -inf, softmax over the survivors.
//
// One wavefront per token.  The router matrix W_g [8, d] is staged once per
// workgroup in LDS; each lane accumulates 8 fp32 partial dot products over
// its share of d, a butterfly (xor-shuffle) sum gives every lane all 8
// scores, and lane 0 selects the pair in registers and writes it.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <typename T>
__global__ void __launch_bounds__(256) router_top2_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                          const float* __restrict__ bias, int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out, float* __restrict__ logits_out,
                                                          int64_t T_tokens, int d) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* wg_s = reinterpret_cast<T*>(smem_raw);
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load

  // Stage W_g in LDS (E * d elements, d a multiple of 128).
  const int n_vec = kExperts * d / VEC;
  for (int i = threadIdx.x; i < n_vec; i += blockDim.x)
    reinterpret_cast<uint4*>(wg_s)[i] = reinterpret_cast<const uint4*>(wg)[i];
  __syncthreads();

  const int lane = threadIdx.x % kWave;
  const int waves_per_block = blockDim.x / kWave;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * waves_per_block + threadIdx.x / kWave;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * waves_per_block;

  float b[kExperts];
#pragma unroll
  for (int e = 0; e < kExperts; ++e) b[e] = bias ? bias[e] : 0.0f;

  for (int64_t t = wave_id; t < T_tokens; t += n_waves) {
    const T* xr = x + t * d;
    float acc[kExperts];
#pragma unroll
    for (int e = 0; e < kExperts; ++e) acc[e] = 0.0f;
    for (int i = lane * VEC; i < d; i += kWave * VEC) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xr + i);
      const T* xe = reinterpret_cast<const T*>(&xv);
      float xf[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) xf[v] = to_f32<T>(xe[v]);
#pragma unroll
      for (int e = 0; e < kExperts; ++e) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wg_s + e * d + i);
        const T* we = reinterpret_cast<const T*>(&wv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[e] = fmaf(xf[v], to_f32<T>(we[v]), acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < kExperts; ++e) acc[e] = wave_sum(acc[e]) + b[e];

    if (lane == 0) {
      // Two largest, larger first; strict '>' keeps the lower index on ties.
      int ia = 0;
      float la = acc[0];
#pragma unroll
      for (int e = 1; e < kExperts; ++e)
        if (acc[e] > la) { la = acc[e]; ia = e; }
      int ib = -1;
      float lb = 0.0f;
#pragma unroll
      for (int e = 0; e < kExperts; ++e)
        if (e != ia && (ib < 0 || acc[e] > lb)) { lb = acc[e]; ib = e; }
      // softmax over {la, lb} with the others at -inf
      const float r = expf(lb - la);
      const float ga = 1.0f / (1.0f + r);
      const float gb = r / (1.0f + r);
      idx_out[2 * t] = ia;
      idx_out[2 * t + 1] = ib;
      w_out[2 * t] = ga;
      w_out[2 * t + 1] = gb;
    }
    if (logits_out && lane < kExperts) {
      float v = acc[0];
#pragma unroll
      for (int e = 1; e < kExperts; ++e)
        if (lane == e) v = acc[e];
      logits_out[t * kExperts + lane] = v;
    }
  }
}

hipError_t launch_router(int dtype, const void* x, const void* wg, const float* bias, int32_t* idx, float* w,
                         float* logits, int64_t T, int d, int n_cu, hipStream_t s) {
  const int threads = 256;
  const size_t elem = dtype == kDtypeBF16 ? 2 : 4;
  const size_t lds = kExperts * static_cast<size_t>(d) * elem;
  // Enough workgroups to cover every CU twice; each wave loops over tokens.
  int64_t blocks = (T + 3) / 4;
  const int64_t cap = static_cast<int64_t>(n_cu) * 2;
  if (blocks > cap) blocks = cap;
  if (lds > 64 * 1024) {
    const void* fn = dtype == kDtypeBF16 ? reinterpret_cast<const void*>(&router_top2_kernel<bf16_t>)
                                         : reinterpret_cast<const void*>(&router_top2_kernel<float>);
    const hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
  }
  if (dtype == kDtypeBF16) {
    hipLaunchKernelGGL(router_top2_kernel<bf16_t>, dim3(blocks), dim3(threads), lds, s,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(wg), bias, idx, w, logits, T, d);
  } else {
    hipLaunchKernelGGL(router_top2_kernel<float>, dim3(blocks), dim3(threads), lds, s,
                       static_cast<const float*>(x), static_cast<const float*>(wg), bias, idx, w, logits, T, d);
  }
  return hipGetLastError();
}

}  // namespace moe
