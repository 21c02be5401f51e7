// The chip's bf16 matrix-core ceiling under its power limit, measured: the
// prefill GEMM's MFMA pattern with nothing else.  Each wave holds the GEMM's
// 128 x 128 wave tile (8 x 8 v_mfma_f32_16x16x32_bf16 tiles, 256 fp32
// accumulators) and issues its 64 MFMAs per 32-deep step over and over on
// distinct operand fragments taken from the caller's data, one wave per
// SIMD on every CU (the GEMM's occupancy), so the matrix cores run at the
// clock their own power draw allows.  The achieved rate against this
// ceiling separates what the GEMM loses to its loads, LDS traffic and
// epilogues from what the chip gives dense bf16 MFMA work with such data.
// Per workgroup the shader clock counter and the constant 100 MHz reference
// counter are stored at the start and the end of the loop.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_ceiling_kernel(const bf16x8* __restrict__ operands, long long* __restrict__ clk, float* __restrict__ sink,
                    int iters) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  // 16 distinct fragments per wave (8 for each operand), different per wave
  bf16x8 fa[8], fb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fa[i] = operands[((wave * 16 + i) % 64) * kWave + lane];
    fb[i] = operands[((wave * 16 + 8 + i) % 64) * kWave + lane];
  }
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const long long cyc0 = __builtin_amdgcn_s_memtime();
  const long long ref0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  const long long cyc1 = __builtin_amdgcn_s_memtime();
  const long long ref1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;  // keeps the MFMAs live
  if (threadIdx.x == 0) {
    long long* c = clk + 4 * static_cast<int64_t>(blockIdx.x);
    c[0] = cyc0;
    c[1] = cyc1;
    c[2] = ref0;
    c[3] = ref1;
  }
}

}  // namespace

hipError_t launch_mfma_ceiling(const bf16_t* operands, long long* clk, float* sink, int iters, int n_cu,
                               hipStream_t s) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(prefill_grid(n_cu)), dim3(256), 0, s,
                     reinterpret_cast<const bf16x8*>(operands), clk, sink, iters);
  return hipGetLastError();
}

}  // namespace moe
