// Router: scores x W_g^T, top-2 selection and the softmax over the kept pair.
// "Mixtral of Experts" (azimuth.plus), router paragraph: one linear map to 8
// scores, keep the two largest, all others -inf, softmax over the survivors.
// (Or, with the full gating, the softmax over all 8 scores of "Mixtral &
// Sparse MoE (2024) > The Solution": see select_top2.)
//
// bf16: the scores are a [T, d] x [d, 8] contraction and run on MFMA (the 8
// router rows padded to 16), the reduction over d split across waves and
// summed in LDS in a fixed order; lanes then select the pair per token.
// fp32: one wavefront per token; the router matrix W_g [8, d] is staged in
// LDS, each lane accumulates 8 fp32 partial dot products over its share of
// d, a butterfly (xor-shuffle) sum gives every lane all 8 scores, and lane 0
// selects the pair.  For small batches (T <= 64) the routing is followed by
// the slot sort in the same workgroup: bf16 after a launch that computes the
// router's d-slices on one workgroup each, fp32 in a single workgroup.
#include "common.hpp"
#include "launch.hpp"
#include "permute_dev.hpp"

namespace moe {

// Top-2 from the 8 scores (larger first; strict '>' keeps the lower index
// on ties) and the two gates.  kGatingPair: softmax over the kept pair with
// the other six at -inf, g_a = 1/(1+r), g_b = r/(1+r), r = exp(l_b - l_a)
// ("Mixtral of Experts", azimuth.plus, router paragraph).  kGatingFull:
// softmax over all eight scores, the pair's probabilities kept as they are
// (no renormalisation), g = (1, r) / sum_e exp(l_e - l_a), summed in expert
// order ("Mixtral & Sparse MoE (2024) > The Solution", routing paragraph).
__device__ __forceinline__ void select_top2(const float* sc, int gating, int32_t* idx_out, float* w_out) {
  int ia = 0;
  float la = sc[0];
#pragma unroll
  for (int e = 1; e < kExperts; ++e)
    if (sc[e] > la) { la = sc[e]; ia = e; }
  int ib = -1;
  float lb = 0.0f;
#pragma unroll
  for (int e = 0; e < kExperts; ++e)
    if (e != ia && (ib < 0 || sc[e] > lb)) { lb = sc[e]; ib = e; }
  const float r = expf(lb - la);
  float den = 1.0f + r;
  if (gating == kGatingFull) {
    den = 0.0f;
#pragma unroll
    for (int e = 0; e < kExperts; ++e) den += expf(sc[e] - la);
  }
  idx_out[0] = ia;
  idx_out[1] = ib;
  w_out[0] = 1.0f / den;
  w_out[1] = r / den;
}

// Route one token with one wavefront: 8 fp32 dot products over d (the
// router matrix is in LDS), butterfly sums so every lane holds all 8 scores,
// then lane 0 keeps the two largest and their gates (select_top2).
template <typename T>
__device__ __forceinline__ void route_token(const T* __restrict__ xr, const T* wg_s, const float* b, int d, int lane,
                                            int gating, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                            float* __restrict__ logits_out) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  // A lane's x chunks are loaded kChunks at a time before any arithmetic, so
  // a token costs one memory latency per kChunks * 64 * VEC elements.
  constexpr int kChunks = 8;
  float acc[kExperts];
#pragma unroll
  for (int e = 0; e < kExperts; ++e) acc[e] = 0.0f;
  for (int base = 0; base < d; base += kChunks * kWave * VEC) {
    uint4 xv[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)  // clamped, unconditional: one latency for all
      xv[c] = *reinterpret_cast<const uint4*>(xr + min(base + (lane + c * kWave) * VEC, d - VEC));
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int i = base + (lane + c * kWave) * VEC;
      if (i < d) {
        const T* xe = reinterpret_cast<const T*>(&xv[c]);
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
    }
  }
#pragma unroll
  for (int e = 0; e < kExperts; ++e) acc[e] = wave_sum(acc[e]) + b[e];

  if (lane == 0) select_top2(acc, gating, idx_out, w_out);
  if (logits_out && lane < kExperts) {
    float v = acc[0];
#pragma unroll
    for (int e = 1; e < kExperts; ++e)
      if (lane == e) v = acc[e];
    logits_out[lane] = v;
  }
}

// Stage W_g [8, d] in LDS (d a multiple of 128) and the bias in registers.
template <typename T>
__device__ __forceinline__ void stage_router(const T* __restrict__ wg, const float* __restrict__ bias, T* wg_s, int d,
                                             float* b) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int kBatch = 8;  // loads in flight per thread before the LDS stores
  const int n_vec = kExperts * d / VEC;
  const int step = blockDim.x;
  for (int base = threadIdx.x; base < n_vec; base += kBatch * step) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)  // unconditional (clamped) loads issue back to back
      v[u] = reinterpret_cast<const uint4*>(wg)[min(base + u * step, n_vec - 1)];
    // Out-of-range slots load and store the last element (same value), so the
    // stores need no branch either.
#pragma unroll
    for (int u = 0; u < kBatch; ++u) reinterpret_cast<uint4*>(wg_s)[min(base + u * step, n_vec - 1)] = v[u];
  }
#pragma unroll
  for (int e = 0; e < kExperts; ++e) b[e] = bias ? bias[e] : 0.0f;
  __syncthreads();
}

template <typename T>
__global__ void __launch_bounds__(256) router_top2_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                          const float* __restrict__ bias, int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out, float* __restrict__ logits_out,
                                                          int64_t T_tokens, int d, int gating) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* wg_s = reinterpret_cast<T*>(smem_raw);
  float b[kExperts];
  stage_router(wg, bias, wg_s, d, b);
  const int lane = threadIdx.x % kWave;
  const int waves_per_block = blockDim.x / kWave;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * waves_per_block + threadIdx.x / kWave;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  for (int64_t t = wave_id; t < T_tokens; t += n_waves)
    route_token(x + t * d, wg_s, b, d, lane, gating, idx_out + 2 * t, w_out + 2 * t,
                logits_out ? logits_out + t * kExperts : nullptr);
}

// The residual add and RMSNorm of the glue between stacked layers with the
// next layer's router fused in: resid += y_add (optional); u = resid /
// sqrt(mean(resid^2) + eps) rounded to T; then that layer's scores from the
// rounded u (what the router would read back), top-2 and gates
// (select_top2).  One wavefront per token row, W_g staged in LDS once per
// workgroup; a lane keeps its d/64 elements of the row in registers (8
// consecutive ones per 16-byte step), so the row is read once.  ("Mixtral
// of Experts", azimuth.plus, router paragraph, for the routing; the norm is
// the stacked workload's glue.)
// 8 consecutive elements of T as floats (16 or 32 bytes, aligned), and back.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out) {
  if constexpr (sizeof(T) == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 c = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const T* e = reinterpret_cast<const T*>(&a);
#pragma unroll
    for (int q = 0; q < 8; ++q) out[q] = to_f32<T>(e[q]);
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const T* in) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(in[4], in[5], in[6], in[7]);
  } else {
    uint4 a;
    T* e = reinterpret_cast<T*>(&a);
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = in[q];
    *reinterpret_cast<uint4*>(p) = a;
  }
}

// The addend of the glue: the layer's output y_add [T, d] (dtype, or none),
// or (COMBINE) the layer's combine itself, y[t] = g0 * y_rows[slot_rows[2t]]
// + g1 * y_rows[slot_rows[2t+1]] (each row plus its second partial y_rows2
// when the down projection split its reduction), computed and rounded to the
// dtype exactly as combine_kernel does it, so y is never written.
struct GlueAddend {
  const void* y_add;
  const float* y_rows;
  const float* y_rows2;
  const int32_t* slot_rows;
  const float* gates;
};

// With wg == nullptr the routing is skipped (the glue after the last layer).
// A row is kSteps steps of 8 elements per lane (d <= 512 * kSteps); rows of
// up to 4096 take half the registers, and eight waves then share the LDS
// copy of W_g (twice the waves per CU).
template <typename T, bool COMBINE, int kSteps>
__global__ void __launch_bounds__(kSteps <= 8 ? 512 : 256)
    __attribute__((amdgpu_waves_per_eu(kSteps <= 8 ? 4 : 1))) rmsnorm_route_kernel(float* __restrict__ resid,
                                                                                    GlueAddend add,
                                                            T* __restrict__ u, const T* __restrict__ wg,
                                                            const float* __restrict__ bias,
                                                            int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                            int64_t T_tokens, int d, float eps, int gating) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* wg_s = reinterpret_cast<T*>(smem_raw);
  float b[kExperts];
  if (wg) stage_router(wg, bias, wg_s, d, b);
  const T* __restrict__ y_add = static_cast<const T*>(add.y_add);
  constexpr int kVec = 8;                       // elements per lane and step
  static_assert(kSteps * kWave * kVec <= kMaxNormRouteD, "row length");
  const int lane = threadIdx.x % kWave;
  const int waves_per_block = blockDim.x / kWave;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * waves_per_block + threadIdx.x / kWave; t < T_tokens;
       t += n_waves) {
    float* r = resid + t * d;
    // COMBINE: the token's two rows and gates (a dropped slot, row -1, reads
    // row 0 and adds nothing, as in combine_kernel)
    int64_t s0 = 0, s1 = 0;
    float g0 = 0.0f, g1 = 0.0f;
    bool k0 = false, k1 = false;
    if constexpr (COMBINE) {
      s0 = add.slot_rows[2 * t];
      s1 = add.slot_rows[2 * t + 1];
      g0 = add.gates[2 * t];
      g1 = add.gates[2 * t + 1];
      k0 = s0 >= 0;
      k1 = s1 >= 0;
      s0 = k0 ? s0 : 0;
      s1 = k1 ? s1 : 0;
    }
    float v[kSteps][kVec];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int i = (j * kWave + lane) * kVec;
#pragma unroll
      for (int q = 0; q < kVec; ++q) v[j][q] = 0.0f;
      if (i < d) {
        const float4 r0 = *reinterpret_cast<const float4*>(r + i);
        const float4 r1 = *reinterpret_cast<const float4*>(r + i + 4);
        v[j][0] = r0.x; v[j][1] = r0.y; v[j][2] = r0.z; v[j][3] = r0.w;
        v[j][4] = r1.x; v[j][5] = r1.y; v[j][6] = r1.z; v[j][7] = r1.w;
        bool added = false;
        if constexpr (COMBINE) {
          float a[kVec], c[kVec];
          load8(add.y_rows + s0 * d + i, a);
          load8(add.y_rows + s1 * d + i, c);
          if (add.y_rows2) {
            float a2[kVec], c2[kVec];
            load8(add.y_rows2 + s0 * d + i, a2);
            load8(add.y_rows2 + s1 * d + i, c2);
#pragma unroll
            for (int q = 0; q < kVec; ++q) {
              a[q] = __fadd_rn(a[q], a2[q]);
              c[q] = __fadd_rn(c[q], c2[q]);
            }
          }
#pragma unroll
          for (int q = 0; q < kVec; ++q)
            v[j][q] += to_f32<T>(from_f32<T>(combine_pair(a[q], c[q], g0, g1, k0, k1)));
          added = true;
        } else if (y_add) {
          float ya[kVec];
          load8(y_add + t * d + i, ya);
#pragma unroll
          for (int q = 0; q < kVec; ++q) v[j][q] += ya[q];
          added = true;
        }
        if (added) {
          *reinterpret_cast<float4*>(r + i) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
          *reinterpret_cast<float4*>(r + i + 4) = make_float4(v[j][4], v[j][5], v[j][6], v[j][7]);
        }
#pragma unroll
        for (int q = 0; q < kVec; ++q) ss += v[j][q] * v[j][q];
      }
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
    float acc[kExperts];
#pragma unroll
    for (int e = 0; e < kExperts; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int i = (j * kWave + lane) * kVec;
      if (i < d) {
        T uq[kVec];
        float uf[kVec];
#pragma unroll
        for (int q = 0; q < kVec; ++q) {
          uq[q] = from_f32<T>(v[j][q] * inv);
          uf[q] = to_f32<T>(uq[q]);
        }
        store8(u + t * d + i, uq);
        if (wg) {
#pragma unroll
          for (int e = 0; e < kExperts; ++e) {
            float wf[kVec];
            load8(wg_s + e * d + i, wf);
#pragma unroll
            for (int q = 0; q < kVec; ++q) acc[e] = fmaf(uf[q], wf[q], acc[e]);
          }
        }
      }
    }
    if (wg) {
#pragma unroll
      for (int e = 0; e < kExperts; ++e) acc[e] = wave_sum(acc[e]) + b[e];
      if (lane == 0) select_top2(acc, gating, idx_out + kTopK * t, w_out + kTopK * t);
    }
  }
}

namespace {
template <typename T, bool COMBINE, int kSteps>
hipError_t launch_glue_rows(float* resid, const GlueAddend& add, void* u, const void* wg, const float* bias,
                            int32_t* idx, float* w, int64_t n_tokens, int d, float eps, int gating, int n_cu,
                            hipStream_t s) {
  constexpr int kThreads = kSteps <= 8 ? 512 : 256;
  constexpr int kRowsPerBlock = kThreads / kWave;  // a wave per row at a time
  const size_t lds = wg ? kExperts * static_cast<size_t>(d) * sizeof(T) : 0;
  if (lds > 64 * 1024) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&rmsnorm_route_kernel<T, COMBINE, kSteps>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
  }
  int64_t blocks = (n_tokens + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t cap = static_cast<int64_t>(n_cu) * 2;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((rmsnorm_route_kernel<T, COMBINE, kSteps>), dim3(blocks), dim3(kThreads), lds, s, resid, add,
                     static_cast<T*>(u), static_cast<const T*>(wg), bias, idx, w, n_tokens, d, eps, gating);
  return hipGetLastError();
}

template <typename T, bool COMBINE>
hipError_t launch_glue(float* resid, const GlueAddend& add, void* u, const void* wg, const float* bias, int32_t* idx,
                       float* w, int64_t n_tokens, int d, float eps, int gating, int n_cu, hipStream_t s) {
  if (d <= 8 * kWave * 8)
    return launch_glue_rows<T, COMBINE, 8>(resid, add, u, wg, bias, idx, w, n_tokens, d, eps, gating, n_cu, s);
  return launch_glue_rows<T, COMBINE, kMaxNormRouteD / (kWave * 8)>(resid, add, u, wg, bias, idx, w, n_tokens, d,
                                                                    eps, gating, n_cu, s);
}
}  // namespace

hipError_t launch_rmsnorm_route(int dtype, float* resid, const void* y_add, void* u, const void* wg,
                                const float* bias, int32_t* idx, float* w, int64_t T, int d, float eps, int gating,
                                int n_cu, hipStream_t s) {
  const GlueAddend add{y_add, nullptr, nullptr, nullptr, nullptr};
  if (dtype == kDtypeBF16)
    return launch_glue<bf16_t, false>(resid, add, u, wg, bias, idx, w, T, d, eps, gating, n_cu, s);
  return launch_glue<float, false>(resid, add, u, wg, bias, idx, w, T, d, eps, gating, n_cu, s);
}

hipError_t launch_combine_rmsnorm_route(int dtype, const float* y_rows, const float* y_rows2, const int32_t* slot_rows,
                                        const float* gates, float* resid, void* u, const void* wg, const float* bias,
                                        int32_t* idx, float* w, int64_t T, int d, float eps, int gating, int n_cu,
                                        hipStream_t s) {
  const GlueAddend add{nullptr, y_rows, y_rows2, slot_rows, gates};
  if (dtype == kDtypeBF16)
    return launch_glue<bf16_t, true>(resid, add, u, wg, bias, idx, w, T, d, eps, gating, n_cu, s);
  return launch_glue<float, true>(resid, add, u, wg, bias, idx, w, T, d, eps, gating, n_cu, s);
}

// bf16 scores on MFMA: one 16-token group times the 8 router rows (padded to
// 16 with zeros) per v_mfma_f32_16x16x32_bf16, with fp32 accumulation (the
// bf16 products are exact in fp32, as in the VALU form).  `slices` waves
// split the reduction over d; their partial scores meet in LDS and are added
// in slice order.  Returns, in lanes 0..15 of the reducing wave, the 8
// scores of token (group*16 + lane) in s[0..7].
__device__ __forceinline__ f32x4 router_scores_partial(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                                       int T, int d, int group, int slice, int slices, int lane) {
  const int l16 = lane % 16, lg = lane / 16;
  const int tok = min(group * 16 + l16, T - 1);  // clamped rows are computed, never written
  const int ks = d / slices;                       // a multiple of 32 (see router_slices)
  const bf16_t* xp = x + static_cast<int64_t>(tok) * d + slice * ks + lg * 8;
  const bool real_row = l16 < kExperts;            // rows 8..15 of the padded router are zero
  const bf16_t* wp = wg + static_cast<int64_t>(real_row ? l16 : 0) * d + slice * ks + lg * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  // ks is only a multiple of 32: the k-steps go in batches of 8 whose loads
  // are all issued before their MFMAs (one memory latency per batch, not
  // per step), then one step at a time.
  constexpr int kBatch = 8;
  int k0 = 0;
  for (; k0 + kBatch * 32 <= ks; k0 += kBatch * 32) {
    bf16x8 wa[kBatch], xa[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      wa[j] = real_row ? *reinterpret_cast<const bf16x8*>(wp + k0 + 32 * j) : zero;  // rows 8..15: no load
      xa[j] = *reinterpret_cast<const bf16x8*>(xp + k0 + 32 * j);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[j], xa[j], acc, 0, 0, 0);
  }
  for (; k0 < ks; k0 += 32) {
    const bf16x8 wa = real_row ? *reinterpret_cast<const bf16x8*>(wp + k0) : zero;
    const bf16x8 xa = *reinterpret_cast<const bf16x8*>(xp + k0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xa, acc, 0, 0, 0);
  }
  // acc[q] = score of expert 4*lg + q for token l16 (meaningful for lg < 2)
  return acc;
}

// Number of d-slices (waves) per 16-token group: the largest power of two up
// to `cap` with d divisible by 32 * slices (d % 128 == 0 gives at least 4).
__host__ __device__ inline int router_slices(int d, int cap) {
  int sl = cap;
  while (sl > 4 && d % (32 * sl) != 0) sl /= 2;
  return sl;
}

// Reduce the slice partials of one 16-token group (parked in LDS as
// part[slice][lane] = f32x4) and route its tokens; run by one wave.
// With group_counts, also the group's slots per expert (group_counts[8*group + e]).
__device__ __forceinline__ void router_finish_group(const f32x4 (*part)[kWave], int slices, int group, int T,
                                                    const float* __restrict__ bias, int lane, int gating,
                                                    int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                    float* __restrict__ logits_out,
                                                    int32_t* __restrict__ group_counts) {
  f32x4 sum = part[0][lane];
  for (int sl = 1; sl < slices; ++sl) {
    const f32x4 v = part[sl][lane];
    sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
  }
  // lane t < 16 holds experts 0..3 of token t, lane t+16 experts 4..7
  float sc[kExperts];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    sc[q] = sum[q];
    sc[4 + q] = __shfl(sum[q], (lane % 16) + 16, kWave);
  }
  const int t = group * 16 + lane;
  int32_t pair[kTopK] = {-1, -1};
  if (lane < 16 && t < T) {
#pragma unroll
    for (int e = 0; e < kExperts; ++e) sc[e] += bias ? bias[e] : 0.0f;
    float gate[kTopK];
    select_top2(sc, gating, pair, gate);
    idx_out[kTopK * t] = pair[0];
    idx_out[kTopK * t + 1] = pair[1];
    w_out[kTopK * t] = gate[0];
    w_out[kTopK * t + 1] = gate[1];
    if (logits_out) {
#pragma unroll
      for (int e = 0; e < kExperts; ++e) logits_out[static_cast<int64_t>(t) * kExperts + e] = sc[e];
    }
  }
  if (group_counts) {
    int mine = 0;  // lane e < 8: the group's slots on expert e
#pragma unroll
    for (int e = 0; e < kExperts; ++e) {
      const int c = __popcll(__ballot(pair[0] == e)) + __popcll(__ballot(pair[1] == e));
      if (lane == e) mine = c;
    }
    if (lane < kExperts) group_counts[kExperts * group + lane] = mine;
  }
}

// Router for bf16: workgroup b routes tokens 16b..16b+15; its 16 waves
// split d into router_slices(d, 16) slices (idle waves when fewer).
__global__ void __launch_bounds__(1024) router_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                                           const float* __restrict__ bias,
                                                           int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                           float* __restrict__ logits_out, int T, int d,
                                                           int gating, int32_t* __restrict__ group_counts) {
  __shared__ f32x4 part[16][kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int slices = router_slices(d, 16);
  if (wave < slices) part[wave][lane] = router_scores_partial(x, wg, T, d, blockIdx.x, wave, slices, lane);
  __syncthreads();
  if (wave == 0)
    router_finish_group(part, slices, blockIdx.x, T, bias, lane, gating, idx_out, w_out, logits_out, group_counts);
}

// fp32 small batches: routing and the expert-major permutation in one
// workgroup (one launch and one global round trip fewer).  16 waves route
// the tokens, then the same workgroup sorts the slots.
template <typename T>
__global__ void __launch_bounds__(kPermThreads) route_permute_kernel(
    const T* __restrict__ x, const T* __restrict__ wg, const float* __restrict__ bias, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t T_tokens, int d, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_rows, int32_t* __restrict__ counts_out,
    int gating, int capacity) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* wg_s = reinterpret_cast<T*>(smem_raw);
  float b[kExperts];
  stage_router(wg, bias, wg_s, d, b);
  const int lane = threadIdx.x % kWave;
  for (int t = threadIdx.x / kWave; t < T_tokens; t += kPermWaves)
    route_token(x + static_cast<int64_t>(t) * d, wg_s, b, d, lane, gating, idx_out + 2 * t, w_out + 2 * t, nullptr);
  __syncthreads();  // the ids written above are read back by permute_block
  permute_block(idx_out, T_tokens * kTopK, offsets, sorted_slots, slot_rows, counts_out, capacity);
}

hipError_t launch_router(int dtype, const void* x, const void* wg, const float* bias, int32_t* idx, float* w,
                         float* logits, int64_t T, int d, int gating, int n_cu, hipStream_t s,
                         int32_t* group_counts) {
  if (dtype == kDtypeBF16) {
    const int64_t groups = (T + 15) / 16;
    hipLaunchKernelGGL(router_mfma_kernel, dim3(groups), dim3(1024), 0, s, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(wg), bias, idx, w, logits, static_cast<int>(T), d, gating,
                       group_counts);
    return hipGetLastError();
  }
  if (group_counts) return hipErrorInvalidValue;  // only the bf16 router counts per group
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
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(wg), bias, idx, w, logits, T, d,
                       gating);
  } else {
    hipLaunchKernelGGL(router_top2_kernel<float>, dim3(blocks), dim3(threads), lds, s,
                       static_cast<const float*>(x), static_cast<const float*>(wg), bias, idx, w, logits, T, d,
                       gating);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// bf16 small batches (T <= 64), in two launches: route_slices_kernel runs
// one single-wave workgroup per d-slice (router_slices(d, 16) of them, each
// on its own CU), which multiplies its slice of every token group (up to 4
// groups of 16) by the router rows and stores the partial scores;
// route_finish_kernel (one workgroup) adds the partials in slice order, picks
// each token's pair and gates, writes them to global memory and to LDS, and
// sorts the slots from the LDS copy.  (In one workgroup the 16 waves' router
// loads, 64-byte pieces of 16 rows, all pass through one CU's vector memory
// path: 13.7 us at T = 32 against 10 us for the two launches, with the same
// bits: the partial of a slice is the same MFMA chain, and the slices are
// added in the same order.)
template <int kGroups>
__global__ void __launch_bounds__(kWave) route_slices_kernel(const bf16_t* __restrict__ x,
                                                             const bf16_t* __restrict__ wg, int32_t T_tokens, int d,
                                                             f32x4* __restrict__ part) {
  const int lane = threadIdx.x, slice = blockIdx.x;
  const int l16 = lane % 16, lg = lane / 16;
  const int groups = (T_tokens + 15) / 16;
  const int ks = d / static_cast<int>(gridDim.x);  // a multiple of 32 (see router_slices)
  const bool real_row = l16 < kExperts;            // rows 8..15 of the padded router are zero
  const bf16_t* wp = wg + static_cast<int64_t>(real_row ? l16 : 0) * d + slice * ks + lg * 8;
  const bf16_t* xp[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g)  // clamped rows are computed, never written
    xp[g] = x + static_cast<int64_t>(min(g * 16 + l16, T_tokens - 1)) * d + slice * ks + lg * 8;
  f32x4 acc[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  // k-steps in batches of 8 whose loads are all issued before their MFMAs
  // (a single-wave workgroup has the registers), then one step at a time
  constexpr int kBatch = 8;
  int k0 = 0;
  for (; k0 + kBatch * 32 <= ks; k0 += kBatch * 32) {
    bf16x8 wa[kBatch], xa[kBatch][kGroups];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      wa[j] = real_row ? *reinterpret_cast<const bf16x8*>(wp + k0 + 32 * j) : zero;  // rows 8..15: no load
#pragma unroll
      for (int g = 0; g < kGroups; ++g) xa[j][g] = *reinterpret_cast<const bf16x8*>(xp[g] + k0 + 32 * j);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        if (g < groups) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[j], xa[j][g], acc[g], 0, 0, 0);
  }
  for (; k0 < ks; k0 += 32) {
    const bf16x8 wa = real_row ? *reinterpret_cast<const bf16x8*>(wp + k0) : zero;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (g < groups) {
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(xp[g] + k0);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xa, acc[g], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
    if (g < groups) part[(slice * kGroups + g) * kWave + lane] = acc[g];
}

template <int kGroups>
__global__ void __launch_bounds__(kPermThreads) route_finish_kernel(
    const f32x4* __restrict__ part, int slices, const float* __restrict__ bias, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t T_tokens, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ slot_rows, int32_t* __restrict__ counts_out, int gating, int capacity) {
  __shared__ int32_t idx_s[kGroups * 16 * kTopK];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int groups = (T_tokens + 15) / 16;
  if (wave < groups) {
    // acc[q] of lane t (< 16): expert q of token group*16 + t; lane t+16: expert 4+q
    const int g = wave;
    // every slice's partial loaded before the first add (one memory
    // latency), then added in slice order
    f32x4 v[kRouteSlices];
#pragma unroll
    for (int sl = 0; sl < kRouteSlices; ++sl)
      v[sl] = sl < slices ? part[(sl * kGroups + g) * kWave + lane] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 sum = v[0];
#pragma unroll
    for (int sl = 1; sl < kRouteSlices; ++sl) {
      if (sl < slices) {
        sum[0] += v[sl][0]; sum[1] += v[sl][1]; sum[2] += v[sl][2]; sum[3] += v[sl][3];
      }
    }
    float sc[kExperts];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sc[q] = sum[q];
      sc[4 + q] = __shfl(sum[q], (lane % 16) + 16, kWave);
    }
    const int t = g * 16 + lane;
    if (lane < 16 && t < T_tokens) {
#pragma unroll
      for (int e = 0; e < kExperts; ++e) sc[e] += bias ? bias[e] : 0.0f;
      int32_t pair[kTopK];
      float gate[kTopK];
      select_top2(sc, gating, pair, gate);
      idx_out[kTopK * t] = pair[0];
      idx_out[kTopK * t + 1] = pair[1];
      w_out[kTopK * t] = gate[0];
      w_out[kTopK * t + 1] = gate[1];
      idx_s[kTopK * t] = pair[0];
      idx_s[kTopK * t + 1] = pair[1];
    }
  }
  __syncthreads();
  permute_block(idx_s, T_tokens * kTopK, offsets, sorted_slots, slot_rows, counts_out, capacity);
}

}  // namespace moe

namespace moe {

namespace {
template <int kGroups>
hipError_t launch_route_split(const bf16_t* x, const bf16_t* wg, const float* bias, int32_t* idx, float* w, int32_t T,
                              int d, int gating, int capacity, int32_t* offsets, int32_t* sorted_slots,
                              int32_t* slot_rows, int32_t* counts_out, float* partials, hipStream_t s) {
  const int slices = router_slices(d, kRouteSlices);
  f32x4* part = reinterpret_cast<f32x4*>(partials);
  hipLaunchKernelGGL(route_slices_kernel<kGroups>, dim3(slices), dim3(kWave), 0, s, x, wg, T, d, part);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_finish_kernel<kGroups>, dim3(1), dim3(kPermThreads), 0, s, part, slices, bias, idx, w, T,
                     offsets, sorted_slots, slot_rows, counts_out, gating, capacity);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_route_permute(int dtype, const void* x, const void* wg, const float* bias, int32_t* idx, float* w,
                                int32_t T, int d, int gating, int capacity, int32_t* offsets, int32_t* sorted_slots,
                                int32_t* slot_rows, int32_t* counts_out, float* partials, hipStream_t s) {
  if (dtype == kDtypeBF16) {
    if (T > kRouteSplitMaxTokens || !partials) return hipErrorInvalidValue;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(wg);
    if (T <= 32)
      return launch_route_split<2>(xb, wb, bias, idx, w, T, d, gating, capacity, offsets, sorted_slots, slot_rows,
                                   counts_out, partials, s);
    return launch_route_split<4>(xb, wb, bias, idx, w, T, d, gating, capacity, offsets, sorted_slots, slot_rows,
                                 counts_out, partials, s);
  }
  const size_t lds = kExperts * static_cast<size_t>(d) * (dtype == kDtypeBF16 ? 2 : 4);
  const void* fn = dtype == kDtypeBF16 ? reinterpret_cast<const void*>(&route_permute_kernel<bf16_t>)
                                       : reinterpret_cast<const void*>(&route_permute_kernel<float>);
  if (lds > 64 * 1024) {
    const hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
  }
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(route_permute_kernel<bf16_t>, dim3(1), dim3(kPermThreads), lds, s,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(wg), bias, idx, w, T, d, offsets,
                       sorted_slots, slot_rows, counts_out, gating, capacity);
  else
    hipLaunchKernelGGL(route_permute_kernel<float>, dim3(1), dim3(kPermThreads), lds, s,
                       static_cast<const float*>(x), static_cast<const float*>(wg), bias, idx, w, T, d, offsets,
                       sorted_slots, slot_rows, counts_out, gating, capacity);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Load-balancing loss E * sum_e f_e * P_e (f_e: fraction of the T*k slots
// routed to e; P_e: mean over tokens of the softmax over all E scores at e),
// the reading of the auxiliary losses of "Mixtral & Sparse MoE (2024) > The
// Solution" (load-balancing paragraph).  One workgroup: thread i takes tokens
// i, i + 1024, ...; the per-thread sums are added over the lanes of a wave
// (butterfly) and then over the waves in wave order, so the result is
// deterministic.
__global__ void __launch_bounds__(kPermThreads) load_balance_loss_kernel(const float* __restrict__ logits,
                                                                          const int32_t* __restrict__ idx,
                                                                          int64_t T, float* __restrict__ loss) {
  __shared__ float wsum[kPermWaves][2 * kExperts];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  float p[kExperts], n[kExperts];
#pragma unroll
  for (int e = 0; e < kExperts; ++e) p[e] = n[e] = 0.0f;
  for (int64_t t = tid; t < T; t += kPermThreads) {
    float l[kExperts];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kExperts; ++e) {
      l[e] = logits[t * kExperts + e];
      mx = fmaxf(mx, l[e]);
    }
    float z = 0.0f;
#pragma unroll
    for (int e = 0; e < kExperts; ++e) {
      l[e] = expf(l[e] - mx);
      z += l[e];
    }
    const float rz = 1.0f / z;
#pragma unroll
    for (int e = 0; e < kExperts; ++e) p[e] += l[e] * rz;
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const int e = idx[t * kTopK + j];
#pragma unroll
      for (int ee = 0; ee < kExperts; ++ee) n[ee] += e == ee ? 1.0f : 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    p[e] = wave_sum(p[e]);
    n[e] = wave_sum(n[e]);
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < kExperts; ++e) {
      wsum[wave][e] = p[e];
      wsum[wave][kExperts + e] = n[e];
    }
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.0f;
    for (int e = 0; e < kExperts; ++e) {
      float pe = 0.0f, ne = 0.0f;
      for (int w = 0; w < kPermWaves; ++w) {
        pe += wsum[w][e];
        ne += wsum[w][kExperts + e];
      }
      acc += (ne / static_cast<float>(T * kTopK)) * (pe / static_cast<float>(T));
    }
    loss[0] = T > 0 ? static_cast<float>(kExperts) * acc : 0.0f;
  }
}

hipError_t launch_load_balance_loss(const float* logits, const int32_t* idx, int64_t T, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(load_balance_loss_kernel, dim3(1), dim3(kPermThreads), 0, s, logits, idx, T, loss);
  return hipGetLastError();
}

}  // namespace moe
