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
// parameters).  Each wavefront owns 32 weight rows of one expert (up: 16 gate
// rows and the same 16 up rows; down: two blocks of 16) over its share of the
// reduction and streams them straight from HBM into registers as the MFMA
// src0 operand (16 rows x 32 k per v_mfma_f32_16x16x32_bf16); the expert's
// tokens, padded to groups of 16, are the src1 operand, read from L2 and
// shared by both row blocks.  Weights are never staged in LDS: no element is
// used twice by the same wave.  KU k-steps of weight loads are issued back to
// back to keep bytes in flight.  At most MAXG token groups (16 rows each)
// share one pass over the weights; an expert with more rows takes more
// passes.  Up projection: MAXG = 2 when T <= 32 (no expert can then hold
// more than 32 rows of a top-2 routing); the smaller register footprint
// measured 10% faster than MAXG = 4.  The down
// projection splits the reduction over S waves (S = 2: twice the waves in
// flight) writing separate partial sums; the combine adds them in order.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kDThreads = 256;
constexpr int kDWaves = kDThreads / kWave;

// Up projection: wave = (expert, 16-row block of w1/w3).
template <int KU, int MAXG>
__global__ void __launch_bounds__(kDThreads) up_decode_kernel(const bf16_t* __restrict__ x,
                                                                const int32_t* __restrict__ sorted_slots,
                                                                const int32_t* __restrict__ offs,
                                                                const bf16_t* __restrict__ w1,
                                                                const bf16_t* __restrict__ w3, bf16_t* __restrict__ h,
                                                                int f, int d) {
  const int lane = threadIdx.x % kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const int fgroups = f / 16;
  const int wid = blockIdx.x * kDWaves + threadIdx.x / kWave;
  const int e = wid / fgroups;
  if (e >= kExperts) return;
  const int fg = wid - e * fgroups;
  const int row_begin = offs[e];
  const int rows = offs[e + 1] - row_begin;
  if (rows <= 0) return;

  const int n_row = fg * 16 + l16;  // weight row this lane streams
  const bf16_t* pg = w1 + (static_cast<int64_t>(e) * f + n_row) * d + lg * 8;
  const bf16_t* pu = w3 + (static_cast<int64_t>(e) * f + n_row) * d + lg * 8;

  for (int base = 0; base < rows; base += 16 * MAXG) {
    const int ng = min(MAXG, (rows - base + 15) / 16);
    const bf16_t* a_ptr[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      const int m = min(base + g * 16 + l16, rows - 1);  // clamped rows are computed, never stored
      a_ptr[g] = x + static_cast<int64_t>(sorted_slots[row_begin + m] / kTopK) * d + lg * 8;
    }
    f32x4 acc_g[MAXG], acc_u[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      acc_g[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_u[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < d; k0 += 32 * KU) {
      bf16x8 wg[KU], wu[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        wg[u] = *reinterpret_cast<const bf16x8*>(pg + k0 + u * 32);
        wu[u] = *reinterpret_cast<const bf16x8*>(pu + k0 + u * 32);
      }
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {
        if (g < ng) {
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            const bf16x8 xa = *reinterpret_cast<const bf16x8*>(a_ptr[g] + k0 + u * 32);
            acc_g[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg[u], xa, acc_g[g], 0, 0, 0);
            acc_u[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wu[u], xa, acc_u[g], 0, 0, 0);
          }
        }
      }
    }
    // acc[g][q]: row base + g*16 + l16, feature fg*16 + 4*lg + q.
    const int n = fg * 16 + 4 * lg;
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      const int m = base + g * 16 + l16;
      if (g >= ng || m >= rows) continue;
      const f32x4 a = acc_g[g], b = acc_u[g];
      uint2 p;
      p.x = pack_bf16x2(silu(a[0]) * b[0], silu(a[1]) * b[1]);
      p.y = pack_bf16x2(silu(a[2]) * b[2], silu(a[3]) * b[3]);
      *reinterpret_cast<uint2*>(h + static_cast<int64_t>(row_begin + m) * f + n) = p;
    }
  }
}

// Down projection: wave = (expert, 32-row block of w2, part s of the
// reduction); part s writes y_rows + s * split_stride.
template <int KU, int MAXG, int S>
__global__ void __launch_bounds__(kDThreads) down_decode_kernel(const bf16_t* __restrict__ h,
                                                                  const int32_t* __restrict__ offs,
                                                                  const bf16_t* __restrict__ w2,
                                                                  float* __restrict__ y_rows, int d, int f,
                                                                  int64_t split_stride) {
  const int lane = threadIdx.x % kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const int nrb = d / 32;
  const int wid = blockIdx.x * kDWaves + threadIdx.x / kWave;
  const int e = wid / (nrb * S);
  if (e >= kExperts) return;
  const int rb = (wid / S) % nrb, s = wid % S;
  const int row_begin = offs[e];
  const int rows = offs[e + 1] - row_begin;
  if (rows <= 0) return;
  const int kp = f / S, k_beg = s * kp;

  const bf16_t* p0 = w2 + (static_cast<int64_t>(e) * d + rb * 32 + l16) * f + k_beg + lg * 8;
  const bf16_t* p1 = p0 + static_cast<int64_t>(16) * f;
  float* out = y_rows + s * split_stride;

  for (int base = 0; base < rows; base += 16 * MAXG) {
    const int ng = min(MAXG, (rows - base + 15) / 16);
    const bf16_t* a_ptr[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g)
      a_ptr[g] = h + static_cast<int64_t>(row_begin + min(base + g * 16 + l16, rows - 1)) * f + k_beg + lg * 8;
    f32x4 acc0[MAXG], acc1[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      acc0[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < kp; k0 += 32 * KU) {
      bf16x8 b0[KU], b1[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        b0[u] = *reinterpret_cast<const bf16x8*>(p0 + k0 + u * 32);
        b1[u] = *reinterpret_cast<const bf16x8*>(p1 + k0 + u * 32);
      }
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {
        if (g < ng) {
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            const bf16x8 ha = *reinterpret_cast<const bf16x8*>(a_ptr[g] + k0 + u * 32);
            acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[u], ha, acc0[g], 0, 0, 0);
            acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[u], ha, acc1[g], 0, 0, 0);
          }
        }
      }
    }
    // acc0[g][q]: row base + g*16 + l16, feature rb*32 + 4*lg + q (acc1: + 16).
    const int n = rb * 32 + 4 * lg;
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      const int m = base + g * 16 + l16;
      if (g >= ng || m >= rows) continue;
      float* o = out + static_cast<int64_t>(row_begin + m) * d + n;
      *reinterpret_cast<float4*>(o) = make_float4(acc0[g][0], acc0[g][1], acc0[g][2], acc0[g][3]);
      *reinterpret_cast<float4*>(o + 16) = make_float4(acc1[g][0], acc1[g][1], acc1[g][2], acc1[g][3]);
    }
  }
}

template <int KU, int MAXG>
hipError_t launch_up(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                     const bf16_t* w3, bf16_t* h, int d, int f, hipStream_t s) {
  const int waves = kExperts * (f / 16);
  hipLaunchKernelGGL((up_decode_kernel<KU, MAXG>), dim3((waves + kDWaves - 1) / kDWaves), dim3(kDThreads), 0, s, x,
                     sorted_slots, offs, w1, w3, h, f, d);
  return hipGetLastError();
}

template <int KU, int MAXG, int S>
hipError_t launch_down(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int d, int f,
                       int64_t split_stride, hipStream_t s) {
  const int waves = kExperts * (d / 32) * S;
  hipLaunchKernelGGL((down_decode_kernel<KU, MAXG, S>), dim3((waves + kDWaves - 1) / kDWaves), dim3(kDThreads), 0, s,
                     h, offs, w2, y_rows, d, f, split_stride);
  return hipGetLastError();
}

}  // namespace

// KU = 4 needs the reduction (d, or f / S) to be a multiple of 128: d and f
// are multiples of 128 (checked at the boundary), and S = 2 is used only when
// f is a multiple of 256.
hipError_t launch_up_decode(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                            const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, hipStream_t s) {
  if (T <= 32) return launch_up<4, 2>(x, offs, sorted_slots, w1, w3, h, d, f, s);
  return launch_up<4, 4>(x, offs, sorted_slots, w1, w3, h, d, f, s);
}

hipError_t launch_down_decode(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T, int d,
                              int f, int split, int64_t split_stride, hipStream_t s) {
  // (MAXG = 4 measured faster here than 2, whatever T.)
  (void)T;
  if (split == 2 && f % 256 == 0) return launch_down<4, 4, 2>(h, offs, w2, y_rows, d, f, split_stride, s);
  return launch_down<4, 4, 1>(h, offs, w2, y_rows, d, f, 0, s);
}

}  // namespace moe
