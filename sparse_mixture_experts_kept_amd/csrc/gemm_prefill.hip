// bf16 grouped expert GEMMs for prefill-sized batches, on gfx950 MFMA.
//
// Up projection with the SwiGLU fused into the epilogue, and the down
// projection ("Mixtral of Experts", azimuth.plus, architecture paragraph:
// SwiGLU experts; "Mixtral > Architecture Overview", parameter-count
// paragraph: gate w1, up w3 and down w2 projections):
//   up:   h[r, n]      = SiLU(x[tok(r)] . w1_e[n]) * (x[tok(r)] . w3_e[n])   -> bf16
//   down: y_rows[r, n] = h[r] . w2_e[n]                                      -> fp32
// for the rows r = offsets[e] .. offsets[e+1]-1 of expert e (tok(r) =
// sorted_slots[r] / k, the gather fused into the A-tile load).
//
// Design (gfx950): persistent workgroups of 256 threads (4 waves, one per
// SIMD), 256 x 256 x 64 block tiles, each wave a 128 x 128 sub-tile built
// from v_mfma_f32_16x16x32_bf16 with fp32 accumulators.  A and B tiles are
// double-buffered in LDS (2 x 64 KiB) and filled one k-step ahead with
// direct global->LDS loads (global_load_lds_dwordx4), so no registers are
// spent on staging.  LDS rows are 128 B with the 16-byte chunk index
// XOR-swizzled by the row so the fragment reads spread over all banks.  For
// the up projection the 256 B rows of a tile are 128 gate rows and the same
// 128 up rows, so every wave holds matching gate/up accumulators and applies
// SiLU(g)*u in registers before one bf16 rounding.
//
// Tile order: the tiles of one expert are walked in groups of 8 n-tiles x all
// its m-tiles, so the 32 workgroups running together on one XCD share weight
// panels (one per n-tile) and token panels (one per m-tile) in that XCD's L2.
// Workgroup b runs on XCD b % 8 (round-robin dispatch); each XCD owns one
// contiguous eighth of the tile list.  The host never learns the per-expert
// counts: every workgroup reads the offsets on the device.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPBM = 256;
constexpr int kPBN = 256;
constexpr int kPBK = 64;
constexpr int kPThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupN = 8;

#define GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Element offset of (row, 16-byte chunk) inside a [rows][64] bf16 LDS tile.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kPBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

// (expert, m-tile, n-tile) of logical tile L; returns false past the end.
__device__ __forceinline__ bool decode_tile(const int32_t* offs, int L, int n_tiles_n, int* e_out, int* mt_out,
                                            int* nt_out) {
  int acc = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    const int cnt = offs[e + 1] - offs[e];
    const int mts = (cnt + kPBM - 1) / kPBM;
    const int tiles = mts * n_tiles_n;
    if (L < acc + tiles) {
      const int local = L - acc;
      const int group = mts * kGroupN;
      const int ng = local / group;
      const int rem = local - ng * group;
      const int gw = min(kGroupN, n_tiles_n - ng * kGroupN);
      *e_out = e;
      *mt_out = rem / gw;
      *nt_out = ng * kGroupN + rem % gw;
      return true;
    }
    acc += tiles;
  }
  return false;
}

template <bool SWIGLU>
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
grouped_gemm_prefill_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ gather, int k_div,
                            const int32_t* __restrict__ offs, const bf16_t* __restrict__ B0,
                            const bf16_t* __restrict__ B1, void* __restrict__ Cout, int N, int K) {
  __shared__ __align__(16) bf16_t As[2][kPBM * kPBK];
  __shared__ __align__(16) bf16_t Bs[2][kPBN * kPBK];

  // Output columns per tile: 128 (SwiGLU: 128 gate + 128 up B rows) or 256.
  constexpr int TN = SWIGLU ? kPBN / 2 : kPBN;
  const int n_tiles_n = (N + TN - 1) / TN;

  int total = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) total += (offs[e + 1] - offs[e] + kPBM - 1) / kPBM;
  total *= n_tiles_n;

  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int beg = xcd * per;
  const int end = min(beg + per, total);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int l16 = lane % 16, lg = lane / 16;
  // Direct-to-LDS loads: one global_load_lds_dwordx4 writes 64 lanes x 16 B =
  // 8 rows of a tile.  Wave w fills rows w*64 + j*8 + lane/8 (j = 0..7); the
  // lane's physical chunk is lane%8, so it fetches the logical chunk that the
  // swizzle maps there.
  const int ld_sub = lane / 8;
  const int ld_pchunk = lane % 8;

  for (int L = beg + slot; L < end; L += slots) {
    int e, mt, nt;
    decode_tile(offs, L, n_tiles_n, &e, &mt, &nt);
    const int row_begin = offs[e];
    const int rows = offs[e + 1] - row_begin;
    const int m0 = mt * kPBM;
    const int n0 = nt * TN;

    const bf16_t* a_ptr[8];
    const bf16_t* b_ptr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = wave * 64 + j * 8 + ld_sub;
      const int lchunk = ld_pchunk ^ ((r >> 1) & 7);
      const int ar = min(m0 + r, rows - 1);  // clamped rows are computed, never stored
      const int64_t g = row_begin + ar;
      const int64_t arow = gather ? static_cast<int64_t>(gather[g] / k_div) : g;
      a_ptr[j] = A + arow * K + lchunk * 8;
      if constexpr (SWIGLU) {
        const bf16_t* base = (r < TN) ? B0 : B1;
        const int br = min(n0 + (r % TN), N - 1);
        b_ptr[j] = base + (static_cast<int64_t>(e) * N + br) * K + lchunk * 8;
      } else {
        const int br = min(n0 + r, N - 1);
        b_ptr[j] = B0 + (static_cast<int64_t>(e) * N + br) * K + lchunk * 8;
      }
    }

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / kPBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r0 = wave * 64 + j * 8;
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(a_ptr[j]), LDS_PTR(&As[0][r0 * kPBK]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(b_ptr[j]), LDS_PTR(&Bs[0][r0 * kPBK]), 16, 0, 0);
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) {
        const int koff = (kt + 1) * kPBK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r0 = wave * 64 + j * 8;
          __builtin_amdgcn_global_load_lds(GLOBAL_PTR(a_ptr[j] + koff), LDS_PTR(&As[cur ^ 1][r0 * kPBK]), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(GLOBAL_PTR(b_ptr[j] + koff), LDS_PTR(&Bs[cur ^ 1][r0 * kPBK]), 16, 0, 0);
        }
      }
      const bf16_t* as = As[cur];
      const bf16_t* bs = Bs[cur];
#pragma unroll
      for (int kk = 0; kk < kPBK / 32; ++kk) {
        const int chunk = kk * 4 + lg;
        bf16x8 af[8], bfr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(&as[lds_off(wm * 128 + i * 16 + l16, chunk)]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          int br;
          if constexpr (SWIGLU)
            br = (j < 4 ? 0 : TN) + wn * 64 + (j % 4) * 16 + l16;
          else
            br = wn * 128 + j * 16 + l16;
          bfr[j] = *reinterpret_cast<const bf16x8*>(&bs[lds_off(br, chunk)]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      // The barrier waits for this wave's outstanding LDS-DMA loads
      // (vmcnt(0)) and for every wave to finish reading the current buffer.
      __syncthreads();
    }

    // Epilogue.  acc[i][j][q] is output row m = wm*128 + i*16 + l16 and
    // column wave_col(j) + 4*lg + q (B rows were MFMA src0).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + wm * 128 + i * 16 + l16;
      if (m >= rows) continue;
      const int64_t orow = row_begin + m;
      if constexpr (SWIGLU) {
        bf16_t* C = static_cast<bf16_t*>(Cout);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + 4 * lg;
          if (n >= N) continue;
          const f32x4 g = acc[i][j];
          const f32x4 u = acc[i][j + 4];
          uint2 p;
          p.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
          p.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
          *reinterpret_cast<uint2*>(C + orow * N + n) = p;
        }
      } else {
        float* C = static_cast<float*>(Cout);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + wn * 128 + j * 16 + 4 * lg;
          if (n >= N) continue;
          const f32x4 v = acc[i][j];
          *reinterpret_cast<float4*>(C + orow * N + n) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

hipError_t launch_up_prefill(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                             const bf16_t* w3, bf16_t* h, int d, int f, int n_cu, hipStream_t s) {
  const int grid = (n_cu / kXcds) * kXcds;
  hipLaunchKernelGGL(grouped_gemm_prefill_kernel<true>, dim3(grid), dim3(kPThreads), 0, s, x, sorted_slots, kTopK,
                     offs, w1, w3, static_cast<void*>(h), f, d);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int d, int f,
                               int n_cu, hipStream_t s) {
  const int grid = (n_cu / kXcds) * kXcds;
  hipLaunchKernelGGL(grouped_gemm_prefill_kernel<false>, dim3(grid), dim3(kPThreads), 0, s, h,
                     static_cast<const int32_t*>(nullptr), 1, offs, w2, static_cast<const bf16_t*>(nullptr),
                     static_cast<void*>(y_rows), d, f);
  return hipGetLastError();
}

}  // namespace moe
