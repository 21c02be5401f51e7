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
// SIMD), 256 x 256 block tiles stepped 32 deep in k, each wave a 128 x 128
// sub-tile built from v_mfma_f32_16x16x32_bf16 with fp32 accumulators.  A and
// B tiles live in a 4-deep LDS ring (4 x 32 KiB) filled by direct
// global->LDS loads (global_load_lds_dwordx4, no staging registers); three
// k-steps of loads are in flight while the MFMAs consume the fourth, and
// each step waits only for its own loads (s_waitcnt vmcnt(N)) before one
// barrier.  LDS rows are 64 B with the 16-byte chunk index XOR-swizzled by
// the row so that the fragment reads of 16 lanes hit 16 distinct 4-bank
// groups (measured: zero bank conflicts).  For
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
constexpr int kPBK = 32;       // k depth of one pipeline stage
constexpr int kStages = 4;     // LDS ring depth
constexpr int kPThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupN = 8;
// Per wave and stage: 4 A loads + 4 B loads of 1 KiB (16 rows x 64 B).
constexpr int kLoadsPerStage = 8;

#define GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima so they are not waited on).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// The same immediate with lgkmcnt forced to 0 (also wait for LDS reads).
constexpr int lgkm0_mask() { return ~(0xF << 8); }
// Wait for every outstanding LDS read only (vmcnt and expcnt at maximum).
constexpr int kLgkm0Only = 0xF | (0x3 << 14) | (0x7 << 4);

// Workgroup barrier for the LDS ring.  The waits it needs are issued
// explicitly before it; the empty asm keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Element offset of (row, logical 16-byte chunk) in a [rows][32] bf16 tile.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kPBK + ((chunk ^ ((row >> 2) & 3)) << 3); }

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
  // One LDS object holds the whole ring: [stage][A tile | B tile].
  __shared__ __align__(16) bf16_t ring[kStages][(kPBM + kPBN) * kPBK];

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
  // 16 rows of 64 B.  Wave w fills rows w*64 + j*16 + lane/4 (j = 0..3); the
  // lane's physical chunk is lane%4, so it fetches the logical chunk that
  // the swizzle stores there.
  const int ld_sub = lane / 4;
  const int ld_pchunk = lane % 4;

  for (int L = beg + slot; L < end; L += slots) {
    int e, mt, nt;
    decode_tile(offs, L, n_tiles_n, &e, &mt, &nt);
    const int row_begin = offs[e];
    const int rows = offs[e + 1] - row_begin;
    const int m0 = mt * kPBM;
    const int n0 = nt * TN;

    const bf16_t* a_ptr[4];
    const bf16_t* b_ptr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 64 + j * 16 + ld_sub;
      const int lchunk = ld_pchunk ^ ((r >> 2) & 3);
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
    auto issue = [&](int kt) {
      const int buf = kt % kStages;
      const int koff = kt * kPBK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = wave * 64 + j * 16;
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(a_ptr[j] + koff), LDS_PTR(&ring[buf][r0 * kPBK]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(b_ptr[j] + koff), LDS_PTR(&ring[buf][(kPBM + r0) * kPBK]), 16, 0,
                                         0);
      }
    };
    // MFMA operands: the 8 token (A) fragments of the current stage and of the
    // next one, and a sliding pair of weight (B) fragments.
    bf16x8 fa0[8], fa1[8], fb0, fb1;
    int b_row[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (SWIGLU)
        b_row[j] = (j < 4 ? 0 : TN) + wn * 64 + (j % 4) * 16 + l16;
      else
        b_row[j] = wn * 128 + j * 16 + l16;
    }
#define MOE_A_FRAG(KT_, I_) \
  (*reinterpret_cast<const bf16x8*>(&ring[(KT_) % kStages][lds_off(wm * 128 + (I_) * 16 + l16, lg)]))
#define MOE_B_FRAG(KT_, J_) \
  (*reinterpret_cast<const bf16x8*>(&ring[(KT_) % kStages][kPBM * kPBK + lds_off(b_row[J_], lg)]))

// One stage k: 8 groups of 8 MFMAs (A fragments 0..7 times B fragment j).
// Group j first waits for the LDS reads issued by group j-1, then starts the
// reads for group j+1 (B fragment j+1), so each read has a group of MFMAs
// (~128 cycles) to land.  At the midpoint the wave waits for stage k+1's
// loads (WAIT_N = loads allowed to stay in flight) and joins the barrier;
// after it every wave is done with ring slot k-1, which is refilled with
// stage k+3 (ISSUE), and the A fragments of stage k+1 are read two per group
// (NEXT).  The last group reads B fragment 0 of stage k+1.  The flags are
// compile-time constants so the steady-state loop has no branches.
#define MOE_STAGE(K_, FA, FA_NXT, FB_CUR, FB_NXT, ISSUE, WAIT_N, NEXT, BARRIER)                     \
  do {                                                                                              \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                            \
      if (j == 4 && (BARRIER)) {                                                                    \
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT_N) & lgkm0_mask());                               \
        lds_barrier();                                                                              \
        if (ISSUE) issue((K_) + 3);                                                                 \
      } else {                                                                                      \
        __builtin_amdgcn_s_waitcnt(kLgkm0Only);                                                     \
      }                                                                                             \
      if (j < 7) FB_NXT = MOE_B_FRAG((K_), j + 1);                                                  \
      if (j >= 4 && (NEXT)) {                                                                       \
        FA_NXT[2 * (j - 4)] = MOE_A_FRAG((K_) + 1, 2 * (j - 4));                                    \
        FA_NXT[2 * (j - 4) + 1] = MOE_A_FRAG((K_) + 1, 2 * (j - 4) + 1);                            \
      }                                                                                             \
      if (j == 7 && (NEXT)) FB_NXT = MOE_B_FRAG((K_) + 1, 0);                                       \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) acc[i][j] =                                     \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(FB_CUR, FA[i], acc[i][j], 0, 0, 0);               \
      FB_CUR = FB_NXT;                                                                              \
    }                                                                                               \
  } while (0)

    // Prologue: stages 0..2 in flight; stage 0's A fragments and B fragment 0.
    // KT = K/32 is even and >= 4 (K is a multiple of 128).
    issue(0);
    issue(1);
    issue(2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerStage));
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) fa0[i] = MOE_A_FRAG(0, i);
    fb0 = MOE_B_FRAG(0, 0);

    // Steady state, two stages per trip so the A-fragment sets swap roles
    // without copies; the last four stages are peeled below.
    int kt = 0;
    for (; kt + 6 <= KT; kt += 2) {
      MOE_STAGE(kt, fa0, fa1, fb0, fb1, true, kLoadsPerStage, true, true);
      MOE_STAGE(kt + 1, fa1, fa0, fb0, fb1, true, kLoadsPerStage, true, true);
    }
    // kt == KT - 4 here.
    MOE_STAGE(kt, fa0, fa1, fb0, fb1, true, kLoadsPerStage, true, true);
    MOE_STAGE(kt + 1, fa1, fa0, fb0, fb1, false, kLoadsPerStage, true, true);
    MOE_STAGE(kt + 2, fa0, fa1, fb0, fb1, false, 0, true, true);
    MOE_STAGE(kt + 3, fa1, fa0, fb0, fb1, false, 0, false, false);
#undef MOE_STAGE
#undef MOE_B_FRAG
#undef MOE_A_FRAG
    // Every wave is done with the ring before the next tile refills it.
    __syncthreads();

    // Epilogue.  acc[i][j][q] is output row m = wm*128 + i*16 + l16 and
    // column wave_col(j) + 4*lg + q (B rows were MFMA src0).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // one 16-row block at a time keeps the accumulators in AGPRs until used
      __builtin_amdgcn_sched_barrier(0);
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
