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
// Design (gfx950): persistent workgroups of 512 threads (8 waves, two per
// SIMD so one wave's LDS reads, loads and barrier waits hide under the other
// wave's MFMAs), 256 x 256 block tiles stepped 32 deep in k, each wave a
// 128 x 64 sub-tile built from v_mfma_f32_16x16x32_bf16 with fp32
// accumulators.  A and B tiles live in a 4-deep LDS ring (4 x 32 KiB) filled
// by direct global->LDS loads (global_load_lds_dwordx4, no staging
// registers) up to four k-steps ahead.  The two waves of each SIMD run a
// ping-pong schedule: one issues its MFMAs while the other refills the ring
// and reads its next fragments, swapping at every barrier.  Waits are
// explicit (s_waitcnt vmcnt(N) / lgkmcnt(0) before raw barriers), so the
// compiler adds none that would serialise the ring.  LDS rows are 64 B with the 16-byte chunk index XOR-swizzled by
// bits 1..2 of the row; of the layouts measured with the LDS bank-conflict
// counter for the ds_read_b128 fragment pattern (16 rows x 4 chunks), this
// one has no conflicts while chunk ^ (row >> 2) and the unswizzled layout
// are 2-way conflicted.  For
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
constexpr int kStages = 4;     // LDS ring depth (4 x 32 KiB)
static_assert(kStages >= 4 && kStages <= 5, "the tail waits below cover rings of 4 or 5 slots");
constexpr int kPThreads = 512;  // 8 waves: two per SIMD
constexpr int kXcds = 8;
constexpr int kGroupN = 8;
// Per wave and stage: 2 A loads + 2 B loads of 1 KiB (16 rows x 64 B).
constexpr int kLoadsPerStage = 4;

#define GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima so they are not waited on).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// The same immediate with lgkmcnt forced to 0 (also wait for LDS reads).
constexpr int lgkm0_mask() { return ~(0xF << 8); }
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

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
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kPBK + ((chunk ^ ((row >> 1) & 3)) << 3); }

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

// SPLITK > 1 (down projection only): each tile's reduction is cut into
// SPLITK equal parts run as separate work units; part s writes its partial
// sums to Cout + s * split_stride (a separate buffer per part; the consumer
// adds them in a fixed order).
template <bool SWIGLU, int SPLITK>
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
grouped_gemm_prefill_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ gather, int k_div,
                            const int32_t* __restrict__ offs, const bf16_t* __restrict__ B0,
                            const bf16_t* __restrict__ B1, void* __restrict__ Cout, int N, int K,
                            int64_t split_stride) {
  static_assert(!SWIGLU || SPLITK == 1, "the SwiGLU epilogue needs the full reduction");
  // One LDS object holds the whole ring: [stage][A tile | B tile].
  __shared__ __align__(16) bf16_t ring[kStages][(kPBM + kPBN) * kPBK];

  // Output columns per tile: 128 (SwiGLU: 128 gate + 128 up B rows) or 256.
  constexpr int TN = SWIGLU ? kPBN / 2 : kPBN;
  const int n_tiles_n = (N + TN - 1) / TN;

  int total = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) total += (offs[e + 1] - offs[e] + kPBM - 1) / kPBM;
  total *= n_tiles_n * SPLITK;

  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int beg = xcd * per;
  const int end = min(beg + per, total);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  // 8 waves as 2 (rows) x 4 (columns); each owns a 128 x 64 output block.
  const int wm = wave / 4, wn = wave % 4;
  const int l16 = lane % 16, lg = lane / 16;
  // Direct-to-LDS loads: one global_load_lds_dwordx4 writes 64 lanes x 16 B =
  // 16 rows of 64 B.  Wave w fills A and B rows w*32 + j*16 + lane/4
  // (j = 0, 1); the lane's physical chunk is lane%4, so it fetches the
  // logical chunk that the swizzle stores there.
  const int ld_sub = lane / 4;
  const int ld_pchunk = lane % 4;

  const int k_part = K / SPLITK;  // reduction length of one work unit
  for (int L = beg + slot; L < end; L += slots) {
    int e, mt, nt;
    const int ks = L % SPLITK;
    decode_tile(offs, L / SPLITK, n_tiles_n, &e, &mt, &nt);
    const int row_begin = offs[e];
    const int rows = offs[e + 1] - row_begin;
    const int m0 = mt * kPBM;
    const int n0 = nt * TN;

    const bf16_t* a_ptr[2];
    const bf16_t* b_ptr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wave * 32 + j * 16 + ld_sub;
      const int lchunk = ld_pchunk ^ ((r >> 1) & 3);
      const int ar = min(m0 + r, rows - 1);  // clamped rows are computed, never stored
      const int64_t g = row_begin + ar;
      const int64_t arow = gather ? static_cast<int64_t>(gather[g] / k_div) : g;
      a_ptr[j] = A + arow * K + ks * k_part + lchunk * 8;
      if constexpr (SWIGLU) {
        const bf16_t* base = (r < TN) ? B0 : B1;
        const int br = min(n0 + (r % TN), N - 1);
        b_ptr[j] = base + (static_cast<int64_t>(e) * N + br) * K + ks * k_part + lchunk * 8;
      } else {
        const int br = min(n0 + r, N - 1);
        b_ptr[j] = B0 + (static_cast<int64_t>(e) * N + br) * K + ks * k_part + lchunk * 8;
      }
    }

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = k_part / kPBK;  // >= kStages (the host guarantees it)
    auto issue = [&](int kt) {
      const int buf = kt % kStages;
      const int koff = kt * kPBK;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r0 = wave * 32 + j * 16;
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(a_ptr[j] + koff), LDS_PTR(&ring[buf][r0 * kPBK]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(b_ptr[j] + koff), LDS_PTR(&ring[buf][(kPBM + r0) * kPBK]), 16, 0,
                                         0);
      }
    };
    // B rows of this wave's 4 weight fragments: SwiGLU = 2 gate + the same 2 up.
    int b_row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (SWIGLU)
        b_row[j] = (j < 2 ? 0 : TN) + wn * 32 + (j % 2) * 16 + l16;
      else
        b_row[j] = wn * 64 + j * 16 + l16;
    }

    // Fragment registers of the current k-step.
    bf16x8 fa[8], fb[4];
    auto read_frags = [&](int kt) {
      const bf16_t* as_ = ring[kt % kStages];
      const bf16_t* bs_ = as_ + kPBM * kPBK;
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(&bs_[lds_off(b_row[j], lg)]);
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(&as_[lds_off(wm * 128 + i * 16 + l16, lg)]);
    };

    // Ping-pong: waves 0-3 (one per SIMD) and waves 4-7 (the other wave of
    // each SIMD) alternate between a compute phase (32 MFMAs from registers)
    // and a memory phase (refill a ring slot, read the next fragments, wait),
    // swapping at every barrier, so each SIMD's matrix pipe always has one
    // wave feeding it.  Waves 4-7 start one phase late.
    //   compute(k): MFMAs of step k.
    //   memory(k):  refill slot k%4 with stage k+4, read step k+1's fragments,
    //               wait for this wave's loads of stage k+2 and for the reads.
    // Every wave waits for its own loads of stage k+1 before the barrier that
    // opens the first memory(k) (end of memory(k-1)), and for its reads of
    // step k before the barrier that opens the first refill of slot k, so
    // LDS data is complete when read and slots are free when refilled.
    // KT = K/32 is a multiple of 4 (K is a multiple of 128) and >= 8.
    const bool late = wave >= 4;
#pragma unroll
    for (int st = 0; st < kStages; ++st) issue(st);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 1) * kLoadsPerStage));
    lds_barrier();
    read_frags(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kLoadsPerStage) & lgkm0_mask());
    if (late) lds_barrier();
    for (int kt = 0; kt < KT; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      // memory(kt): stages issued so far reach min(kt + kStages, KT) - 1; wait
      // for stage kt+2, i.e. allow the ones after it to stay in flight.
      if (kt + kStages < KT) {
        issue(kt + kStages);
        read_frags(kt + 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kLoadsPerStage) & lgkm0_mask());
      } else if (kt + 1 < KT) {
        read_frags(kt + 1);
        const int after = KT - 3 - kt;  // stages issued after kt+2 (< kStages - 2 here)
        if (after >= 2)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerStage) & lgkm0_mask());
        else if (after == 1)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerStage) & lgkm0_mask());
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lgkm0_mask());
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
    }
    if (!late) lds_barrier();
    // Every wave is done with the ring before the next tile refills it.
    __syncthreads();

    // Epilogue.  acc[i][j][q] is output row m = wm*128 + i*16 + l16 and
    // column wave_col(j) + 4*lg + q (B rows were MFMA src0).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // one 16-row block at a time keeps the accumulators in place until used
      __builtin_amdgcn_sched_barrier(0);
      const int m = m0 + wm * 128 + i * 16 + l16;
      if (m >= rows) continue;
      const int64_t orow = row_begin + m;
      if constexpr (SWIGLU) {
        bf16_t* C = static_cast<bf16_t*>(Cout);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 32 + j * 16 + 4 * lg;
          if (n >= N) continue;
          const f32x4 g = acc[i][j];
          const f32x4 u = acc[i][j + 2];
          uint2 p;
          p.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
          p.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
          *reinterpret_cast<uint2*>(C + orow * N + n) = p;
        }
      } else {
        float* C = static_cast<float*>(Cout) + ks * split_stride;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + 4 * lg;
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
  hipLaunchKernelGGL((grouped_gemm_prefill_kernel<true, 1>), dim3(grid), dim3(kPThreads), 0, s, x, sorted_slots, kTopK,
                     offs, w1, w3, static_cast<void*>(h), f, d, int64_t{0});
  return hipGetLastError();
}

hipError_t launch_down_prefill(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int d, int f,
                               int n_cu, int split, int64_t split_stride, hipStream_t s) {
  const int grid = (n_cu / kXcds) * kXcds;
  // each work unit needs K/split to be a multiple of 128 and at least kStages k-steps
  if (split == 2 && f % 256 == 0 && f / 2 >= kStages * kPBK)
    hipLaunchKernelGGL((grouped_gemm_prefill_kernel<false, 2>), dim3(grid), dim3(kPThreads), 0, s, h,
                       static_cast<const int32_t*>(nullptr), 1, offs, w2, static_cast<const bf16_t*>(nullptr),
                       static_cast<void*>(y_rows), d, f, split_stride);
  else
    hipLaunchKernelGGL((grouped_gemm_prefill_kernel<false, 1>), dim3(grid), dim3(kPThreads), 0, s, h,
                       static_cast<const int32_t*>(nullptr), 1, offs, w2, static_cast<const bf16_t*>(nullptr),
                       static_cast<void*>(y_rows), d, f, int64_t{0});
  return hipGetLastError();
}

}  // namespace moe
