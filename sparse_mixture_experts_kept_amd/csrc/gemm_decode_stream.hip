// bf16 grouped expert GEMMs for decode batches of at most 64 tokens, built to
// stream the routed experts' weights from HBM at close to the memory's rate.
// Same functions as the other expert kernels:
//   up:   h[r, n]      = SiLU(x[tok(r)] . w1_e[n]) * (x[tok(r)] . w3_e[n])   -> bf16
//   down: y_rows[r, n] = h[r] . w2_e[n]                                      -> fp32
// ("Mixtral of Experts", azimuth.plus, architecture paragraph; "Mixtral >
// Architecture Overview", parameter-count paragraph.)
//
// With a handful of rows per expert the layer is a stream over the touched
// experts' weights ("Mixtral of Experts", azimuth.plus, paragraph on active
// versus stored parameters), so the design is about the access pattern:
// - Weights go from HBM straight into LDS (buffer_load ... lds, nontemporal)
//   in runs of 256 contiguous bytes per row: each load instruction moves 4
//   rows x 256 B = 1 KiB.  Measured on MI355X, such loads sustain about
//   6.4-6.7 TB/s where the 64-byte pieces of 16 rows that a register-direct
//   MFMA operand load touches reach about 5.5 TB/s.
// - One wavefront per workgroup, two workgroups per CU, persistent: wave w
//   takes work units w, w + G, ... (G workgroups) and streams them as one
//   continuous sequence of stages, S stages in flight in a private LDS ring
//   (no workgroup barrier anywhere; each wave reads only what it loaded).
// - A stage is 128 reduction elements: for the up projection 16 rows of w1
//   and the same 16 rows of w3, for the down projection 32 rows of w2, plus
//   the unit's token rows (MAXG groups of 16, 256 B each, loaded the same
//   way; the up projection gathers x rows through the permutation).  Every
//   stage issues the same number of loads, so "this stage has landed" is
//   one s_waitcnt vmcnt with a constant.
// - LDS rows are 256 B with the 16-byte chunk index XOR the row (mod 16), set
//   by which chunk each lane loads; the MFMA fragment reads (16 rows x one
//   chunk) then touch 16 distinct bank groups.
// - MFMA v_mfma_f32_16x16x32_bf16: weights as src0 (16 rows = output
//   features), tokens as src1, fp32 accumulators; SwiGLU or the fp32 store at
//   the end of each unit.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRowBytes = 256;                 // bytes of a row per stage
constexpr int kStageK = kRowBytes / 2;         // reduction elements per stage
constexpr int kBlockElems = 16 * kStageK;      // one 16-row block of a stage (4 KiB)
constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per LDS row
constexpr int kBufferFlags = 0x00020000;       // word 3 of a raw buffer resource on gfx9
constexpr int kNontemporal = 2;                // cache-policy bits of the weight loads

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate: at most n vector-memory ops outstanding (vmcnt in bits
// 3:0 and 15:14), expcnt and lgkmcnt not waited on.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// ... and lgkmcnt(0) alone.
constexpr int lgkm0_imm() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Work unit u of the non-empty experts (each has `per_expert` units) -> expert, index within it.
__device__ __forceinline__ void unit_of(const int* o, int per_expert, int u, int* e_out, int* r_out) {
  int pre = 0, e_sel = 0, pre_sel = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    const int n = o[e + 1] > o[e] ? per_expert : 0;
    if (u >= pre && u < pre + n) {
      e_sel = e;
      pre_sel = pre;
    }
    pre += n;
  }
  *e_out = e_sel;
  *r_out = u - pre_sel;
}

// UP: units (expert, 16 rows of w1 and w3), act = x, out = h (bf16).
// DOWN: units (expert, 32 rows of w2), act = h, out = y_rows (fp32).
template <bool UP, int MAXG, int S>
__global__ void __launch_bounds__(kWave) decode_stream_kernel(const bf16_t* __restrict__ act,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const int32_t* __restrict__ offs,
                                                              const bf16_t* __restrict__ wa,
                                                              const bf16_t* __restrict__ wb, void* __restrict__ out,
                                                              int d, int f, int n_slots) {
  constexpr int kStageElems = (2 + MAXG) * kBlockElems;
  constexpr int kLoads = 8 + 4 * MAXG;  // load instructions per stage
  __shared__ __align__(16) bf16_t ring[S][kStageElems];

  const int lane = threadIdx.x;
  const int l16 = lane % 16, lg = lane / 16;
  const int K = UP ? d : f;                      // reduction length
  const int per_expert = UP ? f / 16 : d / 32;   // units per expert
  const int KS = K / kStageK;                    // stages per unit (>= 1)
  int o[kExperts + 1];
#pragma unroll
  for (int e = 0; e <= kExperts; ++e) o[e] = offs[e];
  int n_units = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) n_units += o[e + 1] > o[e] ? per_expert : 0;
  const int G = gridDim.x;
  if (static_cast<int>(blockIdx.x) >= n_units) return;
  const int total = (n_units - static_cast<int>(blockIdx.x) + G - 1) / G * KS;

  // Weight loads: instruction i of a 16-row block puts rows 4i..4i+3 (row
  // 4i + lg for this lane) into 1 KiB of LDS, this lane's 16 bytes at
  // physical chunk l16, i.e. logical chunk l16 ^ row.
  uint32_t w_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * i + lg;
    w_off[i] = static_cast<uint32_t>(rr * K * 2 + ((l16 ^ rr) * 16));
  }

  // Issue side: unit, stage within it, buffer resources and token offsets.
  int iu = blockIdx.x, iks = 0;
  __amdgpu_buffer_rsrc_t ra, rb;
  // (A fixed extent: an array sized by the template parameter, passed to
  // the buffer-load builtin, keeps clang from emitting the launch stub.)
  static_assert(MAXG <= 4, "at most 64 rows per expert");
  uint32_t t_off[4][4];
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(act), 0, 0x7FFFFFFF, kBufferFlags);
#define SET_ISSUE_UNIT(U_)                                                                                   \
  {                                                                                                        \
    int e_, r_;                                                                                            \
    unit_of(o, per_expert, (U_), &e_, &r_);                                                                \
    const int row_begin = o[e_], rows = o[e_ + 1] - o[e_];                                                 \
    const bf16_t* a0;                                                                                      \
    const bf16_t* b0;                                                                                      \
    if constexpr (UP) {                                                                                    \
      a0 = wa + (static_cast<int64_t>(e_) * f + r_ * 16) * d;                                              \
      b0 = wb + (static_cast<int64_t>(e_) * f + r_ * 16) * d;                                              \
    } else {                                                                                               \
      a0 = wa + (static_cast<int64_t>(e_) * d + r_ * 32) * f;                                              \
      b0 = a0 + static_cast<int64_t>(16) * f;                                                              \
    }                                                                                                      \
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a0), 0, 0x7FFFFFFF, kBufferFlags);          \
    rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(b0), 0, 0x7FFFFFFF, kBufferFlags);          \
    _Pragma("unroll") for (int g = 0; g < MAXG; ++g) _Pragma("unroll") for (int q = 0; q < 4; ++q) {       \
      const int rr = 4 * q + lg; /* row within the 16-row group; clamped rows are loaded, never stored */  \
      int tok;                                                                                             \
      if constexpr (UP) {                                                                                  \
        /* slot ids through the scalar cache (uniform addresses, lgkmcnt): a vector load here would be     \
           ordered behind the weight loads in flight, and waiting for it would drain them; the select is   \
           arithmetic so that all four loads stay unconditional */                                         \
        const int b = 16 * g + 4 * q;                                                                      \
        const int s0 = sorted_slots[row_begin + min(b, rows - 1)];                                         \
        const int s1 = sorted_slots[row_begin + min(b + 1, rows - 1)];                                     \
        const int s2 = sorted_slots[row_begin + min(b + 2, rows - 1)];                                     \
        const int s3 = sorted_slots[row_begin + min(b + 3, rows - 1)];                                     \
        tok = (s0 + (lg >= 1) * (s1 - s0) + (lg >= 2) * (s2 - s1) + (lg >= 3) * (s3 - s2)) / kTopK;         \
      } else {                                                                                             \
        tok = row_begin + min(16 * g + rr, rows - 1);                                                      \
      }                                                                                                    \
      t_off[g][q] = static_cast<uint32_t>(tok) * static_cast<uint32_t>(K * 2) +                           \
                    static_cast<uint32_t>((l16 ^ rr) * 16);                                                \
    }                                                                                                      \
  }
#define ISSUE(SLOT_)                                                                                       \
  {                                                                                                        \
    bf16_t* st_ = ring[SLOT_];                                                                             \
    const int so = iks * kRowBytes;                                                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LDS_PTR(st_ + i * 4 * kStageK), 16, w_off[i], so, 0,    \
                                               kNontemporal);                                              \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LDS_PTR(st_ + kBlockElems + i * 4 * kStageK), 16,       \
                                               w_off[i], so, 0, kNontemporal);                             \
    _Pragma("unroll") for (int g = 0; g < MAXG; ++g) _Pragma("unroll") for (int q = 0; q < 4; ++q)         \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, LDS_PTR(st_ + (2 + g) * kBlockElems + q * 4 * kStageK), \
                                               16, t_off[g][q], so, 0, 0);                                 \
    if (++iks == KS) {                                                                                     \
      iks = 0;                                                                                             \
      iu += G;                                                                                             \
      if (iu < n_units) SET_ISSUE_UNIT(iu);                                                                \
    }                                                                                                      \
  }

  SET_ISSUE_UNIT(iu);
  int islot = 0;
  for (int j = 0; j < S - 1 && j < total; ++j) {
    ISSUE(islot);
    islot = islot == S - 1 ? 0 : islot + 1;
  }

  // Compute side.
  int cu = blockIdx.x, cks = 0, cslot = 0;
  int ce, cr;
  unit_of(o, per_expert, cu, &ce, &cr);
  int c_begin = o[ce], c_rows = o[ce + 1] - o[ce];
  f32x4 acc0[MAXG], acc1[MAXG];
#pragma unroll
  for (int g = 0; g < MAXG; ++g) {
    acc0[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int j = 0; j < total; ++j) {
    if (j + S - 1 < total) {
      // the slot being refilled was read by the previous stage's MFMAs
      __builtin_amdgcn_s_waitcnt(lgkm0_imm());
      ISSUE(islot);
      islot = islot == S - 1 ? 0 : islot + 1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * kLoads));  // stage j has landed
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    asm volatile("" ::: "memory");
    const bf16_t* st = ring[cslot];
#pragma unroll
    for (int s = 0; s < kStageK / 32; ++s) {
      const int off = l16 * kStageK + (((4 * s + lg) ^ l16) & (kChunks - 1)) * 8;
      const bf16x8 fa = *reinterpret_cast<const bf16x8*>(st + off);
      const bf16x8 fb = *reinterpret_cast<const bf16x8*>(st + kBlockElems + off);
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {  // all groups: MFMA time is free here, a branch is not
        const bf16x8 t = *reinterpret_cast<const bf16x8*>(st + (2 + g) * kBlockElems + off);
        acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, t, acc0[g], 0, 0, 0);
        acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, t, acc1[g], 0, 0, 0);
      }
    }
    cslot = cslot == S - 1 ? 0 : cslot + 1;
    if (++cks == KS) {
      // acc[g][q]: unit row 16g + l16, output feature 4*lg + q of the block
      // (down: acc0 rows 0-15 of the unit, acc1 rows 16-31).
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {
        const int m = 16 * g + l16;
        if (m >= c_rows) continue;
        const int64_t orow = c_begin + m;
        if constexpr (UP) {
          const f32x4 a = acc0[g], b = acc1[g];
          uint2 p;
          p.x = pack_bf16x2(silu(a[0]) * b[0], silu(a[1]) * b[1]);
          p.y = pack_bf16x2(silu(a[2]) * b[2], silu(a[3]) * b[3]);
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(out) + orow * f + cr * 16 + 4 * lg) = p;
        } else {
          float* y = static_cast<float*>(out) + orow * d + cr * 32 + 4 * lg;
          *reinterpret_cast<float4*>(y) = make_float4(acc0[g][0], acc0[g][1], acc0[g][2], acc0[g][3]);
          *reinterpret_cast<float4*>(y + 16) = make_float4(acc1[g][0], acc1[g][1], acc1[g][2], acc1[g][3]);
        }
      }
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {
        acc0[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      cks = 0;
      cu += G;
      if (cu < n_units) {
        unit_of(o, per_expert, cu, &ce, &cr);
        c_begin = o[ce];
        c_rows = o[ce + 1] - o[ce];
      }
    }
  }
}

#undef SET_ISSUE_UNIT
#undef ISSUE
#undef LDS_PTR

template <bool UP, int MAXG, int S>
hipError_t launch_stream(const bf16_t* act, const int32_t* sorted_slots, const int32_t* offs, const bf16_t* wa,
                         const bf16_t* wb, void* out, int d, int f, int n_slots, int n_cu, hipStream_t s) {
  hipLaunchKernelGGL((decode_stream_kernel<UP, MAXG, S>), dim3(2 * n_cu), dim3(kWave), 0, s, act, sorted_slots, offs,
                     wa, wb, out, d, f, n_slots);
  return hipGetLastError();
}

}  // namespace

// Rows per expert are at most T (top-2 picks two different experts), so
// MAXG = ceil(T / 16) groups of 16 hold them all: 2 for T <= 32 (4 stages
// in flight, 64 KiB of LDS), 4 for T <= 64 (3 stages, 72 KiB).
hipError_t launch_up_decode_stream(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots,
                                   const bf16_t* w1, const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, int n_cu,
                                   hipStream_t s) {
  if (T > 64) return hipErrorInvalidValue;
  const int n_slots = static_cast<int>(T) * kTopK;
  if (T <= 32) return launch_stream<true, 2, 4>(x, sorted_slots, offs, w1, w3, h, d, f, n_slots, n_cu, s);
  return launch_stream<true, 4, 3>(x, sorted_slots, offs, w1, w3, h, d, f, n_slots, n_cu, s);
}

hipError_t launch_down_decode_stream(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T,
                                     int d, int f, int n_cu, hipStream_t s) {
  if (T > 64) return hipErrorInvalidValue;
  const int n_slots = static_cast<int>(T) * kTopK;
  if (T <= 32) return launch_stream<false, 2, 4>(h, nullptr, offs, w2, nullptr, y_rows, d, f, n_slots, n_cu, s);
  return launch_stream<false, 4, 3>(h, nullptr, offs, w2, nullptr, y_rows, d, f, n_slots, n_cu, s);
}

}  // namespace moe
