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
//   in runs of W = 256 or 512 contiguous bytes per row; each load
//   instruction moves 1 KiB (1024/W rows).  Measured on MI355X, such loads
//   sustain 6.4-6.8 TB/s where the 64-byte pieces of 16 rows that a
//   register-direct MFMA operand load touches reach about 5.5 TB/s.
// - One wavefront per workgroup, two workgroups per CU, persistent: wave w
//   takes work units w, w + G, ... (G workgroups) and streams them as one
//   continuous sequence of stages, S stages in flight in a private LDS ring
//   (no workgroup barrier anywhere; each wave reads only what it loaded).
// - A stage is W/2 reduction elements of each of the unit's weight rows
//   (NB blocks of 16: the up projection's gate rows and the same up rows,
//   or consecutive rows of w2) plus its token rows (groups of 16, loaded the
//   same way; the up projection gathers x rows through the permutation).
//   Every stage issues the same number of loads, so "this stage has landed"
//   is one s_waitcnt vmcnt with a constant, at most 63 loads in flight.
// - LDS rows are W bytes with the 16-byte chunk index XOR the row (mod 16),
//   set by which chunk each lane loads; the MFMA fragment reads (16 rows x
//   one chunk) then touch 16 distinct bank groups.
// - MFMA v_mfma_f32_16x16x32_bf16: weights as src0 (16 rows = output
//   features), tokens as src1, fp32 accumulators; SwiGLU or the fp32 store at
//   the end of each unit.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kBufferFlags = 0x00020000;       // word 3 of a raw buffer resource on gfx9
constexpr int kNontemporal = 2;                // cache-policy bits of the weight loads
constexpr int kTailTile = 256;                 // the prefill GEMM's row tile
constexpr int kTailRows = 32;                  // tails up to this many rows are left to this kernel
static_assert(kTailRows == kTailPartRows, "split tail partials hold every tail row");

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate: at most n vector-memory ops outstanding (vmcnt in bits
// 3:0 and 15:14), expcnt and lgkmcnt not waited on.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// ... and lgkmcnt(0) alone.
constexpr int lgkm0_imm() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Passes over an expert's weights: one per `rows_per_pass` of its rows.
__device__ __forceinline__ int passes_of(int rows, int rows_per_pass) {
  return (rows + rows_per_pass - 1) / rows_per_pass;
}

// Work unit u -> expert, weight-row block r, pass.  Expert e (rc[e] rows)
// contributes per_expert * passes(e) units (none if it has no rows).
__device__ __forceinline__ void unit_of(const int* rc, int per_expert, int rows_per_pass, int u, int* e_out, int* r_out,
                                        int* p_out) {
  int pre = 0, e_sel = 0, pre_sel = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    const int n = per_expert * passes_of(rc[e], rows_per_pass);
    if (u >= pre && u < pre + n) {
      e_sel = e;
      pre_sel = pre;
    }
    pre += n;
  }
  const int local = u - pre_sel;
  *e_out = e_sel;
  *p_out = local / per_expert;
  *r_out = local - *p_out * per_expert;
}

// UP: units (expert, 8*NB rows of w1 and the same rows of w3: NB/2 blocks
// of 16 each, pass), act = x (T rows), out = h (bf16).
// DOWN: units (expert, 16*NB rows of w2, pass), act = h (n_slots rows),
// out = y_rows (fp32).
// TAIL: only the rows of each expert past its last multiple of 256, for
// the experts whose last 256-row tile holds at most kTailRows of them (the
// rows the prefill GEMM leaves out; see its deal); otherwise all its rows.
// A stage covers W bytes (W/2 reduction elements) of each row.  A pass
// handles up to 16*MAXG of the expert's rows; an expert with more rows
// streams its weights once per pass.  Token group g of a unit is loaded only
// if it holds one of the expert's rows; the loads of the other groups use an
// offset past the end of the buffer, which the buffer hardware answers with
// zeros and no memory traffic (the instruction count, and so the wait,
// stays fixed).
// Down-projection tails with few units for the grid (one or two experts
// with tails leave most waves idle) also split the reduction: P parts
// (doubling while the units still fit the grid, at most kMaxTailParts and
// tail_pcap, dividing the stage count), unit u = part u / U of base unit
// u % U.  With P > 1 each part stores fp32 partial sums to tail_part (layout
// in launch.hpp) and a later launch adds them; workgroup 0 records P in the
// buffer's header either way.
template <bool UP, bool TAIL, int W, int NB, int MAXG, int S>
__global__ void __launch_bounds__(kWave) decode_stream_kernel(const bf16_t* __restrict__ act,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const int32_t* __restrict__ offs,
                                                              const bf16_t* __restrict__ wa,
                                                              const bf16_t* __restrict__ wb, void* __restrict__ out,
                                                              int d, int f, int act_rows, float* __restrict__ tail_part,
                                                              int tail_pcap) {
  constexpr int kStageK = W / 2;                  // reduction elements per stage
  constexpr int kChunks = W / 16;                 // 16-byte chunks per LDS row
  constexpr int kBlockElems = 16 * kStageK;       // one 16-row block of a stage
  constexpr int kRowsPerLoad = 1024 / W;          // rows one 1 KiB load instruction covers
  constexpr int kLoadsPerBlock = 16 / kRowsPerLoad;
  constexpr int kStageElems = (NB + MAXG) * kBlockElems;
  constexpr int kLoads = kLoadsPerBlock * (NB + MAXG);  // load instructions per stage
  constexpr int kRowsPerPass = 16 * MAXG;
  static_assert(W == 256 || W == 512, "row run per stage");
  static_assert(NB % 2 == 0 && NB <= 4 && MAXG <= 4, "unit shape");
  static_assert((S - 1) * kLoads <= 63, "vmcnt holds at most 63 loads in flight");
  __shared__ __align__(16) bf16_t ring[S][kStageElems];

  const int lane = threadIdx.x;
  const int l16 = lane % 16, lg = lane / 16;
  const int ld_row = lane / kChunks, ld_chunk = lane % kChunks;  // a load lane's row and physical chunk
  const int K = UP ? d : f;                                      // reduction length
  const int unit_rows = UP ? 8 * NB : 16 * NB;                   // weight rows per unit and matrix
  const int per_expert = (UP ? f : d) / unit_rows;               // weight-row blocks per expert
  const int KS = K / kStageK;                                    // stages per unit (>= 1)
  const uint32_t act_bytes = static_cast<uint32_t>(act_rows) * static_cast<uint32_t>(K * 2);
  int e_begin[kExperts], e_rows[kExperts];  // each expert's first row and row count here
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    const int b = offs[e], c = offs[e + 1] - b;
    if constexpr (TAIL) {
      const int full = (c - 1) / kTailTile * kTailTile;  // rows in the expert's full 256-row tiles
      const bool thin = c > kTailTile && c - full <= kTailRows;
      e_begin[e] = b + full;
      e_rows[e] = thin ? c - full : 0;
    } else {
      e_begin[e] = b;
      e_rows[e] = c;
    }
  }
  int n_units = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) n_units += per_expert * passes_of(e_rows[e], kRowsPerPass);
  const int G = gridDim.x;
  constexpr bool kSplit = TAIL && !UP;  // only these instantiations split the reduction
  int P = 1;  // reduction parts
  if constexpr (kSplit) {
    if (tail_part) {
      while (2 * P <= kMaxTailParts && 2 * P <= tail_pcap && n_units * 2 * P <= G && KS % (2 * P) == 0) P *= 2;
      if (blockIdx.x == 0 && lane == 0) *reinterpret_cast<int*>(tail_part) = P;
    }
  }
  const int n_total = n_units * P;
  const int KSp = KS / P;  // stages per unit
  if (static_cast<int>(blockIdx.x) >= n_total) return;
  const int total = (n_total - static_cast<int>(blockIdx.x) + G - 1) / G * KSp;

  // Loads: instruction i of a 16-row block puts rows kRowsPerLoad*i .. +
  // kRowsPerLoad-1 into 1 KiB of LDS, this lane's 16 bytes at physical
  // chunk ld_chunk of row kRowsPerLoad*i + ld_row, which holds logical chunk
  // ld_chunk ^ row: the fragment reads (16 rows x one logical chunk) then hit
  // 16 distinct bank groups.
  uint32_t w_off[8];  // kLoadsPerBlock <= 8 (fixed extent: see t_off below)
#pragma unroll
  for (int i = 0; i < kLoadsPerBlock; ++i) {
    const int rr = kRowsPerLoad * i + ld_row;
    w_off[i] = static_cast<uint32_t>(rr * K * 2 + ((ld_chunk ^ rr) * 16));
  }

  // Issue side: unit, stage within it, buffer resources and token offsets.
  int iu = blockIdx.x, iks = 0, ikbase = 0;
  __amdgpu_buffer_rsrc_t ra, rb;
  // (Fixed extents: an array sized by a template parameter and passed to
  // the buffer-load builtin keeps clang from emitting the launch stub.)
  uint32_t t_off[4][8];
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(act), 0, act_bytes, kBufferFlags);
#define SET_ISSUE_UNIT(U_)                                                                                   \
  {                                                                                                        \
    int e_, r_, p_;                                                                                        \
    const int part_ = kSplit ? (U_) / n_units : 0;                                                         \
    ikbase = part_ * KSp;                                                                                  \
    unit_of(e_rows, per_expert, kRowsPerPass, (U_) - part_ * n_units, &e_, &r_, &p_);                      \
    const int row_begin = e_begin[e_], rows = e_rows[e_];                                                    \
    const bf16_t* a0;                                                                                      \
    const bf16_t* b0;                                                                                      \
    if constexpr (UP) {                                                                                    \
      a0 = wa + (static_cast<int64_t>(e_) * f + r_ * unit_rows) * d;                                       \
      b0 = wb + (static_cast<int64_t>(e_) * f + r_ * unit_rows) * d;                                       \
    } else {                                                                                               \
      a0 = wa + (static_cast<int64_t>(e_) * d + r_ * unit_rows) * f;                                       \
      b0 = a0;                                                                                             \
    }                                                                                                      \
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a0), 0, 0x7FFFFFFF, kBufferFlags);          \
    rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(b0), 0, 0x7FFFFFFF, kBufferFlags);          \
    _Pragma("unroll") for (int g = 0; g < MAXG; ++g) _Pragma("unroll") for (int q = 0; q < kLoadsPerBlock; ++q) { \
      const int rr = kRowsPerLoad * q + ld_row; /* row of the group; clamped rows are loaded, not stored */ \
      const int m0 = p_ * kRowsPerPass + 16 * g; /* the group's first row */                               \
      int tok;                                                                                             \
      if constexpr (UP) {                                                                                  \
        /* slot ids through the scalar cache (uniform addresses, lgkmcnt): a vector load here would be     \
           ordered behind the weight loads in flight, and waiting for it would drain them; the select is   \
           arithmetic so that all the loads stay unconditional */                                          \
        const int b = m0 + kRowsPerLoad * q;                                                               \
        int sel = sorted_slots[row_begin + min(b, rows - 1)];                                              \
        _Pragma("unroll") for (int k = 1; k < kRowsPerLoad; ++k)                                           \
          sel += (ld_row >= k) * (sorted_slots[row_begin + min(b + k, rows - 1)] -                         \
                                  sorted_slots[row_begin + min(b + k - 1, rows - 1)]);                     \
        tok = sel / kTopK;                                                                                 \
      } else {                                                                                             \
        tok = row_begin + min(m0 + rr, rows - 1);                                                          \
      }                                                                                                    \
      const uint32_t chunk = static_cast<uint32_t>((ld_chunk ^ rr) * 16);                                  \
      t_off[g][q] = m0 < rows ? static_cast<uint32_t>(tok) * static_cast<uint32_t>(K * 2) + chunk         \
                              : act_bytes + chunk; /* past the end: zeros, no traffic */                   \
    }                                                                                                      \
  }
#define ISSUE(SLOT_)                                                                                       \
  {                                                                                                        \
    bf16_t* st_ = ring[SLOT_];                                                                             \
    const int so = (ikbase + iks) * W;                                                                     \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                       \
      const int bo = (UP ? b % (NB / 2) : b) * 16 * K * 2; /* block's first row */                         \
      _Pragma("unroll") for (int i = 0; i < kLoadsPerBlock; ++i)                                           \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(UP && b >= NB / 2 ? rb : ra,                              \
                                                 LDS_PTR(st_ + b * kBlockElems + i * 512), 16, w_off[i],   \
                                                 so + bo, 0, kNontemporal);                                \
    }                                                                                                      \
    _Pragma("unroll") for (int g = 0; g < MAXG; ++g) _Pragma("unroll") for (int q = 0; q < kLoadsPerBlock; ++q) \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, LDS_PTR(st_ + (NB + g) * kBlockElems + q * 512), 16,    \
                                               t_off[g][q], so, 0, 0);                                     \
    if (++iks == KSp) {                                                                                    \
      iks = 0;                                                                                             \
      iu += G;                                                                                             \
      if (iu < n_total) SET_ISSUE_UNIT(iu);                                                                \
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
  int ce, cr, cp, cpart = kSplit ? cu / n_units : 0;
  unit_of(e_rows, per_expert, kRowsPerPass, cu - cpart * n_units, &ce, &cr, &cp);
  f32x4 acc[NB][MAXG];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int g = 0; g < MAXG; ++g) acc[b][g] = f32x4{0.f, 0.f, 0.f, 0.f};
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
      bf16x8 w[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) w[b] = *reinterpret_cast<const bf16x8*>(st + b * kBlockElems + off);
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {  // all groups: MFMA time is free here, a branch is not
        const bf16x8 t = *reinterpret_cast<const bf16x8*>(st + (NB + g) * kBlockElems + off);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[b], t, acc[b][g], 0, 0, 0);
      }
    }
    cslot = cslot == S - 1 ? 0 : cslot + 1;
    if (++cks == KSp) {
      // acc[b][g][q]: expert row cp*16*MAXG + 16g + l16, feature 4*lg + q of
      // weight block b (up: blocks < NB/2 gate, the rest up, same features).
      const int c_begin = e_begin[ce], c_rows = e_rows[ce];
#pragma unroll
      for (int g = 0; g < MAXG; ++g) {
        const int m = cp * kRowsPerPass + 16 * g + l16;
        if (m >= c_rows) continue;
        const int64_t orow = c_begin + m;
        if (kSplit && P > 1) {  // a part's partial sums (tail rows: m < kTailRows)
          float* dst = tail_part + kTailPartHeader + ((cpart * kExperts + ce) * kTailRows + m) * static_cast<int64_t>(d);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            *reinterpret_cast<float4*>(dst + cr * unit_rows + b * 16 + 4 * lg) =
                make_float4(acc[b][g][0], acc[b][g][1], acc[b][g][2], acc[b][g][3]);
          continue;
        }
        if constexpr (UP) {
#pragma unroll
          for (int b = 0; b < NB / 2; ++b) {
            const f32x4 a = acc[b][g], u = acc[b + NB / 2][g];
            uint2 p;
            p.x = pack_bf16x2(silu(a[0]) * u[0], silu(a[1]) * u[1]);
            p.y = pack_bf16x2(silu(a[2]) * u[2], silu(a[3]) * u[3]);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(out) + orow * f + cr * unit_rows + b * 16 + 4 * lg) = p;
          }
        } else {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * d + cr * unit_rows + b * 16 + 4 * lg) =
                make_float4(acc[b][g][0], acc[b][g][1], acc[b][g][2], acc[b][g][3]);
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int g = 0; g < MAXG; ++g) acc[b][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      cks = 0;
      cu += G;
      if (cu < n_total) {
        cpart = kSplit ? cu / n_units : 0;
        unit_of(e_rows, per_expert, kRowsPerPass, cu - cpart * n_units, &ce, &cr, &cp);
      }
    }
  }
}

#undef SET_ISSUE_UNIT
#undef ISSUE
#undef LDS_PTR

// GM workgroups (single waves) per CU.
template <bool UP, int W, int NB, int MAXG, int S, int GM = 2, bool TAIL = false>
hipError_t launch_stream(const bf16_t* act, const int32_t* sorted_slots, const int32_t* offs, const bf16_t* wa,
                         const bf16_t* wb, void* out, int d, int f, int act_rows, int n_cu, hipStream_t s,
                         float* tail_part = nullptr, int tail_pcap = 0) {
  hipLaunchKernelGGL((decode_stream_kernel<UP, TAIL, W, NB, MAXG, S>), dim3(GM * n_cu), dim3(kWave), 0, s, act,
                     sorted_slots, offs, wa, wb, out, d, f, act_rows, tail_part, tail_pcap);
  return hipGetLastError();
}

}  // namespace

// T <= 32: one token group per pass (16 rows; an expert with more takes a
// second pass, rare with 8 rows per expert on average); T <= 64: two groups
// per pass.  Shapes measured at d=4096, f=14336 on MI355X (alternating
// launches in one process, two weight sets): T=32, up projection with
// 512-byte row runs, 3 stages (268-277 us; 256-byte runs, 6 stages: 281-292
// us), down projection with units of 64 rows of w2, 3 stages (138-144 us;
// 32-row units: 158-163 us); T=48 and 64, up with 512-byte runs, 2 stages
// (282-285 us; 256-byte runs: 292-306 us), down with 64-row units, 3 stages
// (141 us; 32-row units: 161-170 us); T=96 and 128 (four groups per pass),
// units of 32 rows of w1 and w3 / 64 rows of w2, 2 stages (up 318-330 us,
// down 159-162 us; 16- and 32-row units with 3 stages: up 368-392, down
// 193-197; 512-byte runs, one workgroup per CU: 633-643 and 317-325).  d and
// f are multiples of 128 (checked at the boundary): 512-byte runs need d to
// be a multiple of 256, the other shapes divide any such d and f.
hipError_t launch_up_decode_stream(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots,
                                   const bf16_t* w1, const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, int n_cu,
                                   hipStream_t s) {
  if (T > kStreamMaxTokens) return hipErrorInvalidValue;
  if (T <= 32) {
    if (d % 256 == 0) return launch_stream<true, 512, 2, 1, 3>(x, sorted_slots, offs, w1, w3, h, d, f, T, n_cu, s);
    return launch_stream<true, 256, 2, 1, 6>(x, sorted_slots, offs, w1, w3, h, d, f, T, n_cu, s);
  }
  if (T <= 64) {
    if (d % 256 == 0) return launch_stream<true, 512, 2, 2, 2>(x, sorted_slots, offs, w1, w3, h, d, f, T, n_cu, s);
    return launch_stream<true, 256, 2, 2, 4>(x, sorted_slots, offs, w1, w3, h, d, f, T, n_cu, s);
  }
  return launch_stream<true, 256, 4, 4, 2>(x, sorted_slots, offs, w1, w3, h, d, f, T, n_cu, s);
}

hipError_t launch_down_decode_stream(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T,
                                     int d, int f, int n_cu, hipStream_t s) {
  if (T > kStreamMaxTokens) return hipErrorInvalidValue;
  const int n_slots = static_cast<int>(T) * kTopK;
  if (T <= 32) return launch_stream<false, 256, 4, 1, 3>(h, nullptr, offs, w2, nullptr, y_rows, d, f, n_slots, n_cu, s);
  if (T <= 64) return launch_stream<false, 256, 4, 2, 3>(h, nullptr, offs, w2, nullptr, y_rows, d, f, n_slots, n_cu, s);
  return launch_stream<false, 256, 4, 4, 2>(h, nullptr, offs, w2, nullptr, y_rows, d, f, n_slots, n_cu, s);
}

// Tails of the prefill layer (rows of an expert past its last full 256-row
// tile when at most 32): one pass of two token groups.  x / h as in the
// prefill launch; n_slots = T * 2.  Shapes measured on the T=4096 layer's
// three tails (alternating launches in one process, bit-identical outputs):
// up projection, units of 32 rows of w1 and w3, 3 stages, two waves per CU:
// 119 us (units of 16 rows, 4 stages: 129; 512-byte runs: 123-143; three
// waves per CU: 124-138; one: 146-183); down projection, units of 32 rows of
// w2, 3 stages, three waves per CU: 60 us (64-row units, two waves per CU,
// the earlier shape: 73; 512-byte runs: 76-86).
hipError_t launch_up_tail_stream(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                                 const bf16_t* w3, bf16_t* h, int64_t T, int d, int f, int n_cu, hipStream_t s) {
  return launch_stream<true, 256, 4, 2, 3, 2, true>(x, sorted_slots, offs, w1, w3, h, d, f, static_cast<int>(T), n_cu,
                                                     s);
}

hipError_t launch_down_tail_stream(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int64_t T,
                                   int d, int f, int n_cu, float* tail_part, int64_t tail_part_bytes, hipStream_t s) {
  const int n_slots = static_cast<int>(T) * kTopK;
  const int pcap = tail_part_capacity(tail_part, tail_part_bytes, d);
  return launch_stream<false, 256, 2, 2, 3, 3, true>(h, nullptr, offs, w2, nullptr, y_rows, d, f, n_slots, n_cu, s,
                                                     pcap >= 2 ? tail_part : nullptr, pcap);
}

}  // namespace moe
