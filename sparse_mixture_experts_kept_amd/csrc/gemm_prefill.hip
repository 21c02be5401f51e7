// bf16 grouped expert GEMMs for prefill-sized batches, on gfx950 MFMA.
//
// Up projection with the SwiGLU fused into the epilogue, and the down
// projection ("Mixtral of Experts", azimuth.plus, architecture paragraph:
// SwiGLU experts; "Mixtral > Architecture Overview", parameter-count
// paragraph: gate w1, up w3 and down w2 projections):
//   up:   h[r, n]      = SiLU(x[tok(r)] . w1_e[n]) * (x[tok(r)] . w3_e[n])   -> bf16
//   down: y_rows[r, n] = h[r] . w2_e[n]                                      -> fp32
// for the rows r = offsets[e] .. offsets[e+1]-1 of expert e (tok(r) =
// sorted_slots[r] / 2, the gather fused into the A-tile load).
//
// Design (gfx950):
// - Persistent workgroups of 256 threads: 4 waves, one per SIMD.  Block tile
//   256 (rows) x 256 (weight rows), stepped 64 deep in k so that every row of
//   a tile is one full 128-byte line.  Each wave owns a 128 x 128 quarter:
//   8 x 8 tiles of v_mfma_f32_16x16x32_bf16 with fp32 accumulators in the 256
//   AGPRs.  Against 8 waves of 128 x 64 this reads a third less LDS per flop.
// - LDS (160 KiB) holds 5 slots of 32 KiB: A tiles in 2 slots, B tiles in 3,
//   so weight loads run up to two stages ahead and token loads one.  Slots
//   are filled with direct global->LDS loads (global_load_lds_dwordx4, 1 KiB
//   = 8 rows per instruction, no staging registers).
// - Per stage and wave: 128 MFMAs in 16 rows of 8; each row is cut into
//   pairs of MFMAs with one load, then one fragment read (ds_read_b128), then
//   another read between them (MFMA MFMA load MFMA MFMA read MFMA MFMA read
//   MFMA MFMA), so the memory instructions issue while the MFMAs run (a
//   load or read burst after each full row left the MFMA pipe idle: 4% on
//   both projections).  One barrier per stage, between its two k-halves.  All waits are explicit (s_waitcnt vmcnt(N) before the raw
//   barrier; the compiler adds the LDS-read waits before the MFMAs).
// - LDS rows are 128 B with the 16-byte chunk index XOR-swizzled by bits 1..3
//   of the row; the bank-conflict counter reads zero for the 16 rows x 4
//   chunks pattern of the fragment reads.
// - Load addresses are a uniform stage base plus a 32-bit per-lane byte
//   offset, so a load costs one address add and an M0 write.
// - Tile order: the tiles of one expert are walked in groups of 4 n-tiles x
//   all its m-tiles; workgroup b runs on XCD b % 8 and each XCD owns one
//   contiguous eighth of the tile list, so the 32 workgroups of an XCD share
//   weight and token panels in that XCD's L2.
// - For the up projection the B tile is [gate 0-63 | up 0-63 | gate 64-127 |
//   up 64-127] of 128 output columns, so each wave holds gate and up sums of
//   the same 64 columns and applies SiLU(g)*u in registers before one bf16
//   rounding.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kBM = 256;       // block rows (slots)
constexpr int kBN = 256;       // block weight rows
constexpr int kBK = 64;        // k depth of one stage (128 B per row)
constexpr int kThreads = 256;  // 4 waves
constexpr int kXcds = 8;
constexpr int kGroupN = 4;     // n-tiles per group in the tile order
constexpr int kThinRows = 32;  // m-tiles with at most this many rows take the thin path
constexpr int kSmallRows = 64;    // ... at most this many, the small path
constexpr int kMediumRows = 128;  // ... and at most this many, the medium path
static_assert(kThinRows == kTailPartRows, "the streamed tails are the thin tiles");
constexpr int kSlotElems = kBM * kBK;  // one 32 KiB slot (kBM == kBN)
// Word 3 of a raw buffer resource on gfx9 (no format conversion).
constexpr int kBufferFlags = 0x00020000;
// num_records of the GEMM's resources: every unsigned 32-bit byte offset but
// the last is in range (offsets here stay below T*d*2 < 2^32).
constexpr int kWholeRange = static_cast<int>(0xFFFFFFFFu);

#define GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate: at most n vector-memory ops outstanding (gfx9
// encoding: vmcnt in bits 3:0 and 15:14), expcnt and lgkmcnt not waited on.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// ... and every LDS read complete as well.
constexpr int lgkm0_mask() { return ~(0xF << 8); }

// Workgroup barrier for the LDS slots; the waits it needs are issued before
// it, the empty asm keeps LDS accesses from moving across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Element offset of (row, logical 16-byte chunk) in a [rows][64] bf16 tile.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

// Work units and their deal.  An expert with c rows has ceil(c / 256)
// m-tiles; when its last one holds at most kThinRows rows and it is not the
// only one, that tile is "thin" (cheap: see the thin path below).  Units are
// (expert, m-tile, n-tile, k-part).  Full units are listed expert by expert,
// each expert's in groups of kGroupN n-tiles x all its full m-tiles (x
// SPLITK, innermost), and split into 8 equal contiguous ranges, one per XCD;
// within an XCD, slot s takes every 32nd full unit, so every workgroup gets
// the same number of full units.  A thin unit (expert, group, n-tile, part)
// is anchored at the full unit (expert, group, last full m-tile, same n-tile,
// same part), which shares its weight panel, and is dealt by the XCD that
// owns its anchor (slots offset by half a round, so thin units and the last
// full units of a round land on different workgroups); a workgroup runs its
// thin units interleaved with its full units in anchor order.
// (Everything below is recomputed from the offsets with unrolled loops: no
// private arrays indexed at run time, which would live in scratch memory.)
__device__ __forceinline__ void expert_shape(const int32_t* offs, int e, int* full_m, bool* thin) {
  const int cnt = offs[e + 1] - offs[e];
  const int mts = (cnt + kBM - 1) / kBM;
  *thin = mts >= 2 && cnt - (mts - 1) * kBM <= kThinRows;
  *full_m = mts - (*thin ? 1 : 0);
}

// Total full units and thin units.
template <int SPLITK>
__device__ __forceinline__ void unit_counts(const int32_t* offs, int n_tiles_n, int* n_full, int* n_thin) {
  int nf = 0, nt = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    int fm;
    bool th;
    expert_shape(offs, e, &fm, &th);
    nf += fm * n_tiles_n * SPLITK;
    nt += th ? n_tiles_n * SPLITK : 0;
  }
  *n_full = nf;
  *n_thin = nt;
}

// Full unit u -> (expert, m-tile, n-tile, part).
template <int SPLITK>
__device__ __forceinline__ void full_unit(const int32_t* offs, int n_tiles_n, int u, int* e_out, int* mt, int* nt,
                                          int* ks) {
  int pre = 0, e_sel = 0, pre_sel = 0, fm_sel = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    int fm;
    bool th;
    expert_shape(offs, e, &fm, &th);
    const int n = fm * n_tiles_n * SPLITK;
    if (u >= pre && u < pre + n) {
      e_sel = e;
      pre_sel = pre;
      fm_sel = fm;
    }
    pre += n;
  }
  const int local = u - pre_sel;
  const int per_group = fm_sel * kGroupN * SPLITK;  // every group but the last is full width
  const int g = local / per_group;
  const int rem = local - g * per_group;
  const int gw = min(kGroupN, n_tiles_n - g * kGroupN);
  const int r2 = rem / SPLITK;
  *e_out = e_sel;
  *ks = rem - r2 * SPLITK;
  *mt = r2 / gw;
  *nt = g * kGroupN + r2 % gw;
}

// Thin unit t -> (expert, its m-tile, n-tile, part); returns the full unit it
// is anchored at.
template <int SPLITK>
__device__ __forceinline__ int thin_unit(const int32_t* offs, int n_tiles_n, int t, int* e_out, int* mt, int* nt,
                                         int* ks) {
  int tpre = 0, fpre = 0, e_sel = 0, tpre_sel = 0, fpre_sel = 0, fm_sel = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    int fm;
    bool th;
    expert_shape(offs, e, &fm, &th);
    const int n = th ? n_tiles_n * SPLITK : 0;
    if (t >= tpre && t < tpre + n) {
      e_sel = e;
      tpre_sel = tpre;
      fpre_sel = fpre;
      fm_sel = fm;
    }
    tpre += n;
    fpre += fm * n_tiles_n * SPLITK;
  }
  const int local = t - tpre_sel;
  const int g = local / (kGroupN * SPLITK);
  const int rem = local - g * kGroupN * SPLITK;
  const int j = rem / SPLITK;
  const int gw = min(kGroupN, n_tiles_n - g * kGroupN);
  *e_out = e_sel;
  *ks = rem - j * SPLITK;
  *mt = fm_sel;
  *nt = g * kGroupN + j;
  return fpre_sel + g * fm_sel * kGroupN * SPLITK + ((fm_sel - 1) * gw + j) * SPLITK + *ks;
}

// Remainder split.  When the full units do not fill whole rounds of the grid
// (n_full = R*G + rem with 0 < rem), running the last rem units whole would
// leave G - rem workgroups idle for a whole unit.  Instead the first R*G units
// are dealt as usual (R per workgroup) and each of the last rem is cut along
// the reduction into P = min(G / rem, KT / 2, planes / rem) parts of at least
// two stages: piece c = p*rem + r (part p of remainder unit r) runs on
// workgroup c and stores its fp32 partial tile in plane c of the partial
// buffer; remainder_fixup_kernel then adds the P planes of each unit in part
// order.  Used only without thin units in the GEMM and without SPLITK.
struct RemSplit {
  int n_main, rem, parts;
};
__device__ __forceinline__ RemSplit remainder_split(int n_full, int grid, int KT, int planes, bool enabled) {
  RemSplit r{n_full, 0, 1};
  if (!enabled || grid <= 0) return r;
  const int R = n_full / grid, rem = n_full - R * grid;
  if (rem == 0) return r;
  const int P = min(min(grid / rem, KT / 2), planes / rem);
  if (P < 2) return r;
  r.n_main = R * grid;
  r.rem = rem;
  r.parts = P;
  return r;
}
constexpr int kPlaneElems = kBM * kBN;  // one fp32 partial tile: [256 tile rows][256 B-tile rows]

// First thin unit whose anchor is at or past full unit u (anchors rise with t).
template <int SPLITK>
__device__ __forceinline__ int first_thin_from(const int32_t* offs, int n_tiles_n, int n_thin, int u) {
  int lo = 0, hi = n_thin;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    int e, mt, nt, ks;
    if (thin_unit<SPLITK>(offs, n_tiles_n, mid, &e, &mt, &nt, &ks) < u)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// ---- pieces of the main loop (macros keep the fragment arrays in registers)

// Load j (0..7) of this wave for stage KT: 8 rows of 128 B, A rows go to A
// slot KT&1, B rows to B slot BSL (0..2).  Buffer loads: a per-tile scalar
// resource, a 32-bit per-lane byte offset fixed for the tile and the stage's
// byte offset as the scalar offset, so a load needs no address arithmetic.
#define LOAD_A(KT_, J)                                                                                   \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, LDS_PTR(&ring[(KT_) & 1][(wave * 64 + (J) * 8) * kBK]), 16, \
                                           a_off[J], (KT_) * (kBK * 2), 0, 0);
#define LOAD_B(KT_, J, BSL)                                                                              \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, LDS_PTR(&ring[2 + (BSL)][(wave * 64 + (J) * 8) * kBK]), 16, \
                                           b_off[J], (KT_) * (kBK * 2), 0, 0);

// Fragments of k-half H (0/1): B block J from B slot BSL, A block I from A slot AS.
#define READ_B(FB, BSL, H, J) \
  FB[J] = *reinterpret_cast<const bf16x8*>(&ring[2 + (BSL)][lds_off(wn * 128 + (J) * 16 + l16, (H) * 4 + lg)]);
#define READ_A(FA, AS, H, I) \
  FA[I] = *reinterpret_cast<const bf16x8*>(&ring[AS][lds_off(wm * 128 + (I) * 16 + l16, (H) * 4 + lg)]);
// Pair Q (0..7) of the 16 fragments of a set, B first: MFMA row 0 needs all
// of B and A block 0.
// (The "& 7" only keeps the untaken branch's indices in range.)
#define READ_PAIR(FA, FB, AS, BSL, H, Q)     \
  if ((Q) < 4) {                             \
    READ_B(FB, BSL, H, (2 * (Q)) & 7);       \
    READ_B(FB, BSL, H, (2 * (Q) + 1) & 7);   \
  } else {                                   \
    READ_A(FA, AS, H, (2 * (Q) - 8) & 7);    \
    READ_A(FA, AS, H, (2 * (Q) - 7) & 7);    \
  }

// Element K (0/1) of pair Q.
#define READ_ONE(FA, FB, AS, BSL, H, Q, K)        \
  if ((Q) < 4) {                                  \
    READ_B(FB, BSL, H, (2 * (Q) + (K)) & 7);      \
  } else {                                        \
    READ_A(FA, AS, H, (2 * (Q) - 8 + (K)) & 7);   \
  }

// MFMA row I is the wave's A block I times its 8 B blocks; MFMA_QROW issues
// pair Q (B blocks 2Q, 2Q+1) of it.
#define MFMA_QROW(FA, FB, I, Q)                                                                           \
  _Pragma("unroll") for (int j = 2 * (Q); j < 2 * (Q) + 2; ++j) acc[I][j] =                               \
      __builtin_amdgcn_mfma_f32_16x16x32_bf16(FB[j], FA[I], acc[I][j], 0, 0, 0);

// Stage KT (A in slot KT&1, B in B slot BS = KT%3; BS1, BS2 = (KT+1)%3, (KT+2)%3):
//   half 0: MFMA rows of set 0; within each row (LD) one B load of stage
//           KT+2 into B slot BS2 (free since the barrier of stage KT-1) and
//           two reads of k-half 1 into set 1
//   wait until only stage KT+2's B loads are in flight; barrier.  All waves
//           have read stage KT completely, and stage KT+1 has landed.
//   half 1: MFMA rows of set 1; within each row (LD) one A load of stage
//           KT+2 into A slot KT&1 and (RD) two reads of k-half 0 of stage
//           KT+1 into set 0.
// Reads are issued one row early at the end of each half so the first MFMAs
// of the next half find them complete.
#define STAGE(KT_, BS, BS1, BS2, LD, RD)                                                \
  {                                                                                     \
    const int as_ = (KT_) & 1;                                                          \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                     \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa0, fb0, i, 0);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (LD) { LOAD_B((KT_) + 2, i, BS2); }                                            \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa0, fb0, i, 1);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (i < 7) { READ_ONE(fa1, fb1, as_, BS, 1, i, 0); }                              \
      if (i == 6) { READ_ONE(fa1, fb1, as_, BS, 1, 7, 0); }                             \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa0, fb0, i, 2);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (i < 7) { READ_ONE(fa1, fb1, as_, BS, 1, i, 1); }                              \
      if (i == 6) { READ_ONE(fa1, fb1, as_, BS, 1, 7, 1); }                             \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa0, fb0, i, 3);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    if (LD)                                                                             \
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(8) & lgkm0_mask());                          \
    else                                                                                \
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lgkm0_mask());                          \
    lds_barrier();                                                                      \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                     \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa1, fb1, i, 0);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (LD) { LOAD_A((KT_) + 2, i); }                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa1, fb1, i, 1);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if ((RD) && i < 7) { READ_ONE(fa0, fb0, as_ ^ 1, BS1, 0, i, 0); }                 \
      if ((RD) && i == 6) { READ_ONE(fa0, fb0, as_ ^ 1, BS1, 0, 7, 0); }                \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa1, fb1, i, 2);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if ((RD) && i < 7) { READ_ONE(fa0, fb0, as_ ^ 1, BS1, 0, i, 1); }                 \
      if ((RD) && i == 6) { READ_ONE(fa0, fb0, as_ ^ 1, BS1, 0, 7, 1); }                \
      __builtin_amdgcn_sched_barrier(0);                                                \
      MFMA_QROW(fa1, fb1, i, 3);                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  }

// One direct global->LDS load of 16 bytes per lane (1 KiB per wave) at byte
// offsets voff (per lane) + soff (uniform) from the resource's base.  (A
// plain function: the compiler's host pass does not resolve this builtin
// when it is called from a device-function template.)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, bf16_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds), 16, voff, soff, 0, 0);
}

// Medium tile: a tile with 65..128 rows (an expert's only or last m-tile).
// As the thin tile, the four waves split the 256 weight rows (64 each) and
// take every token row: 128 rows x 64 weight rows per wave (8 x 4 MFMA
// tiles), half the MFMAs of a full tile.  Loads run two stages ahead: the
// weight tiles in slots 0-2, the 128 token rows (16 KiB per stage; wave w
// fills rows 32w..32w+31) in three sub-slots in slots 3-4.  Each stage
// waits for its own loads, then a barrier, which also frees the slots of the
// stage before.
template <bool SWIGLU>
__device__ __forceinline__ void medium_tile(bf16_t (*ring)[kSlotElems], __amdgpu_buffer_rsrc_t a_rsrc,
                                            __amdgpu_buffer_rsrc_t b_rsrc, const uint32_t (&b_off)[8],
                                            const int32_t* __restrict__ gather, int row_begin, int rows, int m0, int n0,
                                            int K, int N, int wave, int lane, int lc_even, int lc_odd, int kt_n,
                                            float* plane, void* Cout, int ks, int64_t split_stride) {
  constexpr int RB = kMediumRows / 16;  // row blocks of 16
  constexpr int kSub = RB * 16 * kBK;    // elements of one token sub-slot
  constexpr int kALoads = RB / 2;        // token loads per wave and stage (8 rows each)
  constexpr int kLoads = 8 + kALoads;    // loads per wave and stage
  static_assert(3 * kSub <= 2 * kSlotElems, "three token sub-slots fit in slots 3-4");
  bf16_t* const flat = &ring[0][0];
  const int ld_row = lane / 8, l16 = lane % 16, lg = lane / 16;
  uint32_t ma_off[kALoads];
#pragma unroll
  for (int j = 0; j < kALoads; ++j) {
    const int lc = (j & 1) ? lc_odd : lc_even;  // swizzle of LDS row 32*wave + 8*j + ld_row
    if constexpr (SWIGLU)
      ma_off[j] = ((static_cast<uint32_t>(gather[row_begin + min(m0 + wave * 32 + j * 8 + ld_row, rows - 1)]) /
                    kTopK) * static_cast<uint32_t>(K) + lc) * 2u;
    else
      ma_off[j] = (static_cast<uint32_t>(min(wave * 32 + j * 8 + ld_row, rows - 1 - m0)) *
                       static_cast<uint32_t>(K) + lc) * 2u;
  }
#define MED_A(KT_) (flat + 3 * kSlotElems + ((KT_) % 3) * kSub)
#define LOAD_MED(KT_)                                                                                 \
  {                                                                                                   \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                                     \
        load_lds16(b_rsrc, &ring[(KT_) % 3][(wave * 64 + j * 8) * kBK], b_off[j], (KT_) * (kBK * 2)); \
    _Pragma("unroll") for (int j = 0; j < kALoads; ++j)                                               \
        load_lds16(a_rsrc, MED_A(KT_) + (wave * 32 + j * 8) * kBK, ma_off[j], (KT_) * (kBK * 2));     \
  }
  // Fragment reads: every row read sits at 16*block + l16, whose swizzle
  // (row >> 1) & 7 is (l16 >> 1) & 7 for any block, so a read is a uniform
  // block base plus one of two per-lane offsets (k-half 0 or 1).
  const int rd_lane0 = l16 * kBK + ((lg ^ ((l16 >> 1) & 7)) << 3);
  const int rd_lane1 = rd_lane0 ^ 32;  // logical chunk 4 + lg
  int mb_base[4];                      // this wave's B-tile row blocks (as the thin tile), in elements
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (SWIGLU)
      mb_base[j] = ((wave >> 1) * 128 + (j >= 2 ? 64 : 0) + (wave & 1) * 32 + (j & 1) * 16) * kBK;
    else
      mb_base[j] = (wave * 64 + j * 16) * kBK;
  }
  f32x4 macc[RB][4];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) macc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < 2 && st < kt_n; ++st) LOAD_MED(st);
  for (int kt = 0; kt < kt_n; ++kt) {
    // stage kt+1 (if any) may stay in flight
    if (kt + 1 < kt_n)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();  // stage kt landed for all waves; stage kt-1 fully read
    if (kt + 2 < kt_n) LOAD_MED(kt + 2);  // into the slots of stage kt-1
    const bf16_t* sa = MED_A(kt);
    const bf16_t* sb = ring[kt % 3];
    // Both k-halves' fragments are read up front (the second half's reads
    // land while the first half's MFMAs run); left to itself the scheduler
    // reads one fragment per MFMA row and waits for each.
    bf16x8 ma[2][RB], mb[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int rd = hh ? rd_lane1 : rd_lane0;
#pragma unroll
      for (int j = 0; j < 4; ++j) mb[hh][j] = *reinterpret_cast<const bf16x8*>(sb + mb_base[j] + rd);
#pragma unroll
      for (int i = 0; i < RB; ++i) ma[hh][i] = *reinterpret_cast<const bf16x8*>(sa + i * 16 * kBK + rd);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          macc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mb[hh][j], ma[hh][i], macc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef LOAD_MED
#undef MED_A
  // every wave's reads of the last stage are done before the next tile refills the slots
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lgkm0_mask());
  lds_barrier();
  // Epilogue: macc[i][j][q] is row m0 + i*16 + l16, B-tile row block j's
  // row 4*lg + q.  (Lane index re-read: address terms formed here.)
  int elane = lane;
  asm volatile("" : "+v"(elane));
  const int el16 = elane % 16, elg = elane / 16;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int m = m0 + i * 16 + el16;
    if (m >= rows) continue;
    const int64_t orow = row_begin + m;
    if (plane) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int brow = SWIGLU ? (wave >> 1) * 128 + (j >= 2 ? 64 : 0) + (wave & 1) * 32 + (j & 1) * 16
                                : wave * 64 + j * 16;
        const f32x4 v = macc[i][j];
        *reinterpret_cast<float4*>(plane + (i * 16 + el16) * kBN + brow + 4 * elg) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
      continue;
    }
    if constexpr (SWIGLU) {
      bf16_t* C = static_cast<bf16_t*>(Cout);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + (wave >> 1) * 64 + (wave & 1) * 32 + j * 16 + 4 * elg;
        const f32x4 g = macc[i][j];
        const f32x4 u = macc[i][j + 2];
        uint2 p;
        p.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
        p.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
        *reinterpret_cast<uint2*>(C + orow * N + n) = p;
      }
    } else {
      float* C = static_cast<float*>(Cout) + ks * split_stride;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wave * 64 + j * 16 + 4 * elg;
        if (n >= N) continue;
        const f32x4 v = macc[i][j];
        *reinterpret_cast<float4*>(C + orow * N + n) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// SPLITK > 1 (down projection only): each tile's reduction is cut into
// SPLITK equal parts run as separate work units; part s writes its partial
// sums to Cout + s * split_stride (a separate buffer per part; the consumer
// adds them in a fixed order).
// CLOCKED: the same kernel, which also stores per workgroup the shader
// clock counter and the constant-rate (100 MHz) reference counter at its
// start and end, clk[4b .. 4b+3] = {cycles0, cycles1, ref0, ref1}: the
// clock the GEMM ran at, measured while it runs.
template <bool SWIGLU, int SPLITK, bool CLOCKED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
grouped_gemm_prefill_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ gather,
                            const int32_t* __restrict__ offs, const bf16_t* __restrict__ B0,
                            const bf16_t* __restrict__ B1, void* __restrict__ Cout, int N, int K,
                            int64_t split_stride, int thin_elsewhere, float* __restrict__ partials,
                            int planes, long long* __restrict__ clk) {
  static_assert(!SWIGLU || SPLITK == 1, "the SwiGLU epilogue needs the full reduction");
  long long cyc0 = 0, ref0 = 0;
  if constexpr (CLOCKED) {
    cyc0 = __builtin_amdgcn_s_memtime();
    ref0 = __builtin_amdgcn_s_memrealtime();
  }
  // One LDS object for all slots: A slots 0-1, B slots 2-4.
  __shared__ __align__(16) bf16_t ring[5][kSlotElems];

  // Output columns per tile: 128 (SwiGLU: 128 gate + 128 up B rows) or 256.
  constexpr int TN = SWIGLU ? kBN / 2 : kBN;
  const int n_tiles_n = (N + TN - 1) / TN;

  int n_full, n_thin;
  unit_counts<SPLITK>(offs, n_tiles_n, &n_full, &n_thin);
  if (thin_elsewhere) n_thin = 0;  // the thin tiles' rows are computed by another kernel
  const int k_part = K / SPLITK;
  const int KT = k_part / kBK;  // >= 2 (the host guarantees it)
  const RemSplit rs = remainder_split(n_full, gridDim.x, KT, planes, partials != nullptr && SPLITK == 1 && n_thin == 0);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int per = (rs.n_main + kXcds - 1) / kXcds;
  const int fbeg = min(xcd * per, rs.n_main);
  const int fend = min(fbeg + per, rs.n_main);
  const int tbeg = first_thin_from<SPLITK>(offs, n_tiles_n, n_thin, fbeg);
  const int tend = first_thin_from<SPLITK>(offs, n_tiles_n, n_thin, fend);

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / 2, wn = wave % 2;  // 2 x 2 waves of 128 x 128
  const int l16 = lane % 16, lg = lane / 16;
  // Loads: lane -> (row ld_row of the 8, physical chunk pc).  LDS row
  // r = wave*64 + j*8 + ld_row has swizzle (r >> 1) & 7 = (ld_row >> 1) |
  // 4*(j & 1), so the logical chunk a lane fetches takes two values.
  const int ld_row = lane / 8, pc = lane % 8;
  const int lc_even = (pc ^ (ld_row >> 1)) * 8;
  const int lc_odd = lc_even ^ 32;

  // This workgroup's full units fbeg + slot + i*slots and thin units
  // tbeg + (slot + slots/2) % slots + i*slots, merged in anchor order.
  int u = fbeg + slot;
  int t = tbeg + (slot + slots / 2) % slots;
  // ... then its piece of a remainder unit, if any.
  bool piece = static_cast<int>(blockIdx.x) < rs.rem * rs.parts;
  while (u < fend || t < tend || piece) {
    int e, mt, nt, ks;
    int kbeg = 0, kt_n = KT;  // this unit's stages: [kbeg, kbeg + kt_n) of its part
    float* plane = nullptr;   // partial-tile destination of a piece
    bool take_thin = false;
    if (t < tend) {
      int te, tmt, tnt, tks;
      const int anchor = thin_unit<SPLITK>(offs, n_tiles_n, t, &te, &tmt, &tnt, &tks);
      if (u >= fend || anchor < u) {
        take_thin = true;
        e = te;
        mt = tmt;
        nt = tnt;
        ks = tks;
      }
    }
    if (take_thin) {
      t += slots;
    } else if (u < fend) {
      full_unit<SPLITK>(offs, n_tiles_n, u, &e, &mt, &nt, &ks);
      u += slots;
    } else {
      const int c = blockIdx.x;
      const int r = c % rs.rem, p = c / rs.rem;
      full_unit<SPLITK>(offs, n_tiles_n, rs.n_main + r, &e, &mt, &nt, &ks);
      kbeg = p * KT / rs.parts;
      kt_n = (p + 1) * KT / rs.parts - kbeg;
      plane = partials + static_cast<int64_t>(c) * kPlaneElems;
      piece = false;
    }
    const int row_begin = offs[e];
    const int rows = offs[e + 1] - row_begin;
    const int m0 = mt * kBM;
    const int n0 = nt * TN;

    // A: token rows (gathered, up) or this tile's h rows (down), as byte
    // offsets from a uniform base; clamped rows are computed, never stored.
    const bf16_t* a_base;
    uint32_t a_off[8];
    if constexpr (SWIGLU) {
      int32_t slot_id[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) slot_id[j] = gather[row_begin + min(m0 + wave * 64 + j * 8 + ld_row, rows - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j)  // x is below 4 GiB (the host checks)
        a_off[j] = ((static_cast<uint32_t>(slot_id[j]) / kTopK) * static_cast<uint32_t>(K) +
                    ((j & 1) ? lc_odd : lc_even)) * 2u;
      a_base = A + kbeg * kBK;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        a_off[j] = (static_cast<uint32_t>(min(wave * 64 + j * 8 + ld_row, rows - 1 - m0)) * static_cast<uint32_t>(K) +
                    ((j & 1) ? lc_odd : lc_even)) * 2u;
      a_base = A + static_cast<int64_t>(row_begin + m0) * K + ks * k_part + kbeg * kBK;
    }
    // B: a wave's 64 weight rows are contiguous and all in range or all past
    // N (N is a multiple of 128), so clamping the block keeps them in range.
    const bf16_t* bsrc = SWIGLU ? ((wave & 1) ? B1 : B0) : B0;
    const int brow0 = min(SWIGLU ? n0 + (wave >> 1) * 64 : n0 + wave * 64, N - 64);
    const bf16_t* b_base = bsrc + (static_cast<int64_t>(e) * N + brow0) * K + ks * k_part + kbeg * kBK;
    uint32_t b_off[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      b_off[j] = (static_cast<uint32_t>(j * 8 + ld_row) * static_cast<uint32_t>(K) + ((j & 1) ? lc_odd : lc_even)) * 2u;
    // Raw buffer resources (stride 0).  A load whose offset reaches
    // num_records would read zeros, so the range covers every 32-bit offset:
    // the gathered token rows of x reach T*d*2 bytes (up to 4 GiB), and no
    // load here relies on the range check (rows are clamped, weight blocks
    // stay inside their expert).
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a_base), 0,
                                                                           kWholeRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(b_base), 0,
                                                                           kWholeRange, kBufferFlags);

    if (rows - m0 <= kThinRows) {
      // Thin tile: an expert's last m-tile with at most 32 rows.  The four
      // waves split the 256 weight rows instead (32 rows x 64 weight rows
      // each: 2 x 4 MFMA tiles), so the tile costs its loads, not 256 rows of
      // MFMAs.  With little arithmetic to hide them behind, loads run three
      // stages ahead: the weight tiles in slots 1-4 (32 KiB each), the 32
      // token rows (4 KiB per stage, wave w filling rows 8w..8w+7) in 8
      // sub-slots of slot 0.  Each stage waits for its own loads, then a
      // barrier (which also frees the slots of the stage before).
      uint32_t ta_off;
      {
        const int lc = (wave & 1) ? lc_odd : lc_even;  // swizzle of LDS row 8*wave + ld_row
        if constexpr (SWIGLU)
          ta_off = ((static_cast<uint32_t>(gather[row_begin + min(m0 + wave * 8 + ld_row, rows - 1)]) / kTopK) *
                        static_cast<uint32_t>(K) + lc) * 2u;
        else
          ta_off = (static_cast<uint32_t>(min(wave * 8 + ld_row, rows - 1 - m0)) * static_cast<uint32_t>(K) + lc) *
                   2u;
      }
      constexpr int kThinSub = kThinRows * kBK;  // elements of one token sub-slot
      constexpr int kThinLoads = 9;              // loads per wave and stage: 8 weight + 1 token
#define LOAD_THIN(KT_)                                                                                   \
  {                                                                                                      \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, LDS_PTR(&ring[1 + ((KT_) & 3)][(wave * 64 + j * 8) * kBK]), \
                                               16, b_off[j], (KT_) * (kBK * 2), 0, 0);                  \
    }                                                                                                    \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, LDS_PTR(&ring[0][((KT_) & 7) * kThinSub + (wave * 8) * kBK]), \
                                             16, ta_off, (KT_) * (kBK * 2), 0, 0);                       \
  }
      // this wave's B-tile rows: SwiGLU = 32 gate rows and the matching 32 up rows
      int tb_row[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (SWIGLU)
          tb_row[j] = (wave >> 1) * 128 + (j >= 2 ? 64 : 0) + (wave & 1) * 32 + (j & 1) * 16 + l16;
        else
          tb_row[j] = wave * 64 + j * 16 + l16;
      }
      f32x4 tacc[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) tacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int st = 0; st < 3 && st < kt_n; ++st) LOAD_THIN(st);
      for (int kt = 0; kt < kt_n; ++kt) {
        // stages kt+1 and kt+2 (if any) may stay in flight
        const int after = min(2, kt_n - 1 - kt);
        if (after == 2)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kThinLoads));
        else if (after == 1)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kThinLoads));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();  // stage kt landed for all waves; stage kt-1 fully read
        if (kt + 3 < kt_n) LOAD_THIN(kt + 3);  // into the slots of stage kt-1
        bf16x8 ta[2][2], tb[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            tb[hh][j] = *reinterpret_cast<const bf16x8*>(&ring[1 + (kt & 3)][lds_off(tb_row[j], hh * 4 + lg)]);
#pragma unroll
          for (int i = 0; i < 2; ++i)
            ta[hh][i] = *reinterpret_cast<const bf16x8*>(
                &ring[0][(kt & 7) * kThinSub + lds_off(i * 16 + l16, hh * 4 + lg)]);
        }
        __builtin_amdgcn_sched_barrier(0);  // all reads issued before the MFMAs (as the split tiles)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              tacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tb[hh][j], ta[hh][i], tacc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#undef LOAD_THIN
      // every wave's reads of the last stage are done before the next tile refills the slots
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lgkm0_mask());
      lds_barrier();
      // Epilogue: tacc[i][j][q] is row m0 + i*16 + l16, B-tile row tb_row[j]'s
      // block at 4*lg + q.
      // (the lane index re-read: address terms formed here, as in the main epilogue)
      int elane = lane;
      asm volatile("" : "+v"(elane));
      const int el16 = elane % 16, elg = elane / 16;
      if (plane) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int brow = SWIGLU ? (wave >> 1) * 128 + (j >= 2 ? 64 : 0) + (wave & 1) * 32 + (j & 1) * 16
                                    : wave * 64 + j * 16;
            const f32x4 v = tacc[i][j];
            *reinterpret_cast<float4*>(plane + (i * 16 + el16) * kBN + brow + 4 * elg) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + i * 16 + el16;
        if (m >= rows) continue;
        const int64_t orow = row_begin + m;
        if constexpr (SWIGLU) {
          bf16_t* C = static_cast<bf16_t*>(Cout);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int n = n0 + (wave >> 1) * 64 + (wave & 1) * 32 + j * 16 + 4 * elg;
            const f32x4 g = tacc[i][j];
            const f32x4 u = tacc[i][j + 2];
            uint2 p;
            p.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
            p.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
            *reinterpret_cast<uint2*>(C + orow * N + n) = p;
          }
        } else {
          float* C = static_cast<float*>(Cout) + ks * split_stride;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0 + wave * 64 + j * 16 + 4 * elg;
            if (n >= N) continue;
            const f32x4 v = tacc[i][j];
            *reinterpret_cast<float4*>(C + orow * N + n) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
      continue;
    }

    if (rows - m0 <= kSmallRows) {
      // Small tile: 33..64 rows.  As the thin tile with four row blocks
      // (64 rows x 64 weight rows per wave: 4 x 4 MFMA tiles), loads three
      // stages ahead: the weight tiles in slots 1-4, the 64 token rows (8 KiB
      // per stage, wave w filling rows 16w..16w+15) in 4 sub-slots of slot 0.
      uint32_t ta_off[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int lc = (j & 1) ? lc_odd : lc_even;  // swizzle of LDS row 16*wave + 8*j + ld_row
        if constexpr (SWIGLU)
          ta_off[j] = ((static_cast<uint32_t>(gather[row_begin + min(m0 + wave * 16 + j * 8 + ld_row, rows - 1)]) /
                        kTopK) * static_cast<uint32_t>(K) + lc) * 2u;
        else
          ta_off[j] = (static_cast<uint32_t>(min(wave * 16 + j * 8 + ld_row, rows - 1 - m0)) *
                           static_cast<uint32_t>(K) + lc) * 2u;
      }
      constexpr int kThinSub = kSmallRows * kBK;  // elements of one token sub-slot
      constexpr int kThinLoads = 10;              // loads per wave and stage: 8 weight + 2 token
#define LOAD_THIN(KT_)                                                                                   \
  {                                                                                                      \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, LDS_PTR(&ring[1 + ((KT_) & 3)][(wave * 64 + j * 8) * kBK]), \
                                               16, b_off[j], (KT_) * (kBK * 2), 0, 0);                  \
    }                                                                                                    \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc,                                                   \
                                               LDS_PTR(&ring[0][((KT_) & 3) * kThinSub + (wave * 16 + j * 8) * kBK]), \
                                               16, ta_off[j], (KT_) * (kBK * 2), 0, 0);                 \
    }                                                                                                    \
  }
      // this wave's B-tile rows: SwiGLU = 32 gate rows and the matching 32 up rows
      int tb_row[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (SWIGLU)
          tb_row[j] = (wave >> 1) * 128 + (j >= 2 ? 64 : 0) + (wave & 1) * 32 + (j & 1) * 16 + l16;
        else
          tb_row[j] = wave * 64 + j * 16 + l16;
      }
      f32x4 tacc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) tacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int st = 0; st < 3 && st < kt_n; ++st) LOAD_THIN(st);
      for (int kt = 0; kt < kt_n; ++kt) {
        // stages kt+1 and kt+2 (if any) may stay in flight
        const int after = min(2, kt_n - 1 - kt);
        if (after == 2)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kThinLoads));
        else if (after == 1)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kThinLoads));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();  // stage kt landed for all waves; stage kt-1 fully read
        if (kt + 3 < kt_n) LOAD_THIN(kt + 3);  // into the slots of stage kt-1
        bf16x8 ta[2][4], tb[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            tb[hh][j] = *reinterpret_cast<const bf16x8*>(&ring[1 + (kt & 3)][lds_off(tb_row[j], hh * 4 + lg)]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ta[hh][i] = *reinterpret_cast<const bf16x8*>(
                &ring[0][(kt & 3) * kThinSub + lds_off(i * 16 + l16, hh * 4 + lg)]);
        }
        __builtin_amdgcn_sched_barrier(0);  // all reads issued before the MFMAs (as the split tiles)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              tacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tb[hh][j], ta[hh][i], tacc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#undef LOAD_THIN
      // every wave's reads of the last stage are done before the next tile refills the slots
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lgkm0_mask());
      lds_barrier();
      // Epilogue: tacc[i][j][q] is row m0 + i*16 + l16, B-tile row tb_row[j]'s
      // block at 4*lg + q.
      // (the lane index re-read: address terms formed here, as in the main epilogue)
      int elane = lane;
      asm volatile("" : "+v"(elane));
      const int el16 = elane % 16, elg = elane / 16;
      if (plane) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int brow = SWIGLU ? (wave >> 1) * 128 + (j >= 2 ? 64 : 0) + (wave & 1) * 32 + (j & 1) * 16
                                    : wave * 64 + j * 16;
            const f32x4 v = tacc[i][j];
            *reinterpret_cast<float4*>(plane + (i * 16 + el16) * kBN + brow + 4 * elg) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + i * 16 + el16;
        if (m >= rows) continue;
        const int64_t orow = row_begin + m;
        if constexpr (SWIGLU) {
          bf16_t* C = static_cast<bf16_t*>(Cout);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int n = n0 + (wave >> 1) * 64 + (wave & 1) * 32 + j * 16 + 4 * elg;
            const f32x4 g = tacc[i][j];
            const f32x4 u = tacc[i][j + 2];
            uint2 p;
            p.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
            p.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
            *reinterpret_cast<uint2*>(C + orow * N + n) = p;
          }
        } else {
          float* C = static_cast<float*>(Cout) + ks * split_stride;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0 + wave * 64 + j * 16 + 4 * elg;
            if (n >= N) continue;
            const f32x4 v = tacc[i][j];
            *reinterpret_cast<float4*>(C + orow * N + n) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
      continue;
    }

    if (rows - m0 <= kMediumRows) {
      medium_tile<SWIGLU>(ring, a_rsrc, b_rsrc, b_off, gather, row_begin, rows, m0, n0, K, N, wave, lane, lc_even,
                          lc_odd, kt_n, plane, Cout, ks, split_stride);
      continue;
    }

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa0[8], fb0[8], fa1[8], fb1[8];

    // Prologue: stages 0 and 1 (A and B); the steady state then keeps one A
    // stage and two B stages in flight.
#pragma unroll
    for (int j = 0; j < 8; ++j) { LOAD_A(0, j); LOAD_B(0, j, 0); }
#pragma unroll
    for (int j = 0; j < 8; ++j) { LOAD_B(1, j, 1); }
#pragma unroll
    for (int j = 0; j < 8; ++j) { LOAD_A(1, j); }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));  // this wave's stage-0 loads landed
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 8; ++q) { READ_PAIR(fa0, fb0, 0, 0, 0, q); }
    int kt = 0, bs = 0;
    for (; kt < kt_n - 2; ++kt) {
      const int bs1 = bs == 2 ? 0 : bs + 1;
      const int bs2 = bs1 == 2 ? 0 : bs1 + 1;
      STAGE(kt, bs, bs1, bs2, true, true);
      bs = bs1;
    }
    {
      const int bs1 = bs == 2 ? 0 : bs + 1;
      STAGE(kt, bs, bs1, 0, false, true);
      ++kt;
      bs = bs1;
    }
    // The last stage's barrier also orders every wave's final reads before
    // the next tile's prologue refills the slots.
    STAGE(kt, bs, 0, 0, false, false);

    // Epilogue.  acc[i][j][q]: output row m0 + wm*128 + i*16 + l16, B-tile
    // row wn*128 + j*16 + 4*lg + q (the B rows were MFMA src0).
    // A piece stores its raw partial tile instead (plane row = tile row,
    // plane column = B-tile row).  The lane index is re-read here so that
    // the epilogue's per-lane address terms are formed per tile, not kept
    // live across the main loop.
    int elane = lane;
    asm volatile("" : "+v"(elane));
    const int el16 = elane % 16, elg = elane / 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int m = m0 + wm * 128 + i * 16 + el16;
      if (m >= rows) continue;
      const int64_t orow = row_begin + m;
      float* prow = plane + (m - m0) * kBN + wn * 128 + 4 * elg;  // used only by a piece
      if constexpr (SWIGLU) {
        bf16_t* C = static_cast<bf16_t*>(Cout);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + 4 * elg;
          const f32x4 g = acc[i][j];
          const f32x4 u = acc[i][j + 4];
          if (plane) {
            *reinterpret_cast<float4*>(prow + j * 16) = make_float4(g[0], g[1], g[2], g[3]);
            *reinterpret_cast<float4*>(prow + (j + 4) * 16) = make_float4(u[0], u[1], u[2], u[3]);
          } else {
            uint2 p;
            p.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
            p.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
            *reinterpret_cast<uint2*>(C + orow * N + n) = p;
          }
        }
      } else {
        float* C = static_cast<float*>(Cout) + ks * split_stride;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + wn * 128 + j * 16 + 4 * elg;
          if (n >= N) continue;
          const f32x4 v = acc[i][j];
          *reinterpret_cast<float4*>(plane ? prow + j * 16 : C + orow * N + n) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
  if constexpr (CLOCKED) {
    const long long cyc1 = __builtin_amdgcn_s_memtime();
    const long long ref1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
      long long* c = clk + 4 * static_cast<int64_t>(blockIdx.x);
      c[0] = cyc0;
      c[1] = cyc1;
      c[2] = ref0;
      c[3] = ref1;
    }
  }
}

// Sum over parts p = 0..P-1 of src[p * stride .. +3] (or +1), added in part
// order; the loads of up to kPartBatch parts are issued before any add, so
// a row costs one memory latency per batch rather than one per part.
constexpr int kPartBatch = 8;
__device__ __forceinline__ float4 sum_parts4(const float* src, int64_t stride, int P) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < P; p0 += kPartBatch) {
    float4 v[kPartBatch];
#pragma unroll
    for (int j = 0; j < kPartBatch; ++j)
      v[j] = p0 + j < P ? *reinterpret_cast<const float4*>(src + (p0 + j) * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kPartBatch; ++j) {
      if (p0 + j < P) {
        a.x += v[j].x;
        a.y += v[j].y;
        a.z += v[j].z;
        a.w += v[j].w;
      }
    }
  }
  return a;
}
__device__ __forceinline__ float2 sum_parts2(const float* src, int64_t stride, int P) {
  float2 a = make_float2(0.f, 0.f);
  for (int p0 = 0; p0 < P; p0 += kPartBatch) {
    float2 v[kPartBatch];
#pragma unroll
    for (int j = 0; j < kPartBatch; ++j)
      v[j] = p0 + j < P ? *reinterpret_cast<const float2*>(src + (p0 + j) * stride) : make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kPartBatch; ++j) {
      if (p0 + j < P) {
        a.x += v[j].x;
        a.y += v[j].y;
      }
    }
  }
  return a;
}

// Adds the partial tiles of the remainder units (see remainder_split) in
// part order and applies the epilogue the GEMM applies to a whole unit:
// SiLU(gate) * up and one bf16 rounding (up projection) or an fp32 store
// (down projection).  The split is recomputed from the offsets with the
// GEMM's grid size, stage count and plane count.  One wave per output row.
// Down projection only: with tail_part, also the split tails' partial sums
// (layout in launch.hpp): each tail row of y_rows = the sum of its P parts
// in part order.
template <bool SWIGLU>
__global__ void __launch_bounds__(kThreads) remainder_fixup_kernel(const int32_t* __restrict__ offs,
                                                                   const float* __restrict__ partials,
                                                                   void* __restrict__ Cout, int N, int K,
                                                                   int gemm_grid, int planes, int thin_elsewhere,
                                                                   const float* __restrict__ tail_part) {
  constexpr int TN = SWIGLU ? kBN / 2 : kBN;
  constexpr int kWavesPerBlock = kThreads / kWave;
  const int n_tiles_n = (N + TN - 1) / TN;
  int n_full, n_thin;
  unit_counts<1>(offs, n_tiles_n, &n_full, &n_thin);
  if (thin_elsewhere) n_thin = 0;
  const RemSplit rs = remainder_split(n_full, gemm_grid, K / kBK, planes, partials != nullptr && n_thin == 0);
  const int tail_parts = (!SWIGLU && tail_part) ? *reinterpret_cast<const int*>(tail_part) : 1;
  constexpr int kTailChunk = 4 * 4 * kWave;  // columns per tail item (4 float4 per lane)
  const int tail_chunks = (N + kTailChunk - 1) / kTailChunk;
  const int tail_items = tail_parts > 1 ? kExperts * kTailPartRows * tail_chunks : 0;
  if (rs.rem == 0 && tail_items == 0) return;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int64_t part_stride = static_cast<int64_t>(rs.rem) * kPlaneElems;
  const int items = rs.rem * kBM + tail_items;
  for (int item = blockIdx.x * kWavesPerBlock + wave; item < items; item += gridDim.x * kWavesPerBlock) {
    if (item >= rs.rem * kBM) {  // columns [ch*kTailChunk, +kTailChunk) of row m of expert e's split tail
      const int t0 = item - rs.rem * kBM;
      const int ch = t0 % tail_chunks, t = t0 / tail_chunks;
      const int e = t / kTailPartRows, m = t % kTailPartRows;
      int fm;
      bool thin;
      expert_shape(offs, e, &fm, &thin);
      const int row0 = offs[e] + fm * kBM;  // the tail's first row
      if (!thin || row0 + m >= offs[e + 1]) continue;
      const float* src = tail_part + kTailPartHeader + static_cast<int64_t>(e * kTailPartRows + m) * N;
      const int64_t pstride = static_cast<int64_t>(kExperts) * kTailPartRows * N;
      float* dst = static_cast<float*>(Cout) + static_cast<int64_t>(row0 + m) * N;
      const int c_end = min(N, (ch + 1) * kTailChunk);
#pragma unroll 4
      for (int c = ch * kTailChunk + 4 * lane; c < c_end; c += 4 * kWave)
        *reinterpret_cast<float4*>(dst + c) = sum_parts4(src + c, pstride, tail_parts);
      continue;
    }
    const int r = item / kBM, m = item % kBM;
    int e, mt, nt, ks;
    full_unit<1>(offs, n_tiles_n, rs.n_main + r, &e, &mt, &nt, &ks);
    const int row_begin = offs[e];
    const int rows = offs[e + 1] - row_begin;
    const int m0 = mt * kBM;
    if (m0 + m >= rows) continue;
    const int n0 = nt * TN;
    const int64_t orow = row_begin + m0 + m;
    const float* src = partials + static_cast<int64_t>(r) * kPlaneElems + m * kBN;
    if constexpr (SWIGLU) {
      // output columns n0 + c, c + 1: gate sums at B-tile row (c/64)*128 + c%64, up sums 64 rows on
      const int c = 2 * lane;
      const int b = (c / 64) * 128 + c % 64;
      const float2 g = sum_parts2(src + b, part_stride, rs.parts);
      const float2 u = sum_parts2(src + b + 64, part_stride, rs.parts);
      bf16_t* C = static_cast<bf16_t*>(Cout);
      *reinterpret_cast<uint32_t*>(C + orow * N + n0 + c) = pack_bf16x2(silu(g.x) * u.x, silu(g.y) * u.y);
    } else {
      const int c = 4 * lane;
      if (n0 + c >= N) continue;
      *reinterpret_cast<float4*>(static_cast<float*>(Cout) + orow * N + n0 + c) =
          sum_parts4(src + c, part_stride, rs.parts);
    }
  }
}

// Planes of the partial buffer (0 when there is none).
int plane_count(const float* partials, int64_t partial_bytes) {
  if (!partials) return 0;
  const int64_t n = partial_bytes / (static_cast<int64_t>(kPlaneElems) * 4);
  return n > (1 << 20) ? (1 << 20) : static_cast<int>(n);
}

#undef LOAD_A
#undef LOAD_B
#undef READ_B
#undef READ_A
#undef READ_PAIR
#undef MFMA_QROW
#undef READ_ONE
#undef STAGE

}  // namespace

bool prefill_fits(int64_t T, int d, int f) {
  // K/split a multiple of 64 and at least two stages; gathered token rows
  // addressed with 32-bit byte offsets.
  return d % 128 == 0 && f % 128 == 0 && d >= 256 && f >= 256 && T * d * 2 < (int64_t{1} << 32);
}

int prefill_grid(int n_cu) { return (n_cu / kXcds) * kXcds; }

hipError_t launch_up_prefill(const bf16_t* x, const int32_t* offs, const int32_t* sorted_slots, const bf16_t* w1,
                             const bf16_t* w3, bf16_t* h, int d, int f, int n_cu, bool thin_elsewhere,
                             float* partials, int64_t partial_bytes, hipStream_t s, long long* clk,
                             hipEvent_t after_gemm) {
  const int grid = prefill_grid(n_cu);
  const int planes = plane_count(partials, partial_bytes);
  float* part = planes >= 2 ? partials : nullptr;
  if (clk)
    hipLaunchKernelGGL((grouped_gemm_prefill_kernel<true, 1, true>), dim3(grid), dim3(kThreads), 0, s, x, sorted_slots,
                       offs, w1, w3, static_cast<void*>(h), f, d, int64_t{0}, thin_elsewhere ? 1 : 0, part, planes,
                       clk);
  else
    hipLaunchKernelGGL((grouped_gemm_prefill_kernel<true, 1, false>), dim3(grid), dim3(kThreads), 0, s, x,
                       sorted_slots, offs, w1, w3, static_cast<void*>(h), f, d, int64_t{0}, thin_elsewhere ? 1 : 0,
                       part, planes, static_cast<long long*>(nullptr));
  if (after_gemm) {
    const hipError_t err = hipEventRecord(after_gemm, s);
    if (err != hipSuccess) return err;
  }
  if (part)
    hipLaunchKernelGGL((remainder_fixup_kernel<true>), dim3(2 * grid), dim3(kThreads), 0, s, offs,
                       static_cast<const float*>(part), static_cast<void*>(h), f, d, grid, planes,
                       thin_elsewhere ? 1 : 0, static_cast<const float*>(nullptr));
  return hipGetLastError();
}

hipError_t launch_down_prefill(const bf16_t* h, const int32_t* offs, const bf16_t* w2, float* y_rows, int d, int f,
                               int n_cu, int split, int64_t split_stride, bool thin_elsewhere, float* partials,
                               int64_t partial_bytes, hipStream_t s) {
  const int grid = prefill_grid(n_cu);
  // each work unit needs K/split to be a multiple of 64 and at least 2 stages
  if (split == 2 && f % 128 == 0 && f / 2 >= 2 * kBK) {
    hipLaunchKernelGGL((grouped_gemm_prefill_kernel<false, 2, false>), dim3(grid), dim3(kThreads), 0, s, h,
                       static_cast<const int32_t*>(nullptr), offs, w2, static_cast<const bf16_t*>(nullptr),
                       static_cast<void*>(y_rows), d, f, split_stride, thin_elsewhere ? 1 : 0,
                       static_cast<float*>(nullptr), 0, static_cast<long long*>(nullptr));
  } else {
    const int planes = plane_count(partials, partial_bytes);
    float* part = planes >= 2 ? partials : nullptr;
    hipLaunchKernelGGL((grouped_gemm_prefill_kernel<false, 1, false>), dim3(grid), dim3(kThreads), 0, s, h,
                       static_cast<const int32_t*>(nullptr), offs, w2, static_cast<const bf16_t*>(nullptr),
                       static_cast<void*>(y_rows), d, f, int64_t{0}, thin_elsewhere ? 1 : 0, part, planes,
                       static_cast<long long*>(nullptr));
  }
  return hipGetLastError();
}

hipError_t launch_down_prefill_fixup(const int32_t* offs, const float* partials, int64_t partial_bytes,
                                     const float* tail_part, float* y_rows, int d, int f, int n_cu,
                                     bool thin_elsewhere, hipStream_t s) {
  const int grid = (n_cu / kXcds) * kXcds;
  const int planes = plane_count(partials, partial_bytes);
  const float* part = planes >= 2 ? partials : nullptr;
  if (!part && !tail_part) return hipSuccess;
  hipLaunchKernelGGL((remainder_fixup_kernel<false>), dim3(2 * grid), dim3(kThreads), 0, s, offs, part,
                     static_cast<void*>(y_rows), d, f, grid, planes, thin_elsewhere ? 1 : 0, tail_part);
  return hipGetLastError();
}

}  // namespace moe
