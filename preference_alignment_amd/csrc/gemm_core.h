// bf16 MFMA main loop shared by the four LM-head contractions (gfx950).
//
// C[i][j] = sum_k R[i][k] * C[j][k].  An operand is either ROW (its tile rows
// are K-contiguous in memory) or K-MAJOR (contiguous along the MFMA dimension,
// read through transposing LDS reads).  The kernels that use this core differ
// in their operands and epilogues:
//   forward / recompute : R = W_vocab rows, C = hidden rows at completion positions
//   dHidden             : R = D rows (K = vocabulary), C = W_vocab read K-major
//   dW_vocab (as dW^T)  : R = gathered hidden^T rows (K = positions), C = D read K-major
//
// Block tile 256x256x64, 512 threads = 8 waves in a 2x4 grid (two waves per
// SIMD, so one wave's LDS and barrier waits are covered by the other's MFMAs);
// each wave owns a 128x64 sub-tile held as 8x4 fragments of
// v_mfma_f32_16x16x32_bf16 (128 accumulator registers).  With random bf16
// data the part runs power-limited, and the 16x16x32 form moves half the
// accumulator bytes per flop of the 32x32x16 one: the same loop built on
// 32x32x16 sustained ~1.8 GHz and ran 5-8 % slower than this one (~2.0 GHz).
// Operand tiles go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds (16 bytes per lane, no register staging; the
// flat global_load_lds form also counts on the LDS counter, which forces the
// compiler to wait for every fragment read), double buffered (2 stages x 2 operands x
// 32 KiB = 128 KiB of the 160 KiB LDS).  A stage (64 K values) is two 32-wide
// K steps.  The loop is software pipelined one step ahead: while the MFMAs of
// one step issue row by row, each fragment of the next step is read into the
// registers of a fragment the current step has finished with, and the stage
// barrier sits after the first row of a stage's second step.
//
// Both loads place lane L's 16 bytes at (wave base + 16 L), so the LDS
// swizzles below are realised by choosing which global chunk each lane fetches.
//
// MFMA 16x16x32 register layout (CDNA4): lane l supplies A[l % 16][8 (l / 16)
// + 0..7] and B^T likewise; accumulator element e of lane l is
// C[4 (l / 16) + e][l % 16].  The K permutation inside a fragment is
// irrelevant (A and B use the same one); the C layout is what the epilogues
// rely on.
#pragma once

#include "dpo_common.h"

namespace dpo {
namespace gemm {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 512;
constexpr int WAVES_N = 4;             // waves along the MFMA columns
constexpr int FRAG = 16;               // rows / columns of one MFMA fragment
constexpr int FM = 8;                  // row fragments per wave (128 rows)
constexpr int FN = 4;                  // column fragments per wave (64 cols)
constexpr int ACC_N = 4;               // accumulator elements per lane and fragment
constexpr int WAVE_COLS = FRAG * FN;
constexpr int OPER_BYTES = BM * BK * 2;       // 32 KiB
constexpr int STAGE_BYTES = 2 * OPER_BYTES;   // A + B
constexpr int PIPE_BYTES = 2 * STAGE_BYTES;   // double buffer, 128 KiB
constexpr int LOADS_PER_THREAD = BM * (BK / 8) / NTHREADS;  // 4 rows per operand
constexpr int LOADER_ROW_STRIDE = NTHREADS / 8;             // 64
constexpr int NUM_XCD = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The two pipeline stage buffers are distinct LDS objects.  The main loop is
// unrolled over the pair, so every access names its buffer statically, and
// the compiler can tell the direct-to-LDS loads into one buffer from reads
// of the other: it then never waits for a stage's loads before a read of the
// other stage (it did before transposing reads when both buffers were
// offsets into one array).  The epilogues reuse the pair as staging space.
static __shared__ __attribute__((aligned(16))) char g_stage0[STAGE_BYTES];
static __shared__ __attribute__((aligned(16))) char g_stage1[STAGE_BYTES];
#define DPO_STG(b_) ((b_) ? g_stage1 : g_stage0)
// LDS byte address of a stage buffer (a constant once the kernel is laid out)
#define DPO_STG_LDS(b_) ((unsigned)(size_t)(lds_ptr_t)DPO_STG(b_))

struct Acc {
  floatx4 c[FM][FN];
};

// LDS layout of an operand tile (rows of the MFMA dimension, 64 K values
// each): 256 rows x 128 bytes; the 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7).  Fragments are single ds_read_b128.

// ROW operands are read with buffer_load_dwordx4 ... lds: one uniform buffer
// descriptor, a 32-bit byte offset per lane and loaded row (fixed for the
// tile), and the K step in the scalar offset.  Offsets at or beyond the
// descriptor's size read as zero, which is how ragged tiles are padded.
// Buffer resource of an operand (raw buffer, no stride): base address, its
// size in bytes (reads at or past it return zero) and the format flags.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

struct RowOperand {
  i32x4_t rsrc;
  unsigned voff[LOADS_PER_THREAD];  // byte offset of (row, lchunk * 8) at K = 0
};

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit dwords

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, size_t bytes) {
  const unsigned long long b = (unsigned long long)(size_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)min(bytes, (size_t)0xFFFFFFFFu));
  r[3] = kBufferFlags;
  return r;
}

// One 16-byte-per-lane direct-to-LDS load: lane L's 16 bytes land at
// lds_wave + 16 L.  It is issued through inline assembly so that the compiler
// does not track it: otherwise it waits for a stage's loads before reads of
// the other stage whose aliasing it cannot rule out (it did before every
// transposing read), while the loop's own stage barrier already waits for
// them (vmcnt(0)) before any read of that stage.  The load writes no
// register; its LDS destination is read only after that barrier.
__device__ __forceinline__ void dma16(const i32x4_t& rsrc, unsigned lds_wave, unsigned voff, unsigned soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_wave), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// Operand whose tile rows are consecutive rows of a row-major matrix:
// `base` = first row of the tile, `ld` = elements per row, `rows_left` = rows
// that exist from `base` on, `k0` = first K element.
__device__ __forceinline__ RowOperand row_operand(const uint16_t* base, size_t ld, long rows_left, int k0,
                                                  int tid) {
  RowOperand op;
  const size_t bytes = (size_t)max(rows_left, 0L) * ld * 2;
  op.rsrc = buffer_rsrc(base, bytes);
  const int lchunk = (tid & 7) ^ ((tid >> 4) & 7);
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it)
    op.voff[it] = (unsigned)(((size_t)(it * LOADER_ROW_STRIDE + (tid >> 3)) * ld + k0 + lchunk * 8) * 2);
  return op;
}
__device__ __forceinline__ int row_lchunk(int tid) { return (tid & 7) ^ ((tid >> 4) & 7); }
__device__ __forceinline__ int row_loader_row(int it, int tid) { return it * LOADER_ROW_STRIDE + (tid >> 3); }

__device__ __forceinline__ void load_stage(const RowOperand& op, int kstep, unsigned lds_tile, int wave) {
  const unsigned soff = __builtin_amdgcn_readfirstlane((unsigned)kstep * BK * 2);
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it) dma16(op.rsrc, lds_tile + (it * NTHREADS + wave * 64) * 16, op.voff[it], soff);
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// K-MAJOR operands are contiguous along the MFMA dimension (rows of memory =
// K): a tile is 64 K rows x 512 bytes (256 values).  The 16-byte chunk c of K
// row k sits at chunk c ^ kswz(k).  Each 16-lane group of a transposing
// fragment read touches 4 K rows x 2 chunks, and the two groups of a
// half-wave rows 8 apart; kswz gives those 8 rows 8 distinct even XOR values
// below 16, so the 16 chunks a half-wave reads fall in distinct banks.
__device__ __forceinline__ int kswz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }

// Loader of a K-major operand: `base` = element (K row 0, MN column 0) of
// the tile, `ld` = elements per K row, `k_rows` = K rows that exist from base
// on (rows past them read as zero through the descriptor's size).  The K step
// is added to the per-lane offset (not the scalar one) so that every access
// stays inside the descriptor's range check.
struct KOperand {
  i32x4_t rsrc;
  unsigned voff[LOADS_PER_THREAD];  // byte offset of (K row, chunk) at K step 0
  unsigned step;                    // bytes per K step of BK rows
};

__device__ __forceinline__ KOperand kmajor_operand(const uint16_t* base, size_t ld, long k_rows, int tid) {
  KOperand op;
  const size_t bytes = (size_t)max(k_rows, 0L) * ld * 2;
  op.rsrc = buffer_rsrc(base, bytes);
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it) {
    const int k = it * (NTHREADS / 32) + (tid >> 5);
    const int c = (tid & 31) ^ kswz(k);
    op.voff[it] = (unsigned)(((size_t)k * ld + c * 8) * 2);
  }
  op.step = (unsigned)((size_t)BK * ld * 2);
  return op;
}

__device__ __forceinline__ void load_stage(const KOperand& op, int kstep, unsigned lds_tile, int wave) {
  const unsigned koff = (unsigned)kstep * op.step;
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it)
    dma16(op.rsrc, lds_tile + (it * NTHREADS + wave * 64) * 16, op.voff[it] + koff, 0);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr;

// Fragment reader.  `f` = fragment index along the MFMA dimension (16 wide),
// `base` = first MFMA row/column of this wave inside the tile, s = 32-wide K
// step inside the stage.  Lanes 16 q .. 16 q + 15 read the 16-byte chunk
// 4 s + q of 16 consecutive rows: with the swizzle above, each group of 16
// lanes covers all 64 banks once.
struct RowFrag {
  int off[2];  // byte offset of (row, chunk of step s) for fragment 0
  __device__ __forceinline__ void init(int base, int lane) {
    const int sw = ((lane & 15) >> 1) & 7;
#pragma unroll
    for (int s = 0; s < 2; ++s) off[s] = (base + (lane & 15)) * 128 + (((4 * s + (lane >> 4)) ^ sw) << 4);
  }
  __device__ __forceinline__ bf16x8_t read(const char* tile, int f, int s) const {
    return *(const bf16x8_t*)(tile + off[s] + f * FRAG * 128);
  }
};

// Fragment reader of a K-major tile through ds_read_b64_tr_b16 (gfx950).  In
// a 16-lane group the transposing read hands lane i element (i & 3) of the
// 8-byte piece that lane 4 k + (i >> 2) addresses, for k = 0..3.  Lane L of
// group g therefore addresses K row 8 g + (L >> 2) (+ 4 for the second
// read), MFMA columns base + 16 f + 4 (L & 3) .. +3, and receives the K
// values 8 g + 0..3 (then + 4..7) of column base + 16 f + (L & 15): the MFMA
// operand layout.  A fragment's chunk is fragment 0's XOR 2 f (base is a
// multiple of 64 and the swizzle only moves chunks within 16-chunk blocks),
// so one offset per lane serves every fragment.
struct TrFrag {
  int off;  // byte offset of fragment 0's first read at step 0
  __device__ __forceinline__ void init(int base, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const int k = 8 * g + (L >> 2);
    const int mn = base + 4 * (L & 3);
    off = k * 512 + (((mn >> 3) ^ kswz(k)) << 4) + ((mn & 7) << 1);
  }
  __device__ __forceinline__ bf16x8_t read(const char* tile, int f, int s) const {
    const char* p = tile + (off ^ (f << 5)) + s * (32 * 512);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 4 * 512));
    const short __attribute__((ext_vector_type(8))) v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// fragment reader and LDS reads per fragment of each operand kind
template <typename Op>
struct FragOf {
  typedef RowFrag type;
  static constexpr int reads = 1;
};
template <>
struct FragOf<KOperand> {
  typedef TrFrag type;
  static constexpr int reads = 2;
};

// The K loop over nk steps of BK.  nk may be 0 (accumulators stay zero).  The
// R operand supplies the MFMA rows (wave (wm, wn) owns rows wm*128 .. +128),
// the C operand the MFMA columns (columns wn*64 .. +64).
//
// Fragments live in two slots; a step's MFMAs run row by row (row i = the FN
// MFMAs that use A_i), and right behind row i the next step's B_i (i < FN)
// and A_i are read into the other slot, so A is held about once and only B
// twice (128 accumulator + ~72 fragment registers).  Each row is a scheduling
// region of its own with a fixed MFMA / LDS-read interleave.  Per stage: step
// 0 on slot 0 (reading step 1 into slot 1); row 0 of step 1; the stage
// barrier (the next stage's tiles have landed, every wave is done reading
// this stage's buffer); the loads two stages ahead into that buffer; rows
// 1..7 of step 1, reading the next stage's step 0 into slot 0.  On the last
// stage those reads fetch unused values from the idle buffer, which keeps
// the loop free of branches inside the MFMA stream.  The loop body is
// written twice, once per buffer of the pair.
//
// mainloop() issues a tile's first stage, waits for it, issues the second
// and runs the loop.  A kernel whose epilogue leaves the stage buffers alone
// can instead issue the next tile's first two stages with mainloop_issue()
// as soon as mainloop_prefetched() has returned (every wave is then done
// reading them), so that their loads land while the epilogue runs.
template <typename ROp, typename COp>
__device__ __forceinline__ void mainloop_issue(const ROp& rop, const COp& cop, int nk, int wave) {
  if (nk <= 0) return;
  load_stage(rop, 0, DPO_STG_LDS(0), wave);
  load_stage(cop, 0, DPO_STG_LDS(0) + OPER_BYTES, wave);
  if (nk > 1) {
    load_stage(rop, 1, DPO_STG_LDS(1), wave);
    load_stage(cop, 1, DPO_STG_LDS(1) + OPER_BYTES, wave);
  }
}
// PRE: the first two stages were issued by mainloop_issue()
template <bool PRE, typename ROp, typename COp>
__device__ __forceinline__ void mainloop_impl(Acc& acc, const ROp& rop, const COp& cop, int nk, int wave, int lane,
                                              int wm, int wn) {
  static_assert(FN <= FM, "B fragments are read behind the first FN rows");
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < ACC_N; ++e) acc.c[i][j][e] = 0.f;
  if (nk <= 0) return;

  typename FragOf<ROp>::type rf;
  typename FragOf<COp>::type cf;
  constexpr int RA = FragOf<ROp>::reads, RB = FragOf<COp>::reads;
  rf.init(wm * 128, lane);
  cf.init(wn * WAVE_COLS, lane);
  bf16x8_t fa[2][FM], fb[2][FN];
#define DPO_RD_A(buf_, s_, slot_, i_) fa[slot_][i_] = rf.read(DPO_STG(buf_), i_, s_)
#define DPO_RD_B(buf_, s_, slot_, j_) fb[slot_][j_] = cf.read(DPO_STG(buf_) + OPER_BYTES, j_, s_)
#define DPO_ROW(slot_, i_, buf_, s_)                                                                      \
  do {                                                                                                    \
    _Pragma("unroll") for (int j_ = 0; j_ < FN; ++j_) acc.c[i_][j_] =                                     \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot_][i_], fb[slot_][j_], acc.c[i_][j_], 0, 0, 0);    \
    if ((i_) < FN) DPO_RD_B(buf_, s_, (slot_) ^ 1, i_);                                                   \
    DPO_RD_A(buf_, s_, (slot_) ^ 1, i_);                                                                  \
    if ((i_) < FN) {                                                                                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);                                                 \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);                                                 \
    } else {                                                                                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);                                                 \
    }                                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                                    \
  } while (0)
  // one stage held in buffer cur_ (K step kt_): step 0 on slot 0 (reading
  // step 1 into slot 1), row 0 of step 1, the stage barrier, the loads two
  // stages ahead into buffer cur_, rows 1..7 of step 1 (reading the next
  // stage's step 0 from the other buffer into slot 0)
#define DPO_STAGE(cur_, kt_)                                                                              \
  do {                                                                                                    \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) DPO_ROW(0, i, cur_, 1);                                \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) acc.c[0][j] =                                          \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[1][0], fb[1][j], acc.c[0][j], 0, 0, 0);                \
    __builtin_amdgcn_sched_barrier(0);                                                                    \
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");                                           \
    __builtin_amdgcn_s_barrier();                                                                         \
    if ((kt_) + 2 < nk) {                                                                                 \
      load_stage(rop, (kt_) + 2, DPO_STG_LDS(cur_), wave);                                                \
      load_stage(cop, (kt_) + 2, DPO_STG_LDS(cur_) + OPER_BYTES, wave);                                   \
    }                                                                                                     \
    DPO_RD_B((cur_) ^ 1, 0, 0, 0);                                                                        \
    DPO_RD_A((cur_) ^ 1, 0, 0, 0);                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                                    \
    _Pragma("unroll") for (int i = 1; i < FM; ++i) DPO_ROW(1, i, (cur_) ^ 1, 0);                          \
  } while (0)

  if (!PRE) {
    load_stage(rop, 0, DPO_STG_LDS(0), wave);
    load_stage(cop, 0, DPO_STG_LDS(0) + OPER_BYTES, wave);
  }
  wait_loads();
  __syncthreads();
  if (!PRE && nk > 1) {
    load_stage(rop, 1, DPO_STG_LDS(1), wave);
    load_stage(cop, 1, DPO_STG_LDS(1) + OPER_BYTES, wave);
  }
  // the loop's own read order (B_i, A_i, ...), all landed before the loop: the
  // compiler's wait counts at the loop head then follow the loop's reads only
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i < FN) DPO_RD_B(0, 0, 0, i);
    DPO_RD_A(0, 0, 0, i);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  for (int kt = 0; kt < nk; kt += 2) {
    DPO_STAGE(0, kt);
    if (kt + 1 >= nk) break;
    DPO_STAGE(1, kt + 1);
  }
#undef DPO_STAGE
#undef DPO_ROW
#undef DPO_RD_B
#undef DPO_RD_A
  // every wave is done with the LDS tiles before the caller reuses them
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
}
template <typename ROp, typename COp>
__device__ __forceinline__ void mainloop(Acc& acc, const ROp& rop, const COp& cop, int nk, int wave, int lane,
                                         int wm, int wn) {
  mainloop_impl<false>(acc, rop, cop, nk, wave, lane, wm, wn);
}
template <typename ROp, typename COp>
__device__ __forceinline__ void mainloop_prefetched(Acc& acc, const ROp& rop, const COp& cop, int nk, int wave,
                                                    int lane, int wm, int wn) {
  mainloop_impl<true>(acc, rop, cop, nk, wave, lane, wm, wn);
}

// Row (within the 256-row block tile) and column (within the 256-col tile) of
// accumulator element e of fragment (i, j) for this lane.
__device__ __forceinline__ int acc_row(int wm, int i, int e, int lane) {
  return wm * 128 + i * FRAG + 4 * (lane >> 4) + e;
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * WAVE_COLS + j * FRAG + (lane & 15); }

// The dHidden contraction has few output tiles (positions x H), so K (the
// slice's vocabulary) is split to fill the CUs: the split count minimises
// rounds of tiles over the grid times K steps per tile (ties to fewer parts),
// among the counts whose slabs (align(n_c, 256) x H floats each) fit in the
// 2 Mp x H floats the workspace holds.  It depends on N_c, which only the
// device knows; the finish recomputes it.
__host__ __device__ inline int dh_splits(int n_c, int H, int nkt, int grid, int max_split, int Mp) {
  const int mt = cdiv(n_c, BM);
  const long tiles = (long)mt * cdiv(H, BN);
  const long cap = mt > 0 ? (2L * Mp) / ((long)mt * BM) : max_split;
  int best = 1;
  long best_cost = -1;
  for (int s = 1; s <= max_split && s <= (nkt > 1 ? nkt : 1) && s <= cap; ++s) {
    const long cost = (tiles * s + grid - 1) / grid * cdiv(nkt, s);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

// slab ks of the dHidden partial sums: align(n_c, BM) rows of H floats each
__host__ __device__ inline size_t dh_slab(int n_c, int H) { return (size_t)cdiv(n_c, BM) * BM * H; }

// Persistent tile scheduler.  Tiles are numbered in grouped order and the
// numbering is cut into NUM_XCD contiguous parts; the blocks resident on one
// XCD (blockIdx % NUM_XCD) walk their part together, so tiles that share
// operand rows run at the same time on the same L2.  Two group shapes:
//   m-grouped (gn = 0): groups of gm m-tiles, m fastest, then n;
//   n-grouped (gn > 0): groups of gn n-tiles, n fastest, then m.
// With n-grouping each XCD's part is a contiguous range of n-tiles over all
// m-tiles, so every n-side operand row is fetched from HBM by one XCD only
// and the m-side operand must stay in the Infinity Cache.
struct Sched {
  int nMt, nNt, total, gm, gn;
  int begin, end, step;
  __device__ __forceinline__ void init(int nMt_, int nNt_, int gm_, int gn_ = 0) {
    nMt = nMt_;
    nNt = nNt_;
    total = nMt * nNt;
    gm = gm_ < 1 ? 1 : gm_;
    gn = gn_ < 0 ? 0 : gn_;
    const int xcd = blockIdx.x % NUM_XCD;
    const int q = blockIdx.x / NUM_XCD;
    const int part = cdiv(total, NUM_XCD);
    step = (gridDim.x - xcd + NUM_XCD - 1) / NUM_XCD;  // blocks on this XCD
    begin = xcd * part + q;
    end = min(total, (xcd + 1) * part);
  }
  __device__ __forceinline__ void coords(int t, int& mt, int& nt) const {
    if (gn > 0) {
      const int per_group = gn * nMt;
      const int g = t / per_group;
      const int first = g * gn;
      const int gs = min(nNt - first, gn);
      const int r = t - g * per_group;
      nt = first + r % gs;
      mt = r / gs;
      return;
    }
    const int per_group = gm * nNt;
    const int g = t / per_group;
    const int first = g * gm;
    const int gs = min(nMt - first, gm);
    const int r = t - g * per_group;
    mt = first + r % gs;
    nt = r / gs;
  }
};

}  // namespace gemm
}  // namespace dpo
