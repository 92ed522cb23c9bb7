// bf16 MFMA main loop shared by the four LM-head contractions (gfx950).
//
// C[i][j] = sum_k R[i][k] * C[j][k]: both operands are K-contiguous in memory.
// The kernels that use this core differ in their operands and epilogues:
//   forward / recompute : R = W_vocab rows, C = hidden rows at completion positions
//   dHidden             : R = D rows (K = vocabulary), C = W_vocab^T rows
//   dW_vocab            : R = D^T rows (K = positions), C = gathered hidden^T rows
// (the backward writes D^T and W^T so that every operand is K-contiguous: an
// LDS-transposed read of D for dW_vocab measured 40 % slower).
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
struct RowOperand {
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned voff[LOADS_PER_THREAD];  // byte offset of (row, lchunk * 8) at K = 0
};

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit dwords

// Operand whose tile rows are consecutive rows of a row-major matrix:
// `base` = first row of the tile, `ld` = elements per row, `rows_left` = rows
// that exist from `base` on, `k0` = first K element.
__device__ __forceinline__ RowOperand row_operand(const uint16_t* base, size_t ld, long rows_left, int k0,
                                                  int tid) {
  RowOperand op;
  const size_t bytes = (size_t)max(rows_left, 0L) * ld * 2;
  op.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                              (int)min(bytes, (size_t)0xFFFFFFFFu), kBufferFlags);
  const int lchunk = (tid & 7) ^ ((tid >> 4) & 7);
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it)
    op.voff[it] = (unsigned)(((size_t)(it * LOADER_ROW_STRIDE + (tid >> 3)) * ld + k0 + lchunk * 8) * 2);
  return op;
}
__device__ __forceinline__ int row_lchunk(int tid) { return (tid & 7) ^ ((tid >> 4) & 7); }
__device__ __forceinline__ int row_loader_row(int it, int tid) { return it * LOADER_ROW_STRIDE + (tid >> 3); }

__device__ __forceinline__ void load_stage(const RowOperand& op, int kstep, char* lds_tile, int wave) {
  const unsigned soff = __builtin_amdgcn_readfirstlane((unsigned)kstep * BK * 2);
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it) {
    lds_ptr_t dst = (lds_ptr_t)(lds_tile + (it * NTHREADS + wave * 64) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, dst, 16, op.voff[it], soff, 0, 0);
  }
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// the loop free of branches inside the MFMA stream.
template <typename ROp, typename COp>
__device__ __forceinline__ void mainloop(Acc& acc, const ROp& rop, const COp& cop, int nk, char* smem, int wave,
                                         int lane, int wm, int wn) {
  static_assert(FN <= FM, "B fragments are read behind the first FN rows");
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < ACC_N; ++e) acc.c[i][j][e] = 0.f;
  if (nk <= 0) return;

  RowFrag rf, cf;
  rf.init(wm * 128, lane);
  cf.init(wn * WAVE_COLS, lane);
  bf16x8_t fa[2][FM], fb[2][FN];
#define DPO_RD_A(buf_, s_, slot_, i_) fa[slot_][i_] = rf.read(smem + (buf_) * STAGE_BYTES, i_, s_)
#define DPO_RD_B(buf_, s_, slot_, j_) fb[slot_][j_] = cf.read(smem + (buf_) * STAGE_BYTES + OPER_BYTES, j_, s_)
#define DPO_ROW(slot_, i_, buf_, s_)                                                                      \
  do {                                                                                                    \
    _Pragma("unroll") for (int j_ = 0; j_ < FN; ++j_) acc.c[i_][j_] =                                     \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot_][i_], fb[slot_][j_], acc.c[i_][j_], 0, 0, 0);    \
    if ((i_) < FN) DPO_RD_B(buf_, s_, (slot_) ^ 1, i_);                                                   \
    DPO_RD_A(buf_, s_, (slot_) ^ 1, i_);                                                                  \
    if ((i_) < FN) {                                                                                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                  \
    } else {                                                                                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                  \
    }                                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                                    \
  } while (0)

  load_stage(rop, 0, smem, wave);
  load_stage(cop, 0, smem + OPER_BYTES, wave);
  wait_loads();
  __syncthreads();
  if (nk > 1) {
    load_stage(rop, 1, smem + STAGE_BYTES, wave);
    load_stage(cop, 1, smem + STAGE_BYTES + OPER_BYTES, wave);
  }
  // the loop's own read order (B_i, A_i, ...), all landed before the loop: the
  // compiler's wait counts at the loop head then follow the loop's reads only
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i < FN) DPO_RD_B(0, 0, 0, i);
    DPO_RD_A(0, 0, 0, i);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
#pragma unroll
    for (int i = 0; i < FM; ++i) DPO_ROW(0, i, cur, 1);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc.c[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[1][0], fb[1][j], acc.c[0][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < nk) {
      load_stage(rop, kt + 2, smem + cur * STAGE_BYTES, wave);
      load_stage(cop, kt + 2, smem + cur * STAGE_BYTES + OPER_BYTES, wave);
    }
    DPO_RD_B(cur ^ 1, 0, 0, 0);
    DPO_RD_A(cur ^ 1, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < FM; ++i) DPO_ROW(1, i, cur ^ 1, 0);
  }
#undef DPO_ROW
#undef DPO_RD_B
#undef DPO_RD_A
  // every wave is done with the LDS tiles before the caller reuses them
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
}

// Row (within the 256-row block tile) and column (within the 256-col tile) of
// accumulator element e of fragment (i, j) for this lane.
__device__ __forceinline__ int acc_row(int wm, int i, int e, int lane) {
  return wm * 128 + i * FRAG + 4 * (lane >> 4) + e;
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * WAVE_COLS + j * FRAG + (lane & 15); }

// Persistent tile scheduler.  Tiles are numbered in grouped order (GM m-tiles
// wide, m fastest, then n) and the numbering is cut into NUM_XCD contiguous
// parts; the blocks resident on one XCD (blockIdx % NUM_XCD) walk their part
// together, so tiles that share operand rows run at the same time on the same
// L2.
struct Sched {
  int nMt, nNt, total, gm;
  int begin, end, step;
  __device__ __forceinline__ void init(int nMt_, int nNt_, int gm_) {
    nMt = nMt_;
    nNt = nNt_;
    total = nMt * nNt;
    gm = gm_ < 1 ? 1 : gm_;
    const int xcd = blockIdx.x % NUM_XCD;
    const int q = blockIdx.x / NUM_XCD;
    const int part = cdiv(total, NUM_XCD);
    step = (gridDim.x - xcd + NUM_XCD - 1) / NUM_XCD;  // blocks on this XCD
    begin = xcd * part + q;
    end = min(total, (xcd + 1) * part);
  }
  __device__ __forceinline__ void coords(int t, int& mt, int& nt) const {
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
