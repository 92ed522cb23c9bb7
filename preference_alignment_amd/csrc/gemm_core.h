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
// each wave owns a 128x64 sub-tile held as 4x2 fragments of
// v_mfma_f32_32x32x16_bf16 (128 accumulator registers).  Operand tiles go
// from global memory straight into LDS with buffer_load_dwordx4 ... lds
// (global_load_lds_dwordx4 for dHidden; 16 bytes per lane, no register
// staging), double buffered (2 stages x 2 operands x
// 32 KiB = 128 KiB of the 160 KiB LDS).  The K loop is software pipelined:
// the fragments of the next 16-wide K step are read while the MFMAs of the
// current one issue, and the stage barrier sits inside the MFMA stream of the
// last step of a stage, with the next stage's first fragments read across it.
//
// Both loads place lane L's 16 bytes at (wave base + 16 L), so the LDS
// swizzles below are realised by choosing which global chunk each lane fetches.
//
// MFMA 32x32x16 register layout (CDNA3/CDNA4 32x32 family): lane l supplies
// A[l % 32][8 (l / 32) + 0..7] and B^T likewise; accumulator element e of lane
// l is C[8 (e / 4) + 4 (l / 32) + (e % 4)][l % 32].  The K permutation inside
// a fragment is irrelevant (A and B use the same one); the C layout is what the
// epilogues rely on.
#pragma once

#include "dpo_common.h"

namespace dpo {
namespace gemm {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 512;
constexpr int WAVES_N = 4;             // waves along the MFMA columns
constexpr int FM = 4;                  // 32-row fragments per wave (128 rows)
constexpr int FN = 2;                  // 32-col fragments per wave (64 cols)
constexpr int WAVE_COLS = 32 * FN;
constexpr int OPER_BYTES = BM * BK * 2;       // 32 KiB
constexpr int STAGE_BYTES = 2 * OPER_BYTES;   // A + B
constexpr int PIPE_BYTES = 2 * STAGE_BYTES;   // double buffer, 128 KiB
constexpr int LOADS_PER_THREAD = BM * (BK / 8) / NTHREADS;  // 4 rows per operand
constexpr int LOADER_ROW_STRIDE = NTHREADS / 8;             // 64
constexpr int NUM_XCD = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct Acc {
  floatx16 c[FM][FN];
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

// ROW operand read with global_load_lds from per-row 64-bit pointers.  Same
// LDS layout as RowOperand; measured faster than buffer loads for the
// dHidden contraction, whose two operands both stride 256 KiB between rows.
struct FlatRowOperand {
  const uint16_t* rows[LOADS_PER_THREAD];  // element (row, lchunk * 8) at K = 0
};

__device__ __forceinline__ void load_stage(const FlatRowOperand& op, int kstep, char* lds_tile, int wave) {
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it) {
    lds_ptr_t dst = (lds_ptr_t)(lds_tile + (it * NTHREADS + wave * 64) * 16);
    __builtin_amdgcn_global_load_lds((const void*)(op.rows[it] + (size_t)kstep * BK), dst, 16, 0, 0);
  }
}

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

// Fragment readers.  `f` = fragment index along the MFMA dimension (32 wide),
// `base` = first MFMA row/column of this wave inside the tile, kk = 16-wide K step.
struct RowFrag {
  int off[4];  // byte offset of (row, chunk of step kk) for fragment 0
  __device__ __forceinline__ void init(int base, int lane) {
    const int sw = (lane >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) off[kk] = (base + (lane & 31)) * 128 + (((2 * kk + (lane >> 5)) ^ sw) << 4);
  }
  __device__ __forceinline__ bf16x8_t read(const char* tile, int f, int kk) const {
    return *(const bf16x8_t*)(tile + off[kk] + f * 4096);
  }
};

template <typename Op, int NF> struct FragOf;
template <int NF> struct FragOf<RowOperand, NF> { typedef RowFrag type; };
template <int NF> struct FragOf<FlatRowOperand, NF> { typedef RowFrag type; };

// The K loop over nk steps of BK.  nk may be 0 (accumulators stay zero).  The
// R operand supplies the MFMA rows (wave (wm, wn) owns rows wm*128 .. +128),
// the C operand the MFMA columns (columns wn*64 .. +64).  Software pipelined:
// the fragments of the next 16-wide K step are read while the MFMAs of the
// current one issue, and the stage barrier sits inside the MFMA stream of the
// last step of a stage, with the next stage's first fragments read across it.
template <typename ROp, typename COp>
__device__ __forceinline__ void mainloop(Acc& acc, const ROp& rop, const COp& cop, int nk, char* smem, int wave,
                                         int lane, int wm, int wn) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;
  if (nk <= 0) return;

  typename FragOf<ROp, FM>::type rf;
  typename FragOf<COp, FN>::type cf;
  rf.init(wm * 128, lane);
  cf.init(wn * WAVE_COLS, lane);
  bf16x8_t fa[2][FM], fb[2][FN];
#define DPO_READ_FRAGS(stage_, kk_, slot_)                                                     \
  do {                                                                                         \
    const char* base_ = smem + (stage_) * STAGE_BYTES;                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < FM; ++i_) fa[slot_][i_] = rf.read(base_, i_, kk_); \
    _Pragma("unroll") for (int j_ = 0; j_ < FN; ++j_) fb[slot_][j_] =                          \
        cf.read(base_ + OPER_BYTES, j_, kk_);                                                  \
  } while (0)

  load_stage(rop, 0, smem, wave);
  load_stage(cop, 0, smem + OPER_BYTES, wave);
  wait_loads();
  __syncthreads();
  if (nk > 1) {
    load_stage(rop, 1, smem + STAGE_BYTES, wave);
    load_stage(cop, 1, smem + STAGE_BYTES + OPER_BYTES, wave);
  }
  DPO_READ_FRAGS(0, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int sl = kk & 1;
      if (kk < 3) {
        if (sl)
          DPO_READ_FRAGS(cur, kk + 1, 0);
        else
          DPO_READ_FRAGS(cur, kk + 1, 1);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][i], fb[sl][j], acc.c[i][j], 0, 0, 0);
        // one fragment read between consecutive MFMAs
#pragma unroll
        for (int u = 0; u < FM + FN; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        // last 16-wide step of the stage: 2 MFMAs, the stage barrier, the next
        // stage's loads and first fragments, then the remaining MFMAs
        acc.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][0], fb[1][0], acc.c[0][0], 0, 0, 0);
        acc.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][0], fb[1][1], acc.c[0][1], 0, 0, 0);
        if (kt + 1 < nk) {
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          if (kt + 2 < nk) {
            load_stage(rop, kt + 2, smem + cur * STAGE_BYTES, wave);
            load_stage(cop, kt + 2, smem + cur * STAGE_BYTES + OPER_BYTES, wave);
          }
          DPO_READ_FRAGS(cur ^ 1, 0, 0);
        }
#pragma unroll
        for (int u = 2; u < FM * FN; ++u)
          acc.c[u / FN][u % FN] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][u / FN], fb[1][u % FN], acc.c[u / FN][u % FN], 0, 0, 0);
      }
    }
  }
#undef DPO_READ_FRAGS
  // every wave is done with the LDS tiles before the caller reuses them
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
}

// Row (within the 256-row block tile) and column (within the 256-col tile) of
// accumulator element e of fragment (i, j) for this lane.
__device__ __forceinline__ int acc_row(int wm, int i, int e, int lane) {
  return wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * WAVE_COLS + j * 32 + (lane & 31); }

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
