// bf16 MFMA main loop shared by the four LM-head contractions (gfx950).
//
// C[i][j] = sum_k A[i][k] * B[j][k]: both operands K-contiguous ("NT").  The
// kernels that use this core differ only in where operand rows come from and
// in their epilogues:
//   forward / recompute : A = hidden rows at completion positions, B = W_vocab
//   dHidden             : A = D (dlogits, bf16), B = W_vocab^T
//   dW_vocab            : A = D^T,              B = hidden^T at completion positions
//
// Block tile 256x256x64, 512 threads = 8 waves in a 2x4 grid (two waves per
// SIMD, so one wave's LDS and barrier waits are covered by the other's MFMAs);
// each wave owns a 128x64 sub-tile held as 4x2 fragments of
// v_mfma_f32_32x32x16_bf16 (128 accumulator registers).  Operand tiles go
// from global memory straight into LDS with global_load_lds_dwordx4 (16 bytes
// per lane, no register staging), double buffered (2 stages x 2 operands x
// 32 KiB = 128 KiB of the 160 KiB LDS).  The K loop is software pipelined:
// the fragments of the next 16-wide K step are read while the MFMAs of the
// current one issue, and the stage barrier sits inside the MFMA stream of the
// last step of a stage, with the next stage's first fragments read across it.
//
// LDS layout of one operand tile: 256 rows x 128 bytes (64 bf16 of K).  The
// 16-byte chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7) so
// that the fragment reads (32 rows, same logical chunk) spread over all banks
// (no bank conflicts measured).  global_load_lds places lane L's 16 bytes at
// (wave base + 16 L), so the swizzle is realised by choosing which global
// chunk each lane fetches.
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

// Per-thread constants of the loader: this thread fetches rows
// (it * 64 + tid / 8), it = 0..3, at logical chunk lchunk() of each K step.
__device__ __forceinline__ int loader_row(int it, int tid) { return it * LOADER_ROW_STRIDE + (tid >> 3); }
__device__ __forceinline__ int loader_lchunk(int tid) { return (tid & 7) ^ ((tid >> 4) & 7); }

// Issue the global->LDS copies of one operand tile for one K step.
// rows[it] points at element (row, lchunk*8) of the operand; k0 is the K offset.
__device__ __forceinline__ void load_tile(const uint16_t* const (&rows)[LOADS_PER_THREAD], int k0,
                                          char* lds_tile, int wave) {
#pragma unroll
  for (int it = 0; it < LOADS_PER_THREAD; ++it) {
    lds_ptr_t dst = (lds_ptr_t)(lds_tile + (it * NTHREADS + wave * 64) * 16);
    __builtin_amdgcn_global_load_lds((const void*)(rows[it] + k0), dst, 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The K loop over [k_begin, k_begin + nk*BK).  nk may be 0 (accumulators stay
// zero).  The caller guarantees every row pointer is valid over that range.
// SWAP = false: MFMA rows come from the first operand tile (arows) and
// columns from the second (brows).  SWAP = true: the roles are exchanged, so
// accumulator rows index the second operand and columns the first.
// Wave (wm, wn) owns MFMA rows wm*128 .. +128 and columns wn*64 .. +64.
template <bool SWAP>
__device__ __forceinline__ void mainloop(Acc& acc, const uint16_t* const (&arows)[LOADS_PER_THREAD],
                                         const uint16_t* const (&brows)[LOADS_PER_THREAD], int k_begin,
                                         int nk, char* smem, int wave, int lane, int wm, int wn) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;
  if (nk <= 0) return;

  // fragment read offsets (bytes) inside an operand tile
  const int sw = (lane >> 1) & 7;
  const int r_off = (wm * 128 + (lane & 31)) * 128 + (SWAP ? OPER_BYTES : 0);       // MFMA-row fragments
  const int c_off = (wn * WAVE_COLS + (lane & 31)) * 128 + (SWAP ? 0 : OPER_BYTES);  // MFMA-column fragments
  int choff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) choff[kk] = (((2 * kk + (lane >> 5)) ^ sw) << 4);

  bf16x8_t fa[2][FM], fb[2][FN];
#define DPO_READ_FRAGS(stage_, kk_, slot_)                                                     \
  do {                                                                                         \
    const char* base_ = smem + (stage_) * STAGE_BYTES;                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < FM; ++i_) fa[slot_][i_] =                          \
        *(const bf16x8_t*)(base_ + r_off + i_ * 4096 + choff[kk_]);                            \
    _Pragma("unroll") for (int j_ = 0; j_ < FN; ++j_) fb[slot_][j_] =                          \
        *(const bf16x8_t*)(base_ + c_off + j_ * 4096 + choff[kk_]);                            \
  } while (0)

  load_tile(arows, k_begin, smem, wave);
  load_tile(brows, k_begin, smem + OPER_BYTES, wave);
  wait_loads();
  __syncthreads();
  if (nk > 1) {
    load_tile(arows, k_begin + BK, smem + STAGE_BYTES, wave);
    load_tile(brows, k_begin + BK, smem + STAGE_BYTES + OPER_BYTES, wave);
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
            load_tile(arows, k_begin + (kt + 2) * BK, smem + cur * STAGE_BYTES, wave);
            load_tile(brows, k_begin + (kt + 2) * BK, smem + cur * STAGE_BYTES + OPER_BYTES, wave);
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
