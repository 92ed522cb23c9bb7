// bf16 MFMA main loop shared by the four LM-head contractions (gfx950).
//
// C[i][j] = sum_k A[i][k] * B[j][k]: both operands K-contiguous ("NT").  The
// kernels that use this core differ only in where operand rows come from and
// in their epilogues:
//   forward / recompute : A = hidden rows at completion positions, B = W_vocab
//   dHidden             : A = D (dlogits, bf16), B = W_vocab^T
//   dW_vocab            : A = D^T,              B = hidden^T at completion positions
//
// Block tile 256x256x64, 256 threads = 4 waves in a 2x2 grid, each wave owns a
// 128x128 sub-tile held as 4x4 fragments of v_mfma_f32_32x32x16_bf16.
// Operand tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (16 bytes per lane, no register staging), double
// buffered (2 stages x 2 operands x 32 KiB = 128 KiB of the 160 KiB LDS).
//
// LDS layout of one operand tile: 256 rows x 128 bytes (64 bf16 of K).  The
// 16-byte chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7) so
// that the fragment reads (32 rows, same logical chunk) spread over all banks.
// global_load_lds places lane L's 16 bytes at (wave base + 16 L), so the
// swizzle is realised by choosing which global chunk each lane fetches.
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
constexpr int NTHREADS = 256;
constexpr int FM = 4;  // 32-row fragments per wave
constexpr int FN = 4;  // 32-col fragments per wave
constexpr int OPER_BYTES = BM * BK * 2;       // 32 KiB
constexpr int STAGE_BYTES = 2 * OPER_BYTES;   // A + B
constexpr int PIPE_BYTES = 2 * STAGE_BYTES;   // double buffer, 128 KiB
constexpr int LOADS_PER_THREAD = BM * (BK / 8) / NTHREADS;  // 8 rows per operand
constexpr int NUM_XCD = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct Acc {
  floatx16 c[FM][FN];
};

// Per-thread constants of the loader: this thread fetches rows
// (it * 32 + tid / 8), it = 0..7, at logical chunk lchunk() of each K step.
__device__ __forceinline__ int loader_row(int it, int tid) { return it * 32 + (tid >> 3); }
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

// The K loop.  nk = number of BK steps (may be 0: accumulators stay zero).
// The caller guarantees every row pointer is valid for k < nk * BK.
__device__ __forceinline__ void mainloop(Acc& acc, const uint16_t* const (&arows)[LOADS_PER_THREAD],
                                         const uint16_t* const (&brows)[LOADS_PER_THREAD], int nk,
                                         char* smem, int wave, int lane, int wm, int wn) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;
  if (nk <= 0) return;

  // fragment read offsets (bytes) inside an operand tile
  const int sw = (lane >> 1) & 7;
  const int a_off = (wm * 128 + (lane & 31)) * 128;
  const int b_off = (wn * 128 + (lane & 31)) * 128;
  int choff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) choff[kk] = (((2 * kk + (lane >> 5)) ^ sw) << 4);

  load_tile(arows, 0, smem, wave);
  load_tile(brows, 0, smem + OPER_BYTES, wave);
  wait_loads();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    if (kt + 1 < nk) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE_BYTES;
      load_tile(arows, (kt + 1) * BK, nxt, wave);
      load_tile(brows, (kt + 1) * BK, nxt + OPER_BYTES, wave);
    }
    const char* As = cur;
    const char* Bs = cur + OPER_BYTES;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *(const bf16x8_t*)(As + a_off + i * 4096 + choff[kk]);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *(const bf16x8_t*)(Bs + b_off + j * 4096 + choff[kk]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
    }
    wait_loads();
    __syncthreads();
  }
}

// Row (within the 256-row block tile) and column (within the 256-col tile) of
// accumulator element e of fragment (i, j) for this lane.
__device__ __forceinline__ int acc_row(int wm, int i, int e, int lane) {
  return wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 128 + j * 32 + (lane & 31); }

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
