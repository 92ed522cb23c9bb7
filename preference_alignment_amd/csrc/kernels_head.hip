// Fused LM-head kernels of the DPO sequence log-probability path (gfx950).
//
// The method ("DPO Training on GPU, in depth", sections "What one DPO step
// computes" and "A training configuration that fits"): for every completion
// position t of row r, z_t = W_vocab . h_t over the whole vocabulary,
// log p_t = z_t[y_t] - logsumexp(z_t), and the row score is the sum of log p_t
// over the completion positions of the row.  The backward of the sigmoid DPO
// loss through that score is dz_t = w_r (softmax(z_t) - onehot(y_t)), giving
// dHidden_t = dz_t . W_vocab and dW_vocab = sum_t dz_t^T h_t.  The page's
// hand-written loss recomputes the fp32 log-softmax in backward instead of
// keeping it; the fused path here does the same with the contraction itself,
// so no [rows x T x V] logits tensor ever exists.
//
// Kernels, in call order:
//   k_compact        completion positions (row-major), per-row offsets, targets check
//   k_fwd_gemm       Z tile = Hc . W^T on MFMA; epilogue: per-row (max, sum exp) over
//                    the tile's columns and capture of the target logit
//   k_combine        combine of the per-tile (max, sum exp), fp64 sums -> lse, log p
//                    (and of the per-tile logit sums, when asked for)
//   k_row_sums       fp64 per-row sums in a fixed order
//   k_gather_ht      Hc^T (bf16) for the dW contraction
//   k_dprod_gemm     recompute Z tile; epilogue D = w exp(z - lse) -> bf16 D (softmax part)
//   k_dh_gemm        dHidden partials = D . W, K split in parts; each part's fp32 slab
//                    accumulates over the vocabulary slices
//   k_dh_finish      dHidden rows = sum of the slabs - w W[target], scattered to their positions
//   k_dw_gemm        dW_vocab = D^T . Hc (overwrite or accumulate)
//   k_sort_targets   completion positions stably sorted by target id
//   k_onehot_dw(+_join) dW_vocab[y] -= sum of w h over the positions whose target is y
//
// The one-hot term of dlogits is kept out of the bf16 operand D: rounding the
// single large entry w (p_y - 1) to bf16 alone would cost ~1e-3 relative error
// in dHidden.  It is applied exactly in fp32 instead, by a gather of W[y] in
// the dHidden epilogue and a fixed-order per-target sum for dW_vocab.
//   k_zero_rows      dHidden = 0 at positions outside the completion mask
#include <mutex>

#include "dpo_common.h"
#include "gemm_core.h"
#include "launch.h"

namespace dpo {
using namespace gemm;

// ---------------------------------------------------------------------------
// completion positions
// ---------------------------------------------------------------------------
constexpr int kCompactThreads = 1024;
constexpr int kCompactWaves = kCompactThreads / 64;

// One workgroup walks the positions in rounds of 4,096 consecutive ones,
// thread t taking positions 4096 r + 4 t .. + 3.  A position's output slot is
// the running count of earlier rounds plus the count of earlier waves in its
// round (a 16-entry LDS table, double buffered so each round needs one
// barrier) plus the count of earlier lanes of its wave (a prefix sum over the
// lanes' counts) plus that of its thread's earlier positions.  Row-major
// ascending order falls out of this directly.
constexpr int kCompactPer = 4;  // positions per thread and round

__global__ __launch_bounds__(kCompactThreads) void k_compact(CompactArgs a) {
  __shared__ int wtot[2][kCompactWaves];
  __shared__ int err;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const long N = (long)a.rows * a.T;
  if (tid == 0) err = 0;
  int base = 0;  // completion positions before this round
  int bad = 0;
  constexpr int kRound = kCompactThreads * kCompactPer;
  for (long r0 = 0, round = 0; r0 < N; r0 += kRound, ++round) {
    const long p0 = r0 + (long)kCompactPer * tid;
    bool on[kCompactPer];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kCompactPer; ++u) {
      on[u] = p0 + u < N && a.mask[p0 + u] != 0;
      c += on[u];
    }
    // inclusive prefix sum of the lanes' counts
    int inc = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off, 64);
      if (lane >= off) inc += y;
    }
    const int buf = (int)(round & 1);
    if (lane == 63) wtot[buf][wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kCompactWaves; ++w) {
      const int cw = wtot[buf][w];
      before += w < wave ? cw : 0;
      total += cw;
    }
    int pos = base + before + inc - c;
#pragma unroll
    for (int u = 0; u < kCompactPer; ++u) {
      const long p = p0 + u;
      if (p < N) {
        if (p % a.T == 0) a.row_off[p / a.T] = pos;
        if (on[u]) {
          int t = a.targets[p];
          if (t < 0 || t >= a.V_total) {
            bad = 1;
            t = -1;
          } else {
            t -= a.v_begin;
            if (t < 0 || t >= a.V) t = -1;  // held by another vocabulary shard
          }
          a.idx[pos] = (int)p;
          a.tgt_c[pos] = t;
          a.row_c[pos] = (int)(p / a.T);
          ++pos;
        } else {
          if (a.lse_out) a.lse_out[p] = 0.f;
          if (a.off_max) {
            a.off_max[p] = -INFINITY;
            a.off_sum[p] = 0.f;
            a.off_tgt[p] = -INFINITY;
          }
        }
      }
    }
    base += total;
  }
  const int n_c = base;
  if (bad) atomicOr(&err, kStatusTargetRange);
  // padding entries up to the padded position count: a valid row, no target
  for (long m = n_c + tid; m < a.Mp; m += kCompactThreads) {
    a.idx[m] = 0;
    a.tgt_c[m] = -1;
    a.row_c[m] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    a.row_off[a.rows] = n_c;
    a.hdr->n_c = n_c;
    a.hdr->status = err;
  }
}

// ---------------------------------------------------------------------------
// forward contraction with the online log-sum-exp epilogue
// ---------------------------------------------------------------------------
// The MFMA runs with exchanged roles (rows = vocabulary, columns = positions):
// a lane then holds one position and 32 of the wave's 128 vocabulary entries,
// the other 96 sitting in lanes ^ 16, ^ 32 and ^ 48.  The per-position max
// and sum of exponentials over the wave's rows are in-lane reductions plus
// two cross-lane shuffles, and the two vocabulary halves of the block
// (wm = 0, 1) meet through a small LDS table.
constexpr int kEpiBytes = 8192;  // per-position staging + cross-wave reduction
static __shared__ __attribute__((aligned(16))) char g_epi[kEpiBytes];

template <typename F>
__device__ __forceinline__ void for_vocab(const Acc& acc, int j, F f) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < ACC_N; ++e) f(acc.c[i][j][e]);
}

// The lane / thread index through an empty asm: offsets computed from it in an
// epilogue cannot be hoisted out of the persistent tile loop, where they would
// stay live across the main loop and push it into register spills.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Logits of vocabulary rows past V (the zero-filled rows of the last tile)
// become -inf, so the epilogues need no per-element bounds test: they drop
// out of the max, and exp gives 0.  Only the last vocabulary tile takes this.
__device__ __forceinline__ void mask_vocab_tail(Acc& acc, int vbase, int V, int lane) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < ACC_N; ++e)
        if (vbase + i * FRAG + 4 * (lane >> 4) + e >= V) acc.c[i][j][e] = -INFINITY;
}

// Tile order of the forward-shaped contractions (m = position tiles, n =
// vocabulary tiles).  While the gathered hidden rows fit a 128 MiB share of
// the 256 MB Infinity Cache, vocabulary groups of a.gn tiles: each XCD sweeps
// its own vocabulary range over all positions, so W_vocab is read from HBM
// once and the hidden rows come from the cache (0.9 ms per step faster than
// position groups at 8 rows x 2,048, H 4,096).  Past that (e.g. 131,072
// positions at H 4,096), position groups of a.gm tiles bound the hidden rows
// in use at once to 8 XCDs x a.gm tiles.
__device__ __forceinline__ void fwd_sched(Sched& sc, int n_c, int H, int nNt, int gm, int gn) {
  const bool hidden_cached = (size_t)n_c * H * 2 <= (size_t(128) << 20);
  sc.init(cdiv(n_c, BM), nNt, gm, hidden_cached ? gn : 0);
}

template <bool ZSUM>
__global__ __launch_bounds__(NTHREADS) void k_fwd_gemm(FwdArgs a) {
  int* tgt_s = (int*)g_epi;                   // 256 ints
  float2* red = (float2*)(g_epi + 1024);      // [2][256]
  float* red_z = (float*)(g_epi + 5120);      // [2][256] (logit sums)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int n_c = a.hdr->n_c;
  Sched sc;
  fwd_sched(sc, n_c, a.H, cdiv(a.V, BN), a.gm, a.gn);
  const int lchunk = row_lchunk(tid);
  const int nk = a.H / BK;
  // operands of a tile: W rows n0 .. n0+255 (rows past V read as zero);
  // hidden rows gathered by position, addressed from the start of the hidden
  // tensor.  Each tile's stages are issued before the previous tile's epilogue.
  RowOperand wop, hop;
  hop.rsrc = buffer_rsrc(a.hidden, a.hidden_bytes);
  int tgt_cur = 0;
  if (sc.begin < sc.end) {
    int mt, nt;
    sc.coords(sc.begin, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    wop = row_operand(a.w + (size_t)n0 * a.H, a.H, (long)a.V - n0, 0, tid);
#pragma unroll
    for (int it = 0; it < LOADS_PER_THREAD; ++it)
      hop.voff[it] = (unsigned)(((size_t)a.idx[m0 + row_loader_row(it, tid)] * a.H + lchunk * 8) * 2);
    if (tid < BM) tgt_cur = a.tgt_c[m0 + tid];
    mainloop_issue(wop, hop, nk, wave);
  }
  for (int t = sc.begin; t < sc.end; t += sc.step) {
    int mt, nt;
    sc.coords(t, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    if (tid < BM) tgt_s[tid] = tgt_cur;
    // the next tile's position indices and targets, in flight during the main loop
    const int tn = t + sc.step;
    const bool has_next = tn < sc.end;
    int mtn = 0, ntn = 0;
    if (has_next) sc.coords(tn, mtn, ntn);
    int idx_n[LOADS_PER_THREAD];
    int tgt_n = 0;
#pragma unroll
    for (int it = 0; it < LOADS_PER_THREAD; ++it) idx_n[it] = has_next ? a.idx[mtn * BM + row_loader_row(it, tid)] : 0;
    if (has_next && tid < BM) tgt_n = a.tgt_c[mtn * BM + tid];
    Acc acc;
    mainloop_prefetched(acc, wop, hop, nk, wave, lane, wm, wn);
    if (has_next) {
      wop = row_operand(a.w + (size_t)ntn * BN * a.H, a.H, (long)a.V - ntn * BN, 0, tid);
#pragma unroll
      for (int it = 0; it < LOADS_PER_THREAD; ++it)
        hop.voff[it] = (unsigned)(((size_t)idx_n[it] * a.H + lchunk * 8) * 2);
      tgt_cur = tgt_n;
      mainloop_issue(wop, hop, nk, wave);
    }

    const int vbase = n0 + wm * 128;  // first vocabulary row of this wave
    if (n0 + BN > a.V) mask_vocab_tail(acc, vbase, a.V, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int pl = acc_col(wn, j, lane);  // position within the tile
      float mx = -INFINITY;
      for_vocab(acc, j, [&](float v) { mx = fmaxf(mx, v); });
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // a lane group whose rows are all past V keeps (-inf, 0)
      const float ml = mx == -INFINITY ? 0.f : mx * kLog2e;
      float s = 0.f;
      for_vocab(acc, j, [&](float v) { s += fast_exp2(fmaf(v, kLog2e, -ml)); });
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (ZSUM) {
        float zs = 0.f;
        for_vocab(acc, j, [&](float v) { zs += v == -INFINITY ? 0.f : v; });
        zs += __shfl_xor(zs, 16, 64);
        zs += __shfl_xor(zs, 32, 64);
        if (lane < 16) red_z[wm * 256 + pl] = zs;
      }
      const int off = tgt_s[pl] - vbase;
      if (off >= 0 && off < 128) {
        const int r = off & 15;
        if ((r >> 2) == (lane >> 4) && m0 + pl < n_c) {
          const int ii = off >> 4, ee = r & 3;
          // acc.c[ii][j][ee] through a select tree on the index bits (5 lane
          // masks in all, instead of one per candidate element)
          float vi[FM];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const float t0 = (ee & 1) ? acc.c[i][j][1] : acc.c[i][j][0];
            const float t1 = (ee & 1) ? acc.c[i][j][3] : acc.c[i][j][2];
            vi[i] = (ee & 2) ? t1 : t0;
          }
#pragma unroll
          for (int b = 0; b < 3; ++b) {
            const bool hi = (ii >> b) & 1;
#pragma unroll
            for (int k = 0; k < (FM >> (b + 1)); ++k) vi[k] = hi ? vi[2 * k + 1] : vi[2 * k];
          }
          a.tgt_logit[m0 + pl] = vi[0];
        }
      }
      if (lane < 16) red[wm * 256 + pl] = make_float2(mx, s);
    }
    __syncthreads();
    if (tid < BM) {
      const float2 p0 = red[tid], p1 = red[256 + tid];
      const float M = fmaxf(p0.x, p1.x);
      const float S = (p0.x == -INFINITY ? 0.f : p0.y * fast_exp2((p0.x - M) * kLog2e)) +
                      (p1.x == -INFINITY ? 0.f : p1.y * fast_exp2((p1.x - M) * kLog2e));
      if (m0 + tid < n_c) a.part[(size_t)nt * a.Mp + m0 + tid] = make_float2(M, S);
      if (ZSUM && m0 + tid < n_c) a.part_z[(size_t)nt * a.Mp + m0 + tid] = red_z[tid] + red_z[256 + tid];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// combine per-tile partials: lse = M + log(sum_j s_j exp(m_j - M))
// ---------------------------------------------------------------------------
// A block takes 16 positions; its 16 thread groups split the vocabulary tiles
// (tile j goes to group j % 16).  The global max comes first, then each group
// accumulates its share of sum_j s_j exp(m_j - M) in fp64 and the 16 shares
// are added in group order, so the result does not depend on timing.
constexpr int kCombPos = 16;
constexpr int kCombGroups = 16;

__global__ __launch_bounds__(kCombPos * kCombGroups) void k_combine(CombineArgs a) {
  __shared__ float red_m[kCombGroups][kCombPos];
  __shared__ double red_s[kCombGroups][kCombPos];
  __shared__ double red_z[kCombGroups][kCombPos];
  const int p = threadIdx.x % kCombPos, g = threadIdx.x / kCombPos;
  const int m = blockIdx.x * kCombPos + p;
  const int n_c = a.hdr->n_c;
  if (blockIdx.x * kCombPos >= n_c) return;
  const bool live = m < n_c;
  float M = -INFINITY;
  if (live) {
#pragma unroll 4
    for (int j = g; j < a.nVt; j += kCombGroups) M = fmaxf(M, a.part[(size_t)j * a.Mp + m].x);
  }
  red_m[g][p] = M;
  __syncthreads();
  M = red_m[0][p];
  for (int q = 1; q < kCombGroups; ++q) M = fmaxf(M, red_m[q][p]);
  double S = 0.0, Z = 0.0;
  if (live) {
    const float Ml = M * kLog2e;
#pragma unroll 4
    for (int j = g; j < a.nVt; j += kCombGroups) {
      const float2 t = a.part[(size_t)j * a.Mp + m];
      S += (double)(t.y * fast_exp2(fmaf(t.x, kLog2e, -Ml)));
    }
    if (a.part_z)
      for (int j = g; j < a.nVt; j += kCombGroups) Z += (double)a.part_z[(size_t)j * a.Mp + m];
  }
  red_s[g][p] = S;
  if (a.part_z) red_z[g][p] = Z;
  __syncthreads();
  if (g == 0 && live) {
    S = red_s[0][p];
    for (int q = 1; q < kCombGroups; ++q) S += red_s[q][p];
    const double lse = (double)M + log(S);
    const int t = a.tgt_c[m];
    a.lse64[m] = lse;
    a.logp64[m] = t >= 0 ? (double)a.tgt_logit[m] - lse : __builtin_nan("");
    if (a.lse_out) a.lse_out[a.idx[m]] = (float)lse;
    if (a.part_z) {
      Z = red_z[0][p];
      for (int q = 1; q < kCombGroups; ++q) Z += red_z[q][p];
      a.zsum64[m] = Z;
    }
  }
}

// ---------------------------------------------------------------------------
// per-row sums of log p in fp64, fixed reduction order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_row_sums(RowSumArgs a) {
  __shared__ double red[256];
  const int r = blockIdx.x;
  const int lo = a.row_off[r];
  const int hi = r + 1 < a.rows ? a.row_off[r + 1] : a.hdr->n_c;
  double s = 0.0;
  for (int m = lo + threadIdx.x; m < hi; m += 256) s += a.logp64[m];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double v = red[0];
    if (a.sum32) a.sum32[r] = (float)v;
    if (a.sum64) a.sum64[r] = v;
    if (a.n_tokens) a.n_tokens[r] = hi - lo;
  }
}

// ---------------------------------------------------------------------------
// vocabulary shards: a shard's (max, sum exp, target logit) per position, and
// the combine of S shards' values into the whole-vocabulary lse and log p
// ---------------------------------------------------------------------------
// Laid out like k_combine: 16 positions per block, the shard's vocabulary
// tiles split over 16 thread groups (tile j to group j % 16), the groups'
// fp64 shares added in group order.
__global__ __launch_bounds__(kCombPos * kCombGroups) void k_shard_partials(ShardPartialArgs a) {
  __shared__ float red_m[kCombGroups][kCombPos];
  __shared__ double red_s[kCombGroups][kCombPos];
  const int p = threadIdx.x % kCombPos, g = threadIdx.x / kCombPos;
  const int m = blockIdx.x * kCombPos + p;
  const int n_c = a.hdr->n_c;
  if (blockIdx.x * kCombPos >= n_c) return;
  const bool live = m < n_c;
  float M = -INFINITY;
  if (live) {
#pragma unroll 4
    for (int j = g; j < a.nVt; j += kCombGroups) M = fmaxf(M, a.part[(size_t)j * a.Mp + m].x);
  }
  red_m[g][p] = M;
  __syncthreads();
  M = red_m[0][p];
  for (int q = 1; q < kCombGroups; ++q) M = fmaxf(M, red_m[q][p]);
  double S = 0.0;
  if (live) {
    const float Ml = M * kLog2e;
#pragma unroll 4
    for (int j = g; j < a.nVt; j += kCombGroups) {
      const float2 t = a.part[(size_t)j * a.Mp + m];
      S += (double)(t.y * fast_exp2(fmaf(t.x, kLog2e, -Ml)));
    }
  }
  red_s[g][p] = S;
  __syncthreads();
  if (g == 0 && live) {
    S = red_s[0][p];
    for (int q = 1; q < kCombGroups; ++q) S += red_s[q][p];
    const int pos = a.idx[m];
    a.out_max[pos] = M;
    a.out_sum[pos] = (float)S;
    a.out_tgt[pos] = a.tgt_c[m] >= 0 ? a.tgt_logit[m] : -INFINITY;
  }
}

__global__ __launch_bounds__(256) void k_shard_combine(ShardCombineArgs a) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= a.hdr->n_c) return;
  const size_t p = (size_t)a.idx[m];
  float M = -INFINITY, tg = -INFINITY;
  for (int q = 0; q < a.S; ++q) {
    M = fmaxf(M, a.pmax[q * a.stride + p]);
    tg = fmaxf(tg, a.ptgt[q * a.stride + p]);
  }
  double S = 0.0;
  for (int q = 0; q < a.S; ++q) {
    const float mq = a.pmax[q * a.stride + p];
    if (mq != -INFINITY) S += (double)a.psum[q * a.stride + p] * exp((double)mq - (double)M);
  }
  const double lse = (double)M + log(S);
  const bool ok = a.tgt_c[m] >= 0 && tg != -INFINITY;
  if (!ok) atomicOr(&a.hdr->status, kStatusTargetRange);
  a.lse64[m] = lse;
  a.logp64[m] = ok ? (double)tg - lse : __builtin_nan("");
  if (a.lse_out) a.lse_out[p] = (float)lse;
}

// ---------------------------------------------------------------------------
// gathered hidden rows, transposed, for the dW_vocab contraction
// ---------------------------------------------------------------------------
// hidden rows at completion positions -> HT [H, Mp], zero columns m >= n_c.
// 64 positions x 64 hidden columns per block, 16-byte loads and stores.
__global__ __launch_bounds__(256) void k_gather_ht(GatherHTArgs a) {
  __shared__ uint16_t tile[64][72];
  const int n_c = a.hdr->n_c;
  const int m0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  if (m0 >= (int)align_up((size_t)n_c, BM)) return;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = it * 256 + tid;  // 64 positions x 8 chunks of 8 hidden columns
    const int r = q >> 3, c = q & 7;
    const int m = m0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (m < n_c) val = *(const u32x4*)(a.hidden + (size_t)a.idx[m] * a.H + h0 + c * 8);
    *(u32x4*)&tile[r][c * 8] = val;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = it * 256 + tid;  // 64 hidden rows x 8 chunks of 8 positions
    const int h = q >> 3, c = q & 7;
    uint32_t w4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w4[u] = (uint32_t)tile[c * 8 + 2 * u][h] | ((uint32_t)tile[c * 8 + 2 * u + 1][h] << 16);
    const u32x4 o = {w4[0], w4[1], w4[2], w4[3]};
    *(u32x4*)(a.ht + (size_t)(h0 + h) * a.ldt + m0 + c * 8) = o;
  }
}

// ---------------------------------------------------------------------------
// backward: recompute Z, D = w exp(z - lse) in bf16
// ---------------------------------------------------------------------------
// Same MFMA orientation as the forward (rows = vocabulary, columns =
// positions): a lane holds 4 consecutive vocabulary entries of one position
// per fragment, packed to one 8-byte LDS write.  The bf16 tile (256
// positions x 256 vocabulary, 128 KiB) is staged in the freed pipeline LDS
// and leaves as 16-byte coalesced rows of D [Mp, Vp].  Both consumers read D
// as it is: dHidden with K = vocabulary along its rows, dW_vocab with K =
// positions down its columns (transposing LDS reads), so no D^T is written.
// Staging layout: the 16-byte chunk c of position row p sits at chunk
// c ^ f(p), f(p) = (p ^ (p >> 3)) & 31, which keeps the 8-byte writes of the
// four lane groups and the row reads free of bank conflicts.
__device__ __forceinline__ int stage_off(int p, int v) {
  const int f = (p ^ (p >> 3)) & 31;
  return p * 512 + ((((v >> 3) ^ f)) << 4) + ((v & 7) << 1);
}
// positions 0..127 are staged in the first pipeline buffer, 128..255 in the second
__device__ __forceinline__ char* stage_at(int p, int v) {
  return (p < BM / 2 ? g_stage0 : g_stage1) + stage_off(p & (BM / 2 - 1), v);
}

__global__ __launch_bounds__(NTHREADS) void k_dprod_gemm(DProdArgs a) {
  float* lse_s = (float*)g_epi;
  float* w_s = (float*)(g_epi + 1024);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int n_c = a.hdr->n_c;
  Sched sc;
  fwd_sched(sc, n_c, a.H, a.Vp / BN, a.gm, a.gn);
  const int lchunk = row_lchunk(tid);
  for (int t = sc.begin; t < sc.end; t += sc.step) {
    int mt, nt;
    sc.coords(t, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    // W rows n0 .. n0+255 (rows past V read as zero); hidden rows gathered by
    // position, addressed from the start of the hidden tensor
    const RowOperand wop = row_operand(a.w + (size_t)n0 * a.H, a.H, (long)a.V - n0, 0, tid);
    RowOperand hop;
    hop.rsrc = buffer_rsrc(a.hidden, a.hidden_bytes);
#pragma unroll
    for (int it = 0; it < LOADS_PER_THREAD; ++it)
      hop.voff[it] = (unsigned)(((size_t)a.idx[m0 + row_loader_row(it, tid)] * a.H + lchunk * 8) * 2);
    if (tid < BM) {
      const int m = m0 + tid;
      const bool live = m < n_c;
      lse_s[tid] = live ? a.lse[a.idx[m]] * kLog2e : 0.f;
      w_s[tid] = live ? a.weight[a.row_c[m]] : 0.f;
    }
    Acc acc;
    mainloop(acc, wop, hop, a.H / BK, wave, lane, wm, wn);
    if (n0 + BN > a.V) mask_vocab_tail(acc, n0 + wm * 128, a.V, lane);

    // D values (bf16) into the staging tile; the pipeline LDS is free now
    const int elane = opaque(lane), etid = opaque(tid);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int pl = acc_col(wn, j, elane);
      const float L = lse_s[pl];
      const float wr = w_s[pl];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int vl = acc_row(wm, i, 0, elane);  // first of 4 vocabulary rows
        float d[ACC_N];
#pragma unroll
        for (int u = 0; u < ACC_N; ++u) {
          // rows past V hold -inf: exp gives 0
          d[u] = wr * fast_exp2(fmaf(acc.c[i][j][u], kLog2e, -L));
        }
        uint2 pk;
        pk.x = pack_bf16x2(d[0], d[1]);
        pk.y = pack_bf16x2(d[2], d[3]);
        *(uint2*)stage_at(pl, vl) = pk;
      }
    }
    __syncthreads();
    // D rows: position m0+p, vocabulary n0 .. n0+255
#pragma unroll 4
    for (int it = 0; it < BM * 32 / NTHREADS; ++it) {
      const int g = it * NTHREADS + etid;
      const int p = g >> 5, c = g & 31;
      const u32x4 v = *(const u32x4*)stage_at(p, c * 8);
      __builtin_nontemporal_store(v, (u32x4*)(a.D + (size_t)(m0 + p) * a.ldd + n0 + c * 8));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dHidden = D . W  (R = D rows, C = W read K-major), K = the slice's vocabulary
// split in dh_splits() parts.  Part ks of every slice accumulates into fp32
// slab ks (the first slice writes it, later ones add to it: the slices run in
// stream order, so the order of the additions is fixed); k_dh_finish adds the
// slabs in a fixed order, applies the exact one-hot term and scatters rows to
// their positions.
// ---------------------------------------------------------------------------


// The fp32 tile leaves through LDS in two halves of 128 rows (the pipeline
// buffers, free after the main loop, hold 64 rows each): the waves owning a half write their
// accumulators into a 128 x 256 float table (16-column blocks XOR-swizzled by
// row so the four row groups of a wave's write land in distinct banks), then
// all threads move it as 16-byte vectors, one 1 KiB row per wave.  With
// `accumulate`, the slab's current values are loaded first, 8 coalesced
// loads per thread in flight together, and the sums stored.
__device__ __forceinline__ int dh_stage_col(int row, int col) { return col ^ (((row >> 2) & 3) << 4); }
// row r of a half: rows 0..63 in the first pipeline buffer, 64..127 in the second
__device__ __forceinline__ float* dh_stage(int row) {
  return (float*)(row < 64 ? g_stage0 : g_stage1) + (row & 63) * BN;
}

__device__ __forceinline__ void dh_store_tile(const Acc& acc, float* part, int m0, int n0, int n_c, int H,
                                              int accumulate, int tid, int lane, int wm, int wn) {
  constexpr int kIters = (BM / 2) * BN / 4 / NTHREADS;  // 16 float4 per thread per half
  constexpr int kBatch = 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < ACC_N; ++e) {
          const int row = i * FRAG + 4 * (lane >> 4) + e;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            dh_stage(row)[dh_stage_col(row, acc_col(wn, j, lane))] = acc.c[i][j][e];
        }
    }
    __syncthreads();
    // two batches of 8 vectors: 8 coalesced loads in flight per thread
#pragma unroll
    for (int b = 0; b < kIters; b += kBatch) {
      float4 old[kBatch];
      if (accumulate) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int g = (b + u) * NTHREADS + tid;
          const int row = g >> 6, c4 = g & 63;
          const int m = m0 + h * (BM / 2) + row, col = n0 + c4 * 4;
          old[u] = (m < n_c && col < H) ? *(const float4*)(part + (size_t)m * H + col)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int g = (b + u) * NTHREADS + tid;
        const int row = g >> 6, c4 = g & 63;
        const int m = m0 + h * (BM / 2) + row, col = n0 + c4 * 4;
        float4 v = *(const float4*)(dh_stage(row) + dh_stage_col(row, c4 * 4));
        if (accumulate) {
          v.x += old[u].x;
          v.y += old[u].y;
          v.z += old[u].z;
          v.w += old[u].w;
        }
        if (m < n_c && col < H) *(float4*)(part + (size_t)m * H + col) = v;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(NTHREADS) void k_dh_gemm(DhArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int n_c = a.hdr->n_c;
  const int nNt = cdiv(a.H, BN);
  const int nkt = a.Vp / BK;
  const int splitk = dh_splits(n_c, a.H, a.nkt_ref, gridDim.x, a.max_split, a.Mp);
  const int nks = cdiv(nkt, splitk);
  const size_t slab = dh_slab(n_c, a.H);
  Sched sc;
  sc.init(cdiv(n_c, BM), nNt * splitk, a.gm);
  for (int t = sc.begin; t < sc.end; t += sc.step) {
    int mt, ntk;
    sc.coords(t, mt, ntk);
    const int nt = ntk % nNt, ks = ntk / nNt;
    const int m0 = mt * BM, n0 = nt * BN;
    const int kb = ks * nks;
    const int nk = max(0, min(nks, nkt - kb));
    const RowOperand dop = row_operand(a.D + (size_t)m0 * a.ldd, a.ldd, (long)a.Mp - m0, kb * BK, tid);
    const KOperand wop = kmajor_operand(a.w + (size_t)kb * BK * a.H + n0, a.H, (long)a.V - kb * BK, tid);
    Acc acc;
    mainloop(acc, dop, wop, nk, wave, lane, wm, wn);
    float* part = a.part + (size_t)ks * slab;
    dh_store_tile(acc, part, m0, n0, n_c, a.H, a.accumulate, opaque(tid), opaque(lane), wm, wn);
    __syncthreads();
  }
}

// one block per completion position: dH = sum of the slabs - w W[target]
__global__ __launch_bounds__(256) void k_dh_finish(DhFinishArgs a) {
  const int m = blockIdx.x;
  const int n_c = a.hdr->n_c;
  if (m >= n_c) return;
  const int tg = a.tgt_c[m];
  const float wr = tg >= 0 ? a.weight[a.row_c[m]] : 0.f;
  const uint16_t* wrow = a.w + (size_t)(tg >= 0 ? tg : 0) * a.H;
  float* dst = a.d_hidden + (size_t)a.idx[m] * a.H;
  const int splitk = dh_splits(n_c, a.H, a.nkt_ref, a.grid, a.max_split, a.Mp);
  const size_t slab = dh_slab(n_c, a.H);
  for (int c = threadIdx.x * 4; c < a.H; c += 256 * 4) {
    float4 s = *(const float4*)(a.part + (size_t)m * a.H + c);
    for (int ks = 1; ks < splitk; ++ks) {
      const float4 p = *(const float4*)(a.part + ks * slab + (size_t)m * a.H + c);
      s.x += p.x;
      s.y += p.y;
      s.z += p.z;
      s.w += p.w;
    }
    const uint2 wv = *(const uint2*)(wrow + c);
    s.x = fmaf(-wr, bf16_lo(wv.x), s.x);
    s.y = fmaf(-wr, bf16_hi(wv.x), s.y);
    s.z = fmaf(-wr, bf16_lo(wv.y), s.z);
    s.w = fmaf(-wr, bf16_hi(wv.y), s.w);
    *(float4*)(dst + c) = s;
  }
}

// ---------------------------------------------------------------------------
// dW_vocab = D^T . Hc, K = completion positions, computed as its transpose
// (R = Hc^T rows, C = D read K-major)
// ---------------------------------------------------------------------------
// dW tile with exchanged roles: MFMA rows = hidden columns h, columns =
// vocabulary rows v, so the K-major operand (D) supplies the 4 column
// fragments (8 transposing reads per K step instead of 16).  The tile is
// transposed on its way out: waves holding vocabulary rows [128 hv, 128 hv +
// 128) write T[v][h..h+3] as 16-byte LDS writes (chunk c of row v at c ^ (v &
// 15): the 16 rows of a lane group land in distinct banks), then every thread
// moves 16-byte vectors of T's rows to dW[v][h].
__device__ __forceinline__ float* dwt_row(int v) {
  return (float*)(v < 64 ? g_stage0 : g_stage1) + (v & 63) * BM;
}
__device__ __forceinline__ void dwt_store_tile(const Acc& acc, float* dw, int h0, int v0, int V, int H, int accumulate,
                                               int tid, int lane, int wm, int wn) {
  constexpr int kIters = (BN / 2) * BM / 4 / NTHREADS;  // 16 float4 per thread per half
  constexpr int kBatch = 8;
#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    if ((wn >> 1) == hv) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int v = acc_col(wn, j, lane) - hv * (BN / 2);  // 0..127
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int c = (acc_row(wm, i, 0, lane)) >> 2;     // h chunk of 4
          *(floatx4*)(dwt_row(v) + ((c ^ (v & 15)) << 2)) = acc.c[i][j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kIters; b += kBatch) {
      float4 old[kBatch];
      if (accumulate) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int g = (b + u) * NTHREADS + tid;
          const int v = g >> 6, c4 = g & 63;
          const int vv = v0 + hv * (BN / 2) + v, col = h0 + c4 * 4;
          old[u] = (vv < V && col < H) ? *(const float4*)(dw + (size_t)vv * H + col) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int g = (b + u) * NTHREADS + tid;
        const int v = g >> 6, c4 = g & 63;
        const int vv = v0 + hv * (BN / 2) + v, col = h0 + c4 * 4;
        float4 x = *(const float4*)(dwt_row(v) + ((c4 ^ (v & 15)) << 2));
        if (accumulate) {
          x.x += old[u].x;
          x.y += old[u].y;
          x.z += old[u].z;
          x.w += old[u].w;
        }
        if (vv < V && col < H) *(float4*)(dw + (size_t)vv * H + col) = x;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(NTHREADS) void k_dw_gemm(DwArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int n_c = a.hdr->n_c;
  const int nk = cdiv(n_c, BK);
  Sched sc;
  sc.init(cdiv(a.H, BM), a.Vp / BN, a.gm);
  for (int t = sc.begin; t < sc.end; t += sc.step) {
    int mt, nt;
    sc.coords(t, mt, nt);
    const int h0 = mt * BM, v0 = nt * BN;
    const RowOperand hop = row_operand(a.ht + (size_t)h0 * a.ldt, a.ldt, (long)a.H - h0, 0, tid);
    const KOperand dop = kmajor_operand(a.D + v0, a.ldd, (long)align_up((size_t)n_c, BM), tid);
    Acc acc;
    mainloop(acc, hop, dop, nk, wave, lane, wm, wn);
    dwt_store_tile(acc, a.d_w, h0, v0, a.V, a.H, a.accumulate, opaque(tid), opaque(lane), wm, wn);
  }
}

// ---------------------------------------------------------------------------
// one-hot term of dW_vocab: positions sorted by target, then a fixed-order sum
// ---------------------------------------------------------------------------
// Stable LSD radix sort of the completion positions by target id, in one
// workgroup of 16 waves, in as few passes of at most 9-bit digits as cover
// the key range (two at vocabularies up to 2^18).  Each wave owns a
// contiguous slice of the input; per pass it counts its digits (LDS), the
// counts are scanned digit-major / wave-minor (one thread per digit over the
// waves, then one wave's prefix sum over the digits), and each wave scatters
// its slice 64 keys at a time: a key's rank among equal digits of its 64-key
// chunk comes from one ballot per digit bit (the lanes sharing all its digit
// bits), so equal keys keep their input order.  Out-of-range targets (-1)
// sort last.  The payload is the compact index of each position.
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortMaxDigits = 1 << kSortMaxBits;
constexpr int kSortBatch = 8;  // 64-key chunks whose loads are in flight together

// Lanes of the wave whose (valid) digit equals this lane's: one ballot per
// digit bit.
__device__ __forceinline__ unsigned long long digit_peers(int d, bool valid, int dbits) {
  const unsigned long long vmask = __ballot(valid);
  unsigned long long peers = vmask;
#pragma unroll
  for (int bit = 0; bit < kSortMaxBits; ++bit) {
    if (bit < dbits) {
      const bool set = (d >> bit) & 1;
      const unsigned long long bb = __ballot(valid && set);
      peers &= set ? bb : (vmask & ~bb);
    }
  }
  return peers;
}

// pass 0 reads the targets and maps the ones outside [0, V) to V
__device__ __forceinline__ int sort_key(const int* kin, int i, int pass, int V) {
  const int k = kin[i];
  return (pass > 0 || ((unsigned)k < (unsigned)V)) ? k : V;
}

__global__ __launch_bounds__(kSortThreads) void k_sort_targets(SortArgs a) {
  __shared__ int cnt[kSortWaves][kSortMaxDigits];
  __shared__ int dig_tot[kSortMaxDigits];
  __shared__ int dig_base[kSortMaxDigits];
  const int n = a.hdr->n_c;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int per = cdiv(n, kSortWaves);
  const int lo = min(n, per * wave), hi = min(n, lo + per);
  const unsigned long long below = (1ull << lane) - 1ull;
  const int nd = 1 << a.dbits;
  const unsigned dmask = (unsigned)nd - 1u;
  const int* kin = a.tgt_c;
  const int* vin = nullptr;
  int* kout = a.keysB;
  int* vout = a.valsB;
  for (int p = 0; p < a.passes; ++p) {
    const int shift = a.dbits * p;
    for (int d = lane; d < nd; d += 64) cnt[wave][d] = 0;
    __syncthreads();
    // keys are loaded kSortBatch chunks at a time, so one load latency
    // serves several chunks
    for (int base = lo; base < hi; base += 64 * kSortBatch) {
      int kk[kSortBatch];
#pragma unroll
      for (int j = 0; j < kSortBatch; ++j) {
        const int i = base + 64 * j + lane;
        kk[j] = i < hi ? sort_key(kin, i, p, a.V) : -1;
      }
      // one LDS add per distinct digit of a chunk (the lowest lane of each
      // group of equal digits): skewed targets would serialise per-key atomics
#pragma unroll
      for (int j = 0; j < kSortBatch; ++j) {
        if (base + 64 * j >= hi) break;
        const bool valid = kk[j] >= 0;
        const int d = (int)(((unsigned)kk[j] >> shift) & dmask);
        const unsigned long long peers = digit_peers(d, valid, a.dbits);
        if (valid && __popcll(peers & below) == 0) cnt[wave][d] += __popcll(peers);
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    for (int d = tid; d < nd; d += kSortThreads) {
      int run = 0;
      for (int w = 0; w < kSortWaves; ++w) {
        const int c = cnt[w][d];
        cnt[w][d] = run;
        run += c;
      }
      dig_tot[d] = run;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 8 l .. 8 l + 7: exclusive prefix sum over digits
      constexpr int kPer = kSortMaxDigits / 64;
      int v[kPer];
      int s = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int d = kPer * lane + j;
        v[j] = d < nd ? dig_tot[d] : 0;
        s += v[j];
      }
      int inc = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
      }
      int run = inc - s;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int d = kPer * lane + j;
        if (d < nd) dig_base[d] = run;
        run += v[j];
      }
    }
    __syncthreads();
    for (int base = lo; base < hi; base += 64 * kSortBatch) {
      int kk[kSortBatch], vv[kSortBatch];
#pragma unroll
      for (int j = 0; j < kSortBatch; ++j) {
        const int i = base + 64 * j + lane;
        kk[j] = i < hi ? sort_key(kin, i, p, a.V) : 0;
        vv[j] = i < hi ? (vin ? vin[i] : i) : 0;
      }
#pragma unroll
      for (int j = 0; j < kSortBatch; ++j) {
        if (base + 64 * j >= hi) break;
        const int i = base + 64 * j + lane;
        const bool valid = i < hi;
        const int k = kk[j];
        const int d = (int)(((unsigned)k >> shift) & dmask);
        const unsigned long long peers = digit_peers(d, valid, a.dbits);
        const int rank = __popcll(peers & below);
        const int slot = valid ? dig_base[d] + cnt[wave][d] + rank : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
          kout[slot] = k;
          vout[slot] = vv[j];
          if (rank == 0) cnt[wave][d] += __popcll(peers);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    kin = kout;
    vin = vout;
    kout = (kout == a.keysB) ? a.keysA : a.keysB;
    vout = (vout == a.valsB) ? a.valsA : a.valsB;
  }
}

// Two phases over the sorted list, cut in chunks of 64 entries (1024 columns
// per block, 4 per thread).  Phase 1 sums, in ascending position order, every
// piece of a run of equal targets that lies in its chunk: a run contained in
// the chunk is subtracted from its dW_vocab row at once; the piece of a run
// that started in an earlier chunk goes to cont[chunk], the piece of a run
// that continues into the next chunk goes to head[chunk].  Phase 2 adds, for
// each run that crosses chunks, head and the following cont pieces in chunk
// order and subtracts the total.  The order of every sum is fixed.
constexpr int kOnehotChunk = 64;
constexpr int kOnehotCols = 1024;
constexpr int kOnehotBatch = 8;  // hidden-row loads in flight per thread

__device__ __forceinline__ void sub4(float* dst, float4 v) {
  float4 d = *(float4*)dst;
  d.x -= v.x;
  d.y -= v.y;
  d.z -= v.z;
  d.w -= v.w;
  *(float4*)dst = d;
}

// The chunk's keys (with the entries on either side), positions and weights
// are staged in LDS once; the hidden-row loads are then issued a batch at a
// time, independent of where runs start and end, while each run is still
// summed entry by entry in ascending order.
__global__ __launch_bounds__(256) void k_onehot_dw(OnehotDwArgs a) {
  __shared__ int key_s[kOnehotChunk + 2];  // key_s[t] = keys[i0 - 1 + t]; -2 outside [0, n)
  __shared__ int pos_s[kOnehotChunk];
  __shared__ float w_s[kOnehotChunk];
  const int n = a.hdr->n_c;
  const int ch = blockIdx.x;
  const int i0 = ch * kOnehotChunk;
  if (i0 >= n) return;  // the whole block
  const int i1 = min(n, i0 + kOnehotChunk);
  const int m = i1 - i0;
  const int tid = threadIdx.x;
  if (tid < kOnehotChunk + 2) {
    const int i = i0 - 1 + tid;
    key_s[tid] = (i >= 0 && i < n) ? a.keys[i] : -2;
  }
  if (tid < kOnehotChunk) {
    // flat position and row weight of each sorted entry
    const int c = tid < m ? a.vals[i0 + tid] : 0;
    pos_s[tid] = tid < m ? a.idx[c] : 0;
    w_s[tid] = tid < m ? a.weight[a.row_c[c]] : 0.f;
  }
  __syncthreads();
  const int c0 = blockIdx.y * kOnehotCols + tid * 4;
  if (c0 >= a.H) return;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  bool starts_here = true;  // the current run began in this chunk
  for (int jb = 0; jb < m; jb += kOnehotBatch) {
    uint2 hh[kOnehotBatch];
#pragma unroll
    for (int u = 0; u < kOnehotBatch; ++u) {
      const int k = jb + u < m ? key_s[jb + u + 1] : -2;
      hh[u] = make_uint2(0u, 0u);
      if (k >= 0 && k < a.V) hh[u] = *(const uint2*)(a.hidden + (size_t)pos_s[jb + u] * a.H + c0);
    }
    // runs that start and end in this batch's entries: their dW rows are
    // updated together after the batch, so the row loads overlap
    int ek[kOnehotBatch];
    float4 ev[kOnehotBatch];
#pragma unroll
    for (int u = 0; u < kOnehotBatch; ++u) {
      ek[u] = -1;
      const int j = jb + u;
      if (j >= m) continue;
      const int k = key_s[j + 1];
      if (k < 0 || k >= a.V) continue;  // no target in this vocabulary range (sorted last)
      if (key_s[j] != k)
        starts_here = true;
      else if (j == 0)
        starts_here = false;
      const float w = w_s[j];
      acc0 = fmaf(w, bf16_lo(hh[u].x), acc0);
      acc1 = fmaf(w, bf16_hi(hh[u].x), acc1);
      acc2 = fmaf(w, bf16_lo(hh[u].y), acc2);
      acc3 = fmaf(w, bf16_hi(hh[u].y), acc3);
      const bool ends_here = key_s[j + 2] != k;  // the run ends at j (the sentinel covers j = n - 1)
      if (ends_here || j == m - 1) {
        const float4 v = make_float4(acc0, acc1, acc2, acc3);
        if (!starts_here)
          *(float4*)(a.cont + (size_t)ch * a.H + c0) = v;
        else if (!ends_here)
          *(float4*)(a.head + (size_t)ch * a.H + c0) = v;
        else {
          ek[u] = k;
          ev[u] = v;
        }
        acc0 = acc1 = acc2 = acc3 = 0.f;
      }
    }
    float4 dv[kOnehotBatch];
#pragma unroll
    for (int u = 0; u < kOnehotBatch; ++u)
      if (ek[u] >= 0) dv[u] = *(const float4*)(a.d_w + (size_t)ek[u] * a.H + c0);
#pragma unroll
    for (int u = 0; u < kOnehotBatch; ++u)
      if (ek[u] >= 0)
        *(float4*)(a.d_w + (size_t)ek[u] * a.H + c0) =
            make_float4(dv[u].x - ev[u].x, dv[u].y - ev[u].y, dv[u].z - ev[u].z, dv[u].w - ev[u].w);
  }
}

// Phase 2, one block per chunk whose last run crosses into the next chunk
// and starts in it: the block's threads test the following chunk boundaries
// in parallel to find the chunk where the run ends, then every thread adds
// head and the cont pieces in chunk order for its 4 columns.
__global__ __launch_bounds__(256) void k_onehot_dw_join(OnehotDwArgs a) {
  __shared__ int end_s;
  const int n = a.hdr->n_c;
  const int ch = blockIdx.x;
  const int i0 = ch * kOnehotChunk;
  if (i0 >= n) return;
  const int i1 = min(n, i0 + kOnehotChunk);
  if (i1 == n) return;
  const int k = a.keys[i1 - 1];
  if (a.keys[i1] != k || k < 0 || k >= a.V) return;  // the last run does not cross into the next chunk
  // an earlier chunk owns the run if it already ran through this chunk's start
  if (i0 > 0 && a.keys[i0] == k && a.keys[i0 - 1] == k) return;
  const int tid = threadIdx.x;
  const int nch = (n + kOnehotChunk - 1) / kOnehotChunk;
  // the first chunk c > ch whose end is the end of the run (every run ends by the last chunk)
  int last = nch - 1;
  for (int base = ch + 1; base < nch; base += 256) {
    if (tid == 0) end_s = nch;
    __syncthreads();
    const int c = base + tid;
    if (c < nch) {
      const int e = min(n, (c + 1) * kOnehotChunk);
      if (e == n || a.keys[e] != k) atomicMin(&end_s, c);
    }
    __syncthreads();
    const int found = end_s;
    __syncthreads();
    if (found < nch) {
      last = found;
      break;
    }
  }
  const int c0 = blockIdx.y * kOnehotCols + tid * 4;
  if (c0 >= a.H) return;
  float4 t = *(const float4*)(a.head + (size_t)ch * a.H + c0);
  for (int c = ch + 1; c <= last; ++c) {
    const float4 p = *(const float4*)(a.cont + (size_t)c * a.H + c0);
    t.x += p.x;
    t.y += p.y;
    t.z += p.z;
    t.w += p.w;
  }
  sub4(a.d_w + (size_t)k * a.H + c0, t);
}

// dHidden rows outside the completion mask are exactly zero.
__global__ __launch_bounds__(256) void k_zero_rows(ZeroRowsArgs a) {
  const long p = blockIdx.x;
  if (a.mask[p] != 0) return;
  float4* dst = (float4*)(a.d_hidden + p * a.H);
  for (int c = threadIdx.x; c < a.H / 4; c += 256) dst[c] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// The contractions' LDS (two 64 KiB stage buffers and the 8 KiB epilogue
// area, 136 KiB of the 160 KiB a CU has) is static, part of each kernel's
// code object: nothing is set up at launch.
hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_gemm(const FwdArgs& a, int grid, hipStream_t s) {
  if (a.part_z)
    hipLaunchKernelGGL(k_fwd_gemm<true>, dim3(grid), dim3(NTHREADS), 0, s, a);
  else
    hipLaunchKernelGGL(k_fwd_gemm<false>, dim3(grid), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_shard_partials(const ShardPartialArgs& a, int Mp, hipStream_t s) {
  hipLaunchKernelGGL(k_shard_partials, dim3(Mp / kCombPos), dim3(kCombPos * kCombGroups), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_shard_combine(const ShardCombineArgs& a, int Mp, hipStream_t s) {
  hipLaunchKernelGGL(k_shard_combine, dim3(Mp / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3(a.Mp / kCombPos), dim3(kCombPos * kCombGroups), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_row_sums(const RowSumArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_row_sums, dim3(a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_ht(const GatherHTArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_gather_ht, dim3(a.Mp / 64, a.H / 64), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dprod_gemm(const DProdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_dprod_gemm, dim3(grid), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dh_finish(const DhFinishArgs& a, int Mp, hipStream_t s) {
  hipLaunchKernelGGL(k_dh_finish, dim3(Mp), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dh_gemm(const DhArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_dh_gemm, dim3(grid), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dw_gemm(const DwArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_dw_gemm, dim3(grid), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sort_targets(const SortArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sort_targets, dim3(1), dim3(kSortThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_onehot_dw(const OnehotDwArgs& a, int Mp, hipStream_t s) {
  const dim3 grid(Mp / kOnehotChunk, cdiv(a.H, kOnehotCols));
  hipLaunchKernelGGL(k_onehot_dw, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_onehot_dw_join, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero_rows(const ZeroRowsArgs& a, long positions, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_rows, dim3((unsigned)positions), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dpo
