// Internal interface between the C-ABI host code and the kernel files.
// Argument structs are passed by value to kernels; all pointers are device
// pointers.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dpo_common.h"

namespace dpo {

struct CompactArgs {
  const uint8_t* mask;
  const int32_t* targets;
  int rows, T, Mp;
  int V;         // vocabulary rows this call works on (a shard's size, or the whole V)
  int v_begin;   // global id of its first row
  int V_total;   // whole vocabulary: targets outside [0, V_total) are errors
  WsHeader* hdr;
  int* idx;      // [Mp] flat position r*T+t of each completion position
  int* tgt_c;    // [Mp] its target relative to v_begin (-1: padding, out of range,
                 //      or held by another vocabulary shard)
  int* row_c;    // [Mp] its row
  int* row_off;  // [rows+1] first completion position of each row
  float* lse_out;  // [rows*T] nullable; zeroed at mask-0 positions
  float* off_max;  // [rows*T] nullable; -inf at mask-0 positions (shard partials)
  float* off_sum;  // [rows*T] nullable; 0 at mask-0 positions
  float* off_tgt;  // [rows*T] nullable; -inf at mask-0 positions
};

struct FwdArgs {
  const uint16_t* hidden;  // [rows*T, H]
  const uint16_t* w;       // [V, H]
  unsigned hidden_bytes;   // rows*T*H*2 (< 4 GiB)
  int H, V, Mp, gm;  // position tiles per scheduler group (narrow)
  int gn;  // vocabulary tiles per scheduler group while the hidden rows fit the cache budget
  const int* idx;
  const int* tgt_c;
  const WsHeader* hdr;
  float2* part;      // [nVt, Mp] per-tile (max, sum exp)
  float* tgt_logit;  // [Mp]
  float* part_z;     // [nVt, Mp] per-tile sum of the logits, or NULL
};

// one vocabulary shard's (max, sum exp, target logit) per position, [rows*T]
struct ShardPartialArgs {
  const float2* part;
  const float* tgt_logit;
  const int* tgt_c;
  const int* idx;
  const WsHeader* hdr;
  int Mp, nVt;
  float* out_max;
  float* out_sum;
  float* out_tgt;
};

struct ShardCombineArgs {
  const float* pmax;  // [S, rows*T]
  const float* psum;
  const float* ptgt;
  int S;
  long stride;  // rows*T
  const int* idx;
  const int* tgt_c;
  WsHeader* hdr;
  double* lse64;
  double* logp64;
  float* lse_out;  // nullable
};

struct CombineArgs {
  const float2* part;
  const float* tgt_logit;
  const int* tgt_c;
  const int* idx;
  const WsHeader* hdr;
  int Mp, nVt;
  double* lse64;   // [Mp]
  double* logp64;  // [Mp]
  float* lse_out;  // [rows*T] nullable
  const float* part_z;  // [nVt, Mp] per-tile logit sums, or NULL
  double* zsum64;       // [Mp] per position: sum of its V logits (with part_z)
};

struct RowSumArgs {
  const double* logp64;
  const int* row_off;
  const WsHeader* hdr;
  int rows;
  float* sum32;     // nullable
  double* sum64;    // nullable
  int32_t* n_tokens;  // nullable
};

struct GatherHTArgs {
  const uint16_t* hidden;
  const int* idx;
  const WsHeader* hdr;
  int H, Mp, ldt;
  uint16_t* ht;  // [H, ldt]: row h holds the completion positions' h-th entries
};

struct DProdArgs {
  int ldd;  // D row stride (elements)
  const uint16_t* hidden;
  const uint16_t* w;
  unsigned hidden_bytes;  // rows*T*H*2 (< 4 GiB)
  int H, V, Vp, Mp, gm;  // position tiles per scheduler group (narrow)
  int gn;  // vocabulary tiles per scheduler group while the hidden rows fit the cache budget
  const int* idx;
  const int* tgt_c;
  const int* row_c;
  const WsHeader* hdr;
  const float* lse;     // [rows*T] from the forward
  const float* weight;  // [rows]
  uint16_t* D;          // [Mp, Vp] bf16
};

struct DhArgs {
  int ldd;  // D row stride (elements)
  const uint16_t* D;    // [Mp, Vp] the slice's D
  const uint16_t* w;    // [V, H] the slice's rows of W_vocab, read K-major (K = vocabulary)
  int H, V, Vp, Mp, gm;
  int max_split;  // the kernel splits K into dh_splits(...) <= this many parts
  int nkt_ref;    // K steps of the first slice: every slice and the finish choose the same split count
  int accumulate;  // 0: the first slice writes the slabs; 1: later slices add to them
  const WsHeader* hdr;
  float* part;  // split slabs, each align(n_c, 256) x H fp32, 2 Mp x H floats in all
};

struct DhFinishArgs {
  const float* part;
  const uint16_t* w;    // [V, H] for the exact one-hot term
  const int* idx;
  const int* tgt_c;
  const int* row_c;
  const float* weight;  // [rows]
  const WsHeader* hdr;
  int H, Mp;
  int max_split;
  int nkt_ref, grid;  // as for k_dh_gemm: the same split count
  float* d_hidden;  // [rows*T, H]
};

struct SortArgs {
  const int* tgt_c;     // [n_c] keys in position order
  const WsHeader* hdr;
  int V;                // keys outside [0, V) sort last, as V
  int passes;           // radix passes covering keys 0..V
  int dbits;            // digit bits per pass (at most kSortMaxBits)
  int* keysA;
  int* valsA;
  int* keysB;
  int* valsB;
};

struct OnehotDwArgs {
  const int* keys;      // [n_c] targets, sorted
  const int* vals;      // [n_c] compact indices, ascending within a target
  const int* idx;       // [n_c] flat position of each compact index
  const int* row_c;     // [n_c] row of each compact index
  const float* weight;  // [rows]
  const uint16_t* hidden;
  const WsHeader* hdr;
  int H, V;
  float* cont;  // [Mp/64, H] piece of a run that started in an earlier chunk
  float* head;  // [Mp/64, H] piece of a run that continues into the next chunk
  float* d_w;
};

struct DwArgs {
  int ldd;  // D row stride (elements)
  const uint16_t* D;    // [Mp, Vp] the slice's D, read K-major (K = positions)
  const uint16_t* ht;   // [H, ldt]
  int V, H, Vp, Mp, ldt, gm, accumulate;
  const WsHeader* hdr;
  float* d_w;  // [V, H]
};

struct ZeroRowsArgs {
  const uint8_t* mask;
  int H;
  float* d_hidden;
};

// The streaming kernels are instantiated for bf16 (uint16_t bits) and fp32
// logits; `logits` / `d_logits` point to that element type.
struct StreamFwdArgs {
  const void* logits;  // [rows*T, V]
  const int32_t* targets;  // [rows*T]
  const uint8_t* mask;     // [rows*T]
  int V;
  WsHeader* hdr;     // status word, reset here and set by the row sums
  double* logp64;    // [rows*T] log p at completion positions, 0 elsewhere
  int* bad;          // [rows*T] 1 where the target is outside [0, V)
  float* lse_out;    // nullable
};

struct StreamRowSumArgs {
  const double* logp64;
  const int* bad;
  const uint8_t* mask;
  WsHeader* hdr;
  int rows, T;
  float* sum32;       // nullable
  double* sum64;      // nullable
  int32_t* n_tokens;  // nullable
};

struct StreamBwdArgs {
  const void* logits;
  const int32_t* targets;
  const uint8_t* mask;
  int T, V;
  const float* lse;     // [rows*T]
  const float* weight;  // [rows]
  WsHeader* hdr;
  void* d_logits;       // [rows*T, V], the input's element type
};

struct LossArgs {
  const double* policy;  // [2B]
  const float* ref;      // [2B]; NULL: reference-free
  const int32_t* n_tokens;  // [2B]; needed for length normalisation and the NLL term
  int num_pairs, layout;
  int length_norm;       // divide row scores by their token counts
  double beta;
  double alpha;          // weight of the NLL term on chosen rows (0: none)
  float* nll;       // [1] nullable
  float* loss;      // [1]
  float* weight;    // [2B]
  float* reward;    // [2B] nullable
  float* margin;    // [B] nullable
  float* accuracy;  // [1] nullable
};

hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
hipError_t launch_fwd_gemm(const FwdArgs& a, int grid, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_row_sums(const RowSumArgs& a, hipStream_t s);
hipError_t launch_gather_ht(const GatherHTArgs& a, hipStream_t s);
hipError_t launch_dprod_gemm(const DProdArgs& a, int grid, hipStream_t s);
hipError_t launch_dh_gemm(const DhArgs& a, int grid, hipStream_t s);
hipError_t launch_dh_finish(const DhFinishArgs& a, int Mp, hipStream_t s);
hipError_t launch_dw_gemm(const DwArgs& a, int grid, hipStream_t s);
hipError_t launch_zero_rows(const ZeroRowsArgs& a, long positions, hipStream_t s);
hipError_t launch_sort_targets(const SortArgs& a, hipStream_t s);
hipError_t launch_onehot_dw(const OnehotDwArgs& a, int Mp, hipStream_t s);
constexpr int kSortThreads = 1024;
constexpr int kSortMaxBits = 9;
hipError_t launch_stream_fwd(const StreamFwdArgs& a, long positions, hipStream_t s);
hipError_t launch_stream_row_sums(const StreamRowSumArgs& a, hipStream_t s);
hipError_t launch_stream_bwd(const StreamBwdArgs& a, long positions, int grid, hipStream_t s);
hipError_t launch_reset_status(WsHeader* hdr, hipStream_t s);
hipError_t launch_write_status(const WsHeader* hdr, int code, int32_t* out, hipStream_t s);
hipError_t launch_loss(const LossArgs& a, hipStream_t s);
hipError_t launch_shard_partials(const ShardPartialArgs& a, int Mp, hipStream_t s);
hipError_t launch_shard_combine(const ShardCombineArgs& a, int Mp, hipStream_t s);
hipError_t launch_stream_fwd_f32(const StreamFwdArgs& a, long positions, hipStream_t s);
hipError_t launch_stream_bwd_f32(const StreamBwdArgs& a, long positions, int grid, hipStream_t s);

struct LogitsMeanArgs {
  const double* logit_sum;  // [2B]
  const int32_t* n_tokens;  // [2B]
  int num_pairs, layout, V;
  float* means;  // [2]: chosen, rejected
};
hipError_t launch_logits_mean(const LogitsMeanArgs& a, hipStream_t s);

}  // namespace dpo
