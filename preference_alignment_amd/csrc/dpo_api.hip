// Host side of the C ABI declared in include/dpo_head.h: argument validation,
// workspace layout, kernel sequencing on the caller's stream, device status
// and optional per-kernel timing.  No device memory is allocated here.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <mutex>
#include <string>
#include <vector>

#include "dpo_head.h"
#include "dpo_common.h"
#include "gemm_core.h"
#include "launch.h"

using namespace dpo;

namespace {

// Tile-group widths of the persistent scheduler: position tiles per group
// (kGroupFwd, kGroupBwd) and, for the forward-shaped contractions while the
// gathered hidden rows fit the cache budget, vocabulary tiles per group.
constexpr int kGroupFwd = 8;
constexpr int kGroupFwdVocab = 4;
constexpr int kGroupBwd = 4;
// The dHidden contraction has few output tiles (positions x H): its K =
// vocabulary range is split in up to this many parts, the count chosen on the
// device from N_c so that the last round of tiles is nearly full.  The parts'
// fp32 slabs take at most 2 Mp x H floats (the device caps the count to fit),
// and every vocabulary slice adds into the same slabs.
constexpr int kMaxSplitDh = 4;
// The backward holds the bf16 softmax part of dlogits (D) only for one slice
// of the vocabulary at a time: D's columns stay under this many bytes
// (balanced slices of whole 256-wide tiles; each D row carries a 128-byte pad).
constexpr size_t kChunkBytes = size_t(2) << 30;
// output tiles one round of the persistent contractions covers (one per CU of MI355X)
constexpr int kRoundTiles = 256;
constexpr int kTransPad = 64;  // elements
constexpr int kDPad = 64;      // elements: D rows 128 bytes off a power-of-two stride
// workgroups per CU of the chunked streaming backward
constexpr int kStreamBwdBlocksPerCU = 32;

// ---------------------------------------------------------------------------
// static scratch of the no-allocation entry point
// ---------------------------------------------------------------------------
// dpo_logits_seq_logps_noalloc keeps its scratch (status header, per-position
// fp64 log p and target flags) in this file-scope device array instead of a
// caller workspace, for callers that cannot allocate.  Each GPU the library
// runs on holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns for the current device.
constexpr long kNoAllocMaxPositions = 1L << 20;  // rows * T
constexpr size_t kScratchLogpOff = 256;
constexpr size_t kScratchBadOff = kScratchLogpOff + (size_t)kNoAllocMaxPositions * 8;
constexpr size_t kScratchBytes = kScratchBadOff + (size_t)kNoAllocMaxPositions * 4;  // 12 MiB + 256 B
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
char* g_scratch_addr[kMaxDevices] = {};

// The scratch's device address on the current device, looked up once per device.
int noalloc_scratch(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DPO_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DPO_ERR_HIP;
    g_scratch_addr[dev] = (char*)p;
  }
  *out = g_scratch_addr[dev];
  return DPO_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct Layout {
  int Mp = 0;   // completion positions rounded up to the GEMM tile (upper bound rows*T)
  int Vp = 0;   // vocabulary rounded up to the GEMM tile
  int nVt = 0;  // vocabulary tiles of the forward contraction
  int chunk_tiles = 0;  // vocabulary tiles per backward slice
  int ldd = 0;          // D row stride (elements)
  int n_chunks = 0;
  int ldt = 0;  // row stride (elements) of Hc^T: positions plus a pad
  size_t hdr = 0, idx = 0, tgt = 0, rowc = 0, rowoff = 0;
  size_t part = 0, tlogit = 0, lse64 = 0, logp64 = 0, partz = 0, zsum64 = 0;
  size_t D = 0, HT = 0;
  size_t keysA = 0, valsA = 0, keysB = 0, valsB = 0, dhpart = 0, ohcont = 0, ohhead = 0;
  size_t total = 0;
#ifdef DPO_HOST_CHECKS
  // every region the layout hands out (offset, bytes), for the host-side checks
  struct Region {
    size_t at, bytes;
  } regions[32];
  int n_regions = 0;
#endif
};

bool op_needs_h(int op) {
  return op == DPO_OP_SEQ_LOGPS || op == DPO_OP_REF_SCORE || op == DPO_OP_HEAD_BACKWARD ||
         op == DPO_OP_SEQ_LOGPS_METRICS;
}

bool op_known(int op) { return op >= DPO_OP_SEQ_LOGPS && op <= DPO_OP_SEQ_LOGPS_METRICS; }

bool shape_ok(int rows, int T, int H, int V, bool need_h) {
  if (rows <= 0 || (rows & 1) || T <= 0 || V <= 0 || (V % 8)) return false;
  if ((long long)rows * T >= (1LL << 31) - gemm::BM) return false;
  if (V >= (1 << 30)) return false;
  if (need_h && (H <= 0 || H % 64 || H >= (1 << 30))) return false;
  // the hidden tensor is addressed with 32-bit byte offsets
  if (need_h && (long long)rows * T * H * 2 >= (1LL << 32)) return false;
  return true;
}

Layout make_layout(int op, int rows, int T, int H, int V) {
  Layout L;
  const size_t A = 256;
  const long long positions = (long long)rows * T;
  L.Mp = (int)align_up((size_t)positions, gemm::BM);
  L.Vp = (int)align_up((size_t)V, gemm::BN);
  L.nVt = cdiv(V, gemm::BN);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, A);
#ifdef DPO_HOST_CHECKS
    if (L.n_regions < 32) L.regions[L.n_regions++] = {at, bytes};
#endif
    return at;
  };
  L.hdr = take(sizeof(WsHeader));
  if (op == DPO_OP_LOGITS_BACKWARD) {
    L.total = o;
    return L;
  }
  L.idx = take((size_t)L.Mp * 4);
  L.tgt = take((size_t)L.Mp * 4);
  L.rowc = take((size_t)L.Mp * 4);
  L.rowoff = take((size_t)(rows + 1) * 4);
  const bool fwd = op == DPO_OP_SEQ_LOGPS || op == DPO_OP_REF_SCORE || op == DPO_OP_SEQ_LOGPS_METRICS;
  if (fwd) {
    L.part = take((size_t)L.nVt * L.Mp * sizeof(float2));
    L.tlogit = take((size_t)L.Mp * 4);
  }
  if (op == DPO_OP_SEQ_LOGPS_METRICS) {
    L.partz = take((size_t)L.nVt * L.Mp * 4);
    L.zsum64 = take((size_t)L.Mp * 8);
  }
  if (op != DPO_OP_HEAD_BACKWARD) {
    L.lse64 = take((size_t)L.Mp * 8);
    L.logp64 = take((size_t)L.Mp * 8);
  }
  if (op == DPO_OP_HEAD_BACKWARD) {
    const size_t tile_bytes = (size_t)L.Mp * gemm::BN * 2;
    const int max_tiles = (int)std::max<size_t>(1, std::min<size_t>(L.nVt, kChunkBytes / tile_bytes));
    // whole slices of a multiple of q tiles, so that a slice's dW contraction
    // (slice tiles x H / 256 output tiles) fills whole rounds of the CUs
    const int nNt = cdiv(H, gemm::BN);
    const int q = kRoundTiles / std::gcd(kRoundTiles, nNt);
    L.chunk_tiles = max_tiles >= L.nVt ? L.nVt : (max_tiles >= q ? max_tiles / q * q : max_tiles);
    L.n_chunks = cdiv(L.nVt, L.chunk_tiles);
    const size_t Vcp = (size_t)L.chunk_tiles * gemm::BN;
    // Hc^T rows are positions long; a pad of 128 bytes keeps their stride off
    // a power of two (2^15 bytes at 16,384 positions), where all rows of a
    // tile would fall on the same HBM channels
    L.ldt = L.Mp + kTransPad;
    // D rows: a pad of 128 bytes keeps their stride off a power of two
    // (131,072 bytes at 256 tiles), as for Hc^T below
    L.ldd = Vcp + kDPad;
    L.D = take((size_t)L.Mp * L.ldd * 2);
    L.HT = take((size_t)H * L.ldt * 2);
    L.keysA = take((size_t)L.Mp * 4);
    L.valsA = take((size_t)L.Mp * 4);
    L.keysB = take((size_t)L.Mp * 4);
    L.valsB = take((size_t)L.Mp * 4);
    // fp32 dHidden partial slabs, one per K split (at most 2 Mp x H floats in
    // all); every slice adds into them, the finish sums them
    L.dhpart = take((size_t)2 * L.Mp * H * 4);
    L.ohcont = take((size_t)(L.Mp / 64) * H * 4);
    L.ohhead = take((size_t)(L.Mp / 64) * H * 4);
  }
  L.total = o;
  return L;
}

// The backward's contractions address one vocabulary slice of D and of W
// with 32-bit byte offsets: both must stay under 4 GiB.
bool backward_addressable(int op, int rows, int T, int H, int V) {
  if (op != DPO_OP_HEAD_BACKWARD) return true;
  const Layout L = make_layout(op, rows, T, H, V);
  const size_t vc = (size_t)L.chunk_tiles * gemm::BN;
  return (size_t)L.Mp * L.ldd * 2 < (size_t(1) << 32) && vc * (size_t)H * 2 < (size_t(1) << 32);
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------------
// device facts
// ---------------------------------------------------------------------------
int persistent_grid() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    // the tile scheduler cuts the tiles into one part per XCD (blockIdx % 8):
    // a grid of fewer than 8 blocks would leave parts unvisited
    cus[dev] = std::max(n, gemm::NUM_XCD);
  }
  return cus[dev];
}


// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
struct ProfSum {
  std::string name;
  double ms;
  int n;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;  // empty: time every kernel
std::vector<ProfRec> g_prof_pending;
std::vector<ProfSum> g_prof_sums;

void prof_clear_locked() {
  for (auto& r : g_prof_pending) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  g_prof_pending.clear();
  g_prof_sums.clear();
}

void prof_drain_locked() {
  for (auto& r : g_prof_pending) {
    float ms = 0.f;
    hipEventSynchronize(r.b);
    hipEventElapsedTime(&ms, r.a, r.b);
    bool found = false;
    for (auto& s : g_prof_sums)
      if (s.name == r.name) {
        s.ms += ms;
        s.n += 1;
        found = true;
        break;
      }
    if (!found) g_prof_sums.push_back({r.name, (double)ms, 1});
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  g_prof_pending.clear();
}

// Runs `f` (which enqueues one kernel on `s`), bracketed by events when timing is on.
template <typename F>
hipError_t timed(const char* name, hipStream_t s, F f) {
  bool on;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    on = g_prof_on && (g_prof_only.empty() || g_prof_only == name);
  }
  if (!on) return f();
  // timing-only events: no system-scope fence (an L2 write-back and
  // invalidate) when they are recorded, which would otherwise sit between the
  // timed kernels and slow the work that follows
  hipEvent_t a, b;
  if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return hipErrorUnknown;
  if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
    hipEventDestroy(a);
    return hipErrorUnknown;
  }
  hipEventRecord(a, s);
  hipError_t e = f();
  hipEventRecord(b, s);
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_pending.push_back({name, a, b});
  return e;
}

#define RUN(name, call)                                     \
  do {                                                      \
    hipError_t _e = timed(name, st, [&]() { return call; }); \
    if (_e != hipSuccess) return DPO_ERR_HIP;               \
  } while (0)

// ---------------------------------------------------------------------------
// shared pieces of the entry points
// ---------------------------------------------------------------------------
int check_common(const void* targets, const void* mask, int rows, int T, int H, int V, bool need_h,
                 int op, size_t ws_bytes, const void* ws) {
  if (!targets || !mask || !ws) return DPO_ERR_NULL;
  if (!shape_ok(rows, T, H, V, need_h) || !backward_addressable(op, rows, T, H, V)) return DPO_ERR_SHAPE;
  if (!aligned16(ws)) return DPO_ERR_ALIGN;
  if (ws_bytes < make_layout(op, rows, T, H, V).total) return DPO_ERR_WORKSPACE;
  return DPO_OK;
}

// Vocabulary slice a call works on: rows [v_begin, v_begin + V) of a
// vocabulary of V_total (the whole vocabulary: v_begin = 0, V_total = V).
struct VocabSlice {
  int v_begin, V_total;
};

struct OffMask {
  float* max = nullptr;
  float* sum = nullptr;
  float* tgt = nullptr;
};

int enqueue_compact(const Layout& L, void* ws, const int32_t* targets, const uint8_t* mask, int rows,
                    int T, int V, float* lse_out, hipStream_t st, VocabSlice vs = {0, -1},
                    OffMask off = OffMask()) {
  CompactArgs c;
  c.mask = mask;
  c.targets = targets;
  c.rows = rows;
  c.T = T;
  c.V = V;
  c.v_begin = vs.v_begin;
  c.V_total = vs.V_total < 0 ? V : vs.V_total;
  c.off_max = off.max;
  c.off_sum = off.sum;
  c.off_tgt = off.tgt;
  c.Mp = L.Mp;
  c.hdr = at<WsHeader>(ws, L.hdr);
  c.idx = at<int>(ws, L.idx);
  c.tgt_c = at<int>(ws, L.tgt);
  c.row_c = at<int>(ws, L.rowc);
  c.row_off = at<int>(ws, L.rowoff);
  c.lse_out = lse_out;
  RUN("compact", launch_compact(c, st));
  return DPO_OK;
}

// compaction + the forward contraction; leaves per-tile partials in the workspace
int enqueue_forward_tiles(const dpo_bf16* hidden, const dpo_bf16* w, const int32_t* targets,
                          const uint8_t* mask, int rows, int T, int H, int V, float* lse, void* ws,
                          int op, hipStream_t st, VocabSlice vs, OffMask off, FwdArgs& f) {
  const Layout L = make_layout(op, rows, T, H, V);
  int rc = enqueue_compact(L, ws, targets, mask, rows, T, V, lse, st, vs, off);
  if (rc) return rc;
  f.hidden = hidden;
  f.w = w;
  f.hidden_bytes = (unsigned)((size_t)rows * T * H * 2);
  f.H = H;
  f.V = V;
  f.Mp = L.Mp;
  f.gm = kGroupFwd;
  f.gn = kGroupFwdVocab;
  f.idx = at<int>(ws, L.idx);
  f.tgt_c = at<int>(ws, L.tgt);
  f.hdr = at<WsHeader>(ws, L.hdr);
  f.part = at<float2>(ws, L.part);
  f.tgt_logit = at<float>(ws, L.tlogit);
  f.part_z = op == DPO_OP_SEQ_LOGPS_METRICS ? at<float>(ws, L.partz) : nullptr;
  RUN("fwd_gemm", launch_fwd_gemm(f, persistent_grid(), st));
  return DPO_OK;
}

int enqueue_fused_forward(const dpo_bf16* hidden, const dpo_bf16* w, const int32_t* targets,
                          const uint8_t* mask, int rows, int T, int H, int V, float* sum32,
                          double* sum64, float* lse, int32_t* n_tokens, void* ws, int op,
                          hipStream_t st, double* logit_sum = nullptr) {
  const Layout L = make_layout(op, rows, T, H, V);
  FwdArgs f;
  int rc = enqueue_forward_tiles(hidden, w, targets, mask, rows, T, H, V, lse, ws, op, st, {0, V},
                                 OffMask(), f);
  if (rc) return rc;
  CombineArgs c;
  c.part = f.part;
  c.tgt_logit = f.tgt_logit;
  c.tgt_c = f.tgt_c;
  c.idx = f.idx;
  c.hdr = f.hdr;
  c.Mp = L.Mp;
  c.nVt = L.nVt;
  c.lse64 = at<double>(ws, L.lse64);
  c.logp64 = at<double>(ws, L.logp64);
  c.lse_out = lse;
  c.part_z = f.part_z;
  c.zsum64 = f.part_z ? at<double>(ws, L.zsum64) : nullptr;
  RUN("combine", launch_combine(c, st));
  RowSumArgs r;
  r.logp64 = c.logp64;
  r.row_off = at<int>(ws, L.rowoff);
  r.hdr = f.hdr;
  r.rows = rows;
  r.sum32 = sum32;
  r.sum64 = sum64;
  r.n_tokens = n_tokens;
  RUN("row_sums", launch_row_sums(r, st));
  if (logit_sum) {
    RowSumArgs q;
    q.logp64 = c.zsum64;
    q.row_off = r.row_off;
    q.hdr = f.hdr;
    q.rows = rows;
    q.sum32 = nullptr;
    q.sum64 = logit_sum;
    q.n_tokens = nullptr;
    RUN("logit_row_sums", launch_row_sums(q, st));
  }
  return DPO_OK;
}

int check_slice(int V_shard, int v_begin, int V_total) {
  if (v_begin < 0 || V_total <= 0 || V_total >= (1 << 30) || (long long)v_begin + V_shard > V_total)
    return DPO_ERR_SHAPE;
  return DPO_OK;
}

int enqueue_head_backward(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                          const uint8_t* mask, int rows, int T, int H, int V, VocabSlice vs,
                          const float* lse, const float* weight, float* d_hidden, float* d_w_vocab,
                          int accumulate_dw, void* workspace, hipStream_t st);

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

size_t dpo_workspace_bytes(int op, int rows, int T, int H, int V) {
  if (!op_known(op)) return 0;
  const bool need_h = op_needs_h(op);
  if (!shape_ok(rows, T, H, V, need_h) || !backward_addressable(op, rows, T, H, V)) return 0;
  return make_layout(op, rows, T, need_h ? H : 0, V).total;
}

int dpo_seq_logps(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                  const uint8_t* mask, int rows, int T, int H, int V, float* logp_sum,
                  double* logp_sum64, float* lse, int32_t* n_tokens, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!hidden || !w_vocab || !logp_sum) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, H, V, true, DPO_OP_SEQ_LOGPS, workspace_bytes, workspace);
  if (rc) return rc;
  if (!aligned16(hidden) || !aligned16(w_vocab) || !aligned16(logp_sum) ||
      (logp_sum64 && !aligned16(logp_sum64)) || (lse && !aligned16(lse)))
    return DPO_ERR_ALIGN;
  return enqueue_fused_forward(hidden, w_vocab, targets, mask, rows, T, H, V, logp_sum, logp_sum64,
                               lse, n_tokens, workspace, DPO_OP_SEQ_LOGPS, (hipStream_t)stream);
}

int dpo_ref_score(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                  const uint8_t* mask, int rows, int T, int H, int V, float* ref_sum,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!hidden || !w_vocab || !ref_sum) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, H, V, true, DPO_OP_REF_SCORE, workspace_bytes, workspace);
  if (rc) return rc;
  if (!aligned16(hidden) || !aligned16(w_vocab) || !aligned16(ref_sum)) return DPO_ERR_ALIGN;
  return enqueue_fused_forward(hidden, w_vocab, targets, mask, rows, T, H, V, ref_sum, nullptr,
                               nullptr, nullptr, workspace, DPO_OP_REF_SCORE, (hipStream_t)stream);
}

int dpo_seq_logps_metrics(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                          const uint8_t* mask, int rows, int T, int H, int V, float* logp_sum,
                          double* logp_sum64, float* lse, int32_t* n_tokens, double* logit_sum,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!hidden || !w_vocab || !logp_sum || !logit_sum) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, H, V, true, DPO_OP_SEQ_LOGPS_METRICS, workspace_bytes,
                        workspace);
  if (rc) return rc;
  if (!aligned16(hidden) || !aligned16(w_vocab) || !aligned16(logp_sum) || !aligned16(logit_sum) ||
      (logp_sum64 && !aligned16(logp_sum64)) || (lse && !aligned16(lse)))
    return DPO_ERR_ALIGN;
  return enqueue_fused_forward(hidden, w_vocab, targets, mask, rows, T, H, V, logp_sum, logp_sum64,
                               lse, n_tokens, workspace, DPO_OP_SEQ_LOGPS_METRICS, (hipStream_t)stream,
                               logit_sum);
}

int dpo_logits_mean(const double* logit_sum, const int32_t* n_tokens, int num_pairs, int V, int layout,
                    float* means, void* stream) {
  if (!logit_sum || !n_tokens || !means) return DPO_ERR_NULL;
  if (num_pairs <= 0 || num_pairs >= (1 << 29) || V <= 0) return DPO_ERR_SHAPE;
  if (layout != DPO_PAIRS_ADJACENT && layout != DPO_PAIRS_HALVES) return DPO_ERR_LAYOUT;
  hipStream_t st = (hipStream_t)stream;
  LogitsMeanArgs a{logit_sum, n_tokens, num_pairs, layout, V, means};
  RUN("logits_mean", launch_logits_mean(a, st));
  return DPO_OK;
}

int dpo_seq_logps_shard(const dpo_bf16* hidden, const dpo_bf16* w_shard, const int32_t* targets,
                        const uint8_t* mask, int rows, int T, int H, int V_shard, int v_begin, int V_total,
                        float* part_max, float* part_sumexp, float* part_tgt, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!hidden || !w_shard || !part_max || !part_sumexp || !part_tgt) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, H, V_shard, true, DPO_OP_SEQ_LOGPS, workspace_bytes,
                        workspace);
  if (rc) return rc;
  rc = check_slice(V_shard, v_begin, V_total);
  if (rc) return rc;
  if (!aligned16(hidden) || !aligned16(w_shard) || !aligned16(part_max) || !aligned16(part_sumexp) ||
      !aligned16(part_tgt))
    return DPO_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const Layout L = make_layout(DPO_OP_SEQ_LOGPS, rows, T, H, V_shard);
  OffMask off;
  off.max = part_max;
  off.sum = part_sumexp;
  off.tgt = part_tgt;
  FwdArgs f;
  rc = enqueue_forward_tiles(hidden, w_shard, targets, mask, rows, T, H, V_shard, nullptr, workspace,
                             DPO_OP_SEQ_LOGPS, st, {v_begin, V_total}, off, f);
  if (rc) return rc;
  ShardPartialArgs p;
  p.part = f.part;
  p.tgt_logit = f.tgt_logit;
  p.tgt_c = f.tgt_c;
  p.idx = f.idx;
  p.hdr = f.hdr;
  p.Mp = L.Mp;
  p.nVt = L.nVt;
  p.out_max = part_max;
  p.out_sum = part_sumexp;
  p.out_tgt = part_tgt;
  RUN("shard_partials", launch_shard_partials(p, L.Mp, st));
  return DPO_OK;
}

int dpo_shard_combine(const float* part_max, const float* part_sumexp, const float* part_tgt,
                      int num_shards, const int32_t* targets, const uint8_t* mask, int rows, int T,
                      int V_total, float* logp_sum, double* logp_sum64, float* lse, int32_t* n_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!part_max || !part_sumexp || !part_tgt || !logp_sum) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, 0, V_total, false, DPO_OP_SHARD_COMBINE, workspace_bytes,
                        workspace);
  if (rc) return rc;
  if (num_shards <= 0 || num_shards > 4096 || (long long)num_shards * rows * T >= (1LL << 40))
    return DPO_ERR_SHAPE;
  if (!aligned16(part_max) || !aligned16(part_sumexp) || !aligned16(part_tgt) || !aligned16(logp_sum) ||
      (logp_sum64 && !aligned16(logp_sum64)) || (lse && !aligned16(lse)))
    return DPO_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const Layout L = make_layout(DPO_OP_SHARD_COMBINE, rows, T, 0, V_total);
  rc = enqueue_compact(L, workspace, targets, mask, rows, T, V_total, lse, st);
  if (rc) return rc;
  ShardCombineArgs c;
  c.pmax = part_max;
  c.psum = part_sumexp;
  c.ptgt = part_tgt;
  c.S = num_shards;
  c.stride = (long)rows * T;
  c.idx = at<int>(workspace, L.idx);
  c.tgt_c = at<int>(workspace, L.tgt);
  c.hdr = at<WsHeader>(workspace, L.hdr);
  c.lse64 = at<double>(workspace, L.lse64);
  c.logp64 = at<double>(workspace, L.logp64);
  c.lse_out = lse;
  RUN("shard_combine", launch_shard_combine(c, L.Mp, st));
  RowSumArgs r;
  r.logp64 = c.logp64;
  r.row_off = at<int>(workspace, L.rowoff);
  r.hdr = c.hdr;
  r.rows = rows;
  r.sum32 = logp_sum;
  r.sum64 = logp_sum64;
  r.n_tokens = n_tokens;
  RUN("row_sums", launch_row_sums(r, st));
  return DPO_OK;
}

int dpo_loss_ex(const double* policy_sum64, const float* ref_sum, const int32_t* n_tokens, int num_pairs,
                double beta, int layout, int flags, double sft_alpha, float* loss, float* weight,
                float* reward, float* margin, float* accuracy, float* nll, void* stream) {
  if (!policy_sum64 || !loss || !weight) return DPO_ERR_NULL;
  if (flags & ~(DPO_LOSS_LENGTH_NORM | DPO_LOSS_REFERENCE_FREE)) return DPO_ERR_LAYOUT;
  const bool ref_free = (flags & DPO_LOSS_REFERENCE_FREE) != 0;
  const bool length_norm = (flags & DPO_LOSS_LENGTH_NORM) != 0;
  if (!ref_free && !ref_sum) return DPO_ERR_NULL;
  if (!(isfinite(sft_alpha) && sft_alpha >= 0.0)) return DPO_ERR_ALPHA;
  if ((length_norm || sft_alpha > 0.0 || nll) && !n_tokens) return DPO_ERR_NULL;
  if (num_pairs <= 0 || num_pairs >= (1 << 29)) return DPO_ERR_SHAPE;
  if (!(isfinite(beta) && beta > 0.0)) return DPO_ERR_BETA;
  if (layout != DPO_PAIRS_ADJACENT && layout != DPO_PAIRS_HALVES) return DPO_ERR_LAYOUT;
  hipStream_t st = (hipStream_t)stream;
  LossArgs a;
  a.policy = policy_sum64;
  a.ref = ref_free ? nullptr : ref_sum;
  a.n_tokens = (length_norm || sft_alpha > 0.0 || nll) ? n_tokens : nullptr;
  a.num_pairs = num_pairs;
  a.layout = layout;
  a.length_norm = length_norm ? 1 : 0;
  a.beta = beta;
  a.alpha = sft_alpha;
  a.nll = nll;
  a.loss = loss;
  a.weight = weight;
  a.reward = reward;
  a.margin = margin;
  a.accuracy = accuracy;
  RUN("loss", launch_loss(a, st));
  return DPO_OK;
}

int dpo_loss(const double* policy_sum64, const float* ref_sum, int num_pairs, double beta, int layout,
             float* loss, float* weight, float* reward, float* margin, float* accuracy, void* stream) {
  if (!policy_sum64 || !ref_sum || !loss || !weight) return DPO_ERR_NULL;
  return dpo_loss_ex(policy_sum64, ref_sum, nullptr, num_pairs, beta, layout, 0, 0.0, loss, weight, reward,
                     margin, accuracy, nullptr, stream);
}

int dpo_head_backward(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                      const uint8_t* mask, int rows, int T, int H, int V, const float* lse,
                      const float* weight, float* d_hidden, float* d_w_vocab, int accumulate_dw,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!hidden || !w_vocab || !lse || !weight || !d_hidden || !d_w_vocab) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, H, V, true, DPO_OP_HEAD_BACKWARD, workspace_bytes,
                        workspace);
  if (rc) return rc;
  if (accumulate_dw != 0 && accumulate_dw != 1) return DPO_ERR_LAYOUT;
  if (!aligned16(hidden) || !aligned16(w_vocab) || !aligned16(lse) || !aligned16(d_hidden) ||
      !aligned16(d_w_vocab))
    return DPO_ERR_ALIGN;
  return enqueue_head_backward(hidden, w_vocab, targets, mask, rows, T, H, V, {0, V}, lse, weight,
                               d_hidden, d_w_vocab, accumulate_dw, workspace, (hipStream_t)stream);
}

int dpo_head_backward_shard(const dpo_bf16* hidden, const dpo_bf16* w_shard, const int32_t* targets,
                            const uint8_t* mask, int rows, int T, int H, int V_shard, int v_begin,
                            int V_total, const float* lse, const float* weight, float* d_hidden,
                            float* d_w_shard, int accumulate_dw, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!hidden || !w_shard || !lse || !weight || !d_hidden || !d_w_shard) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, H, V_shard, true, DPO_OP_HEAD_BACKWARD, workspace_bytes,
                        workspace);
  if (rc) return rc;
  rc = check_slice(V_shard, v_begin, V_total);
  if (rc) return rc;
  if (accumulate_dw != 0 && accumulate_dw != 1) return DPO_ERR_LAYOUT;
  if (!aligned16(hidden) || !aligned16(w_shard) || !aligned16(lse) || !aligned16(d_hidden) ||
      !aligned16(d_w_shard))
    return DPO_ERR_ALIGN;
  return enqueue_head_backward(hidden, w_shard, targets, mask, rows, T, H, V_shard, {v_begin, V_total},
                               lse, weight, d_hidden, d_w_shard, accumulate_dw, workspace,
                               (hipStream_t)stream);
}

}  // extern "C"

namespace {
int enqueue_head_backward(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                          const uint8_t* mask, int rows, int T, int H, int V, VocabSlice vs,
                          const float* lse, const float* weight, float* d_hidden, float* d_w_vocab,
                          int accumulate_dw, void* workspace, hipStream_t st) {
  const Layout L = make_layout(DPO_OP_HEAD_BACKWARD, rows, T, H, V);
  void* ws = workspace;
  int rc = enqueue_compact(L, ws, targets, mask, rows, T, V, nullptr, st, vs);
  if (rc) return rc;
  WsHeader* hdr = at<WsHeader>(ws, L.hdr);
  uint16_t* D = at<uint16_t>(ws, L.D);
  uint16_t* HT = at<uint16_t>(ws, L.HT);

  GatherHTArgs gh{hidden, at<int>(ws, L.idx), hdr, H, L.Mp, L.ldt, HT};
  RUN("gather_ht", launch_gather_ht(gh, st));

  // vocabulary slices: D for the slice; the first slice writes the
  // dHidden partial slabs and later slices add to them in stream order (the
  // finish sums the slabs in a fixed order); each slice's dW rows are complete
  float* dh_part = at<float>(ws, L.dhpart);
  // K steps of the first (widest) slice: the dHidden split count depends on it
  const int nkt_ref = (int)(align_up((size_t)std::min(V, L.chunk_tiles * gemm::BN), gemm::BN) / gemm::BK);
  for (int c = 0; c < L.n_chunks; ++c) {
    const int v0 = c * L.chunk_tiles * gemm::BN;
    const int Vc = std::min(V - v0, L.chunk_tiles * gemm::BN);
    const int Vcp = (int)align_up((size_t)Vc, gemm::BN);
    DProdArgs dp;
    dp.hidden = hidden;
    dp.w = w_vocab + (size_t)v0 * H;
    dp.hidden_bytes = (unsigned)((size_t)rows * T * H * 2);
    dp.H = H;
    dp.V = Vc;
    dp.Vp = Vcp;
    dp.ldd = L.ldd;
    dp.Mp = L.Mp;
    dp.gm = kGroupFwd;
    dp.gn = kGroupFwdVocab;
    dp.idx = at<int>(ws, L.idx);
    dp.tgt_c = at<int>(ws, L.tgt);
    dp.row_c = at<int>(ws, L.rowc);
    dp.hdr = hdr;
    dp.lse = lse;
    dp.weight = weight;
    dp.D = D;
    RUN("dlogits_gemm", launch_dprod_gemm(dp, persistent_grid(), st));

    DhArgs dh;
    dh.D = D;
    dh.w = w_vocab + (size_t)v0 * H;
    dh.H = H;
    dh.V = Vc;
    dh.Vp = Vcp;
    dh.ldd = L.ldd;
    dh.Mp = L.Mp;
    dh.gm = kGroupBwd;
    dh.max_split = kMaxSplitDh;
    dh.nkt_ref = nkt_ref;
    dh.hdr = hdr;
    dh.part = dh_part;
    dh.accumulate = c > 0;
    RUN("dhidden_gemm", launch_dh_gemm(dh, persistent_grid(), st));

    DwArgs dw;
    dw.D = D;
    dw.ht = HT;
    dw.V = Vc;
    dw.H = H;
    dw.Vp = Vcp;
    dw.ldd = L.ldd;
    dw.Mp = L.Mp;
    dw.ldt = L.ldt;
    dw.gm = kGroupBwd;
    dw.accumulate = accumulate_dw;
    dw.hdr = hdr;
    dw.d_w = d_w_vocab + (size_t)v0 * H;
    RUN("dw_gemm", launch_dw_gemm(dw, persistent_grid(), st));
  }
  const int* idx_c = at<int>(ws, L.idx);
  const int* tgt_c = at<int>(ws, L.tgt);
  const int* row_c = at<int>(ws, L.rowc);

  DhFinishArgs df;
  df.part = dh_part;
  df.w = w_vocab;
  df.idx = idx_c;
  df.tgt_c = tgt_c;
  df.row_c = row_c;
  df.weight = weight;
  df.hdr = hdr;
  df.H = H;
  df.Mp = L.Mp;
  df.max_split = kMaxSplitDh;
  df.nkt_ref = nkt_ref;
  df.grid = persistent_grid();
  df.d_hidden = d_hidden;
  RUN("dhidden_finish", launch_dh_finish(df, L.Mp, st));

  ZeroRowsArgs z{mask, H, d_hidden};
  RUN("zero_rows", launch_zero_rows(z, (long)rows * T, st));

  // one-hot term of dW_vocab: sort positions by target, subtract per-target sums
  // (keys span [0, V], V standing for "no target in this slice")
  int bits = 1;
  while (bits < 31 && (1 << bits) <= V) ++bits;
  SortArgs so;
  so.tgt_c = tgt_c;
  so.hdr = hdr;
  so.V = V;
  so.passes = (bits + kSortMaxBits - 1) / kSortMaxBits;
  so.dbits = (bits + so.passes - 1) / so.passes;
  so.keysA = at<int>(ws, L.keysA);
  so.valsA = at<int>(ws, L.valsA);
  so.keysB = at<int>(ws, L.keysB);
  so.valsB = at<int>(ws, L.valsB);
  RUN("sort_targets", launch_sort_targets(so, st));
  OnehotDwArgs oh;
  oh.keys = (so.passes & 1) ? so.keysB : so.keysA;
  oh.vals = (so.passes & 1) ? so.valsB : so.valsA;
  oh.idx = idx_c;
  oh.row_c = row_c;
  oh.weight = weight;
  oh.hidden = hidden;
  oh.hdr = hdr;
  oh.H = H;
  oh.V = V;
  oh.cont = at<float>(ws, L.ohcont);
  oh.head = at<float>(ws, L.ohhead);
  oh.d_w = d_w_vocab;
  RUN("onehot_dw", launch_onehot_dw(oh, L.Mp, st));
  return DPO_OK;
}
}  // namespace

namespace {
// the two launches of the logits forward, on explicit scratch pointers
int enqueue_logits_forward(const void* logits, bool f32, const int32_t* targets, const uint8_t* mask, int rows,
                           int T, int V, float* logp_sum, double* logp_sum64, float* lse, int32_t* n_tokens,
                           WsHeader* hdr, double* logp64, int* bad, hipStream_t st) {
  StreamFwdArgs f;
  f.logits = logits;
  f.targets = targets;
  f.mask = mask;
  f.V = V;
  f.hdr = hdr;
  f.logp64 = logp64;
  f.bad = bad;
  f.lse_out = lse;
  if (f32)
    RUN("stream_fwd_f32", launch_stream_fwd_f32(f, (long)rows * T, st));
  else
    RUN("stream_fwd", launch_stream_fwd(f, (long)rows * T, st));
  StreamRowSumArgs r;
  r.logp64 = f.logp64;
  r.bad = f.bad;
  r.mask = mask;
  r.hdr = f.hdr;
  r.rows = rows;
  r.T = T;
  r.sum32 = logp_sum;
  r.sum64 = logp_sum64;
  r.n_tokens = n_tokens;
  RUN("row_sums", launch_stream_row_sums(r, st));
  return DPO_OK;
}

int logits_forward(const void* logits, bool f32, const int32_t* targets, const uint8_t* mask, int rows,
                   int T, int V, float* logp_sum, double* logp_sum64, float* lse, int32_t* n_tokens,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !logp_sum) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, 0, V, false, DPO_OP_LOGITS_SEQ_LOGPS, workspace_bytes,
                        workspace);
  if (rc) return rc;
  if (!aligned16(logits) || !aligned16(logp_sum) || (logp_sum64 && !aligned16(logp_sum64)) ||
      (lse && !aligned16(lse)))
    return DPO_ERR_ALIGN;
  const Layout L = make_layout(DPO_OP_LOGITS_SEQ_LOGPS, rows, T, 0, V);
  void* ws = workspace;
  return enqueue_logits_forward(logits, f32, targets, mask, rows, T, V, logp_sum, logp_sum64, lse, n_tokens,
                                at<WsHeader>(ws, L.hdr), at<double>(ws, L.logp64), at<int>(ws, L.idx),
                                (hipStream_t)stream);
}

int logits_backward(const void* logits, bool f32, const int32_t* targets, const uint8_t* mask, int rows,
                    int T, int V, const float* lse, const float* weight, void* d_logits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!logits || !lse || !weight || !d_logits) return DPO_ERR_NULL;
  int rc = check_common(targets, mask, rows, T, 0, V, false, DPO_OP_LOGITS_BACKWARD, workspace_bytes,
                        workspace);
  if (rc) return rc;
  if (!aligned16(logits) || !aligned16(lse) || !aligned16(d_logits)) return DPO_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const Layout L = make_layout(DPO_OP_LOGITS_BACKWARD, rows, T, 0, V);
  WsHeader* hdr = at<WsHeader>(workspace, L.hdr);
  RUN("reset_status", launch_reset_status(hdr, st));
  StreamBwdArgs b;
  b.logits = logits;
  b.targets = targets;
  b.mask = mask;
  b.T = T;
  b.V = V;
  b.lse = lse;
  b.weight = weight;
  b.hdr = hdr;
  b.d_logits = d_logits;
  if (f32)
    RUN("stream_bwd_f32", launch_stream_bwd_f32(b, (long)rows * T, persistent_grid() * kStreamBwdBlocksPerCU, st));
  else
    RUN("stream_bwd", launch_stream_bwd(b, (long)rows * T, persistent_grid() * kStreamBwdBlocksPerCU, st));
  return DPO_OK;
}
}  // namespace

extern "C" {

int dpo_logits_seq_logps(const dpo_bf16* logits, const int32_t* targets, const uint8_t* mask, int rows,
                         int T, int V, float* logp_sum, double* logp_sum64, float* lse,
                         int32_t* n_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return logits_forward(logits, false, targets, mask, rows, T, V, logp_sum, logp_sum64, lse, n_tokens,
                        workspace, workspace_bytes, stream);
}

int dpo_logits_backward(const dpo_bf16* logits, const int32_t* targets, const uint8_t* mask, int rows,
                        int T, int V, const float* lse, const float* weight, dpo_bf16* d_logits,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return logits_backward(logits, false, targets, mask, rows, T, V, lse, weight, d_logits, workspace,
                         workspace_bytes, stream);
}

int dpo_logits_f32_seq_logps(const float* logits, const int32_t* targets, const uint8_t* mask, int rows,
                             int T, int V, float* logp_sum, double* logp_sum64, float* lse,
                             int32_t* n_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return logits_forward(logits, true, targets, mask, rows, T, V, logp_sum, logp_sum64, lse, n_tokens,
                        workspace, workspace_bytes, stream);
}

int dpo_logits_f32_backward(const float* logits, const int32_t* targets, const uint8_t* mask, int rows,
                            int T, int V, const float* lse, const float* weight, float* d_logits,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return logits_backward(logits, true, targets, mask, rows, T, V, lse, weight, d_logits, workspace,
                         workspace_bytes, stream);
}

int dpo_logits_seq_logps_noalloc(const dpo_bf16* logits, const int32_t* targets, const uint8_t* mask,
                                 int rows, int T, int V, float* logp_sum, double* logp_sum64, float* lse,
                                 int32_t* n_tokens, int32_t* status, void* stream) {
  if (!logits || !targets || !mask || !logp_sum || !status) return DPO_ERR_NULL;
  if (!shape_ok(rows, T, 0, V, false)) return DPO_ERR_SHAPE;
  if ((long long)rows * T > kNoAllocMaxPositions) return DPO_ERR_SCRATCH;
  if (!aligned16(logits) || !aligned16(logp_sum) || (logp_sum64 && !aligned16(logp_sum64)) ||
      (lse && !aligned16(lse)))
    return DPO_ERR_ALIGN;
  char* base = nullptr;
  int rc = noalloc_scratch(&base);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  WsHeader* hdr = (WsHeader*)base;
  rc = enqueue_logits_forward(logits, false, targets, mask, rows, T, V, logp_sum, logp_sum64, lse, n_tokens, hdr,
                              (double*)(base + kScratchLogpOff), (int*)(base + kScratchBadOff), st);
  if (rc) return rc;
  RUN("write_status", launch_write_status(hdr, DPO_ERR_TARGET_RANGE, status, st));
  return DPO_OK;
}

int dpo_device_status(void* workspace, void* stream) {
  if (!workspace) return DPO_ERR_NULL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DPO_ERR_HIP;
  int status = 0;
  if (hipMemcpy(&status, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return DPO_ERR_HIP;
  return (status & kStatusTargetRange) ? DPO_ERR_TARGET_RANGE : DPO_OK;
}

const char* dpo_strerror(int status) {
  switch (status) {
    case DPO_OK: return "ok";
    case DPO_ERR_NULL: return "a required pointer is NULL";
    case DPO_ERR_SHAPE: return "sizes break the shape rules (rows even > 0, T,H,V > 0, H % 64 == 0, V % 8 == 0)";
    case DPO_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case DPO_ERR_BETA: return "beta must be finite and > 0";
    case DPO_ERR_LAYOUT: return "unknown pair layout or flag value";
    case DPO_ERR_WORKSPACE: return "workspace smaller than dpo_workspace_bytes()";
    case DPO_ERR_TARGET_RANGE:
      return "a target id at a completion position is outside [0, V) (or no vocabulary shard holds it)";
    case DPO_ERR_HIP: return "a HIP runtime call failed";
    case DPO_ERR_ALPHA: return "sft_alpha must be finite and >= 0";
    case DPO_ERR_SCRATCH: return "rows * T exceeds the 2^20 positions of the no-allocation scratch";
    default: return "unknown status";
  }
}

int dpo_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  prof_drain_locked();
  prof_clear_locked();
  g_prof_on = on != 0;
  return DPO_OK;
}

int dpo_profile_select(const char* name) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_only = name ? name : "";
  return DPO_OK;
}

int dpo_profile_count(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  prof_drain_locked();
  return (int)g_prof_sums.size();
}

int dpo_profile_entry(int i, const char** name, double* total_ms, int* launches) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  prof_drain_locked();
  if (i < 0 || i >= (int)g_prof_sums.size()) return DPO_ERR_SHAPE;
  if (name) *name = g_prof_sums[i].name.c_str();
  if (total_ms) *total_ms = g_prof_sums[i].ms;
  if (launches) *launches = g_prof_sums[i].n;
  return DPO_OK;
}

}  // extern "C"
