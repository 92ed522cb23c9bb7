// Host-side checks of the library's workspace layouts, the index ranges its
// kernels reach inside them, and its argument validation.  Built with the host
// code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer and run
// without a GPU by tests/test_host_checks.py: every check here runs host code
// only (sizes, offsets, the split-count rule the kernels share, and entry
// points that must refuse their arguments before any launch).
#define DPO_HOST_CHECKS 1
#include "../preference_alignment_amd/csrc/dpo_api.hip"

#include <stdio.h>

#include <algorithm>
#include <vector>

static int g_failures = 0;
static int g_checks = 0;
#define CHECK(c)                                                             \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(c)) {                                                              \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);           \
      if (++g_failures > 50) return;                                         \
    }                                                                        \
  } while (0)

// bytes of the region that starts at `at` (0 if no region starts there)
static size_t region_bytes(const Layout& L, size_t at) {
  for (int i = 0; i < L.n_regions; ++i)
    if (L.regions[i].at == at) return L.regions[i].bytes;
  return 0;
}

static void check_layout(int op, int rows, int T, int H, int V) {
  const Layout L = make_layout(op, rows, T, H, V);
  // regions: 256-byte aligned, inside the total, disjoint
  CHECK(L.n_regions > 0 && L.n_regions < 32);
  std::vector<Layout::Region> r(L.regions, L.regions + L.n_regions);
  std::sort(r.begin(), r.end(), [](const Layout::Region& a, const Layout::Region& b) { return a.at < b.at; });
  for (size_t i = 0; i < r.size(); ++i) {
    CHECK(r[i].at % 256 == 0);
    CHECK(r[i].at + r[i].bytes <= L.total);
    if (i + 1 < r.size()) CHECK(r[i].at + r[i].bytes <= r[i + 1].at);
  }
  CHECK(dpo_workspace_bytes(op, rows, T, H, V) == L.total);
  if (op == DPO_OP_LOGITS_BACKWARD) return;
  const size_t Mp = (size_t)L.Mp;
  CHECK(Mp >= (size_t)rows * T && Mp % gemm::BM == 0);
  // completion indexing: compaction writes idx/tgt/row for every padded slot
  CHECK(region_bytes(L, L.idx) == Mp * 4 && region_bytes(L, L.tgt) == Mp * 4 && region_bytes(L, L.rowc) == Mp * 4);
  CHECK(region_bytes(L, L.rowoff) == (size_t)(rows + 1) * 4);
  const bool fwd = op == DPO_OP_SEQ_LOGPS || op == DPO_OP_REF_SCORE || op == DPO_OP_SEQ_LOGPS_METRICS;
  if (fwd) {
    // the forward tile (nt, position m) writes part[nt * Mp + m], nt < ceil(V / 256), m < Mp
    CHECK(region_bytes(L, L.part) >= (size_t)cdiv(V, gemm::BN) * Mp * sizeof(float2));
    CHECK(region_bytes(L, L.tlogit) >= Mp * 4);
  }
  if (op == DPO_OP_SEQ_LOGPS_METRICS) CHECK(region_bytes(L, L.partz) >= (size_t)cdiv(V, gemm::BN) * Mp * 4);
  if (op != DPO_OP_HEAD_BACKWARD) {
    CHECK(region_bytes(L, L.lse64) >= Mp * 8 && region_bytes(L, L.logp64) >= Mp * 8);
    return;
  }
  // backward: a slice of vocab_tiles <= chunk_tiles tiles; D rows < align(n_c, 256) <= Mp
  CHECK(L.chunk_tiles >= 1 && L.n_chunks == cdiv(L.nVt, L.chunk_tiles));
  CHECK((long long)(L.n_chunks - 1) * L.chunk_tiles < L.nVt);
  const size_t Vcp = (size_t)L.chunk_tiles * gemm::BN;
  CHECK((size_t)L.ldd >= Vcp && region_bytes(L, L.D) >= Mp * (size_t)L.ldd * 2);
  CHECK(Mp * Vcp * 2 <= kChunkBytes || L.chunk_tiles == 1);
  // Hc^T: H rows of ldt positions; the gather writes positions < align(n_c, 256) <= Mp < ldt
  CHECK((size_t)L.ldt > Mp && region_bytes(L, L.HT) >= (size_t)H * L.ldt * 2);
  // radix sort buffers: n_c <= Mp keys and values each
  CHECK(region_bytes(L, L.keysA) >= Mp * 4 && region_bytes(L, L.valsA) >= Mp * 4);
  CHECK(region_bytes(L, L.keysB) >= Mp * 4 && region_bytes(L, L.valsB) >= Mp * 4);
  // one-hot run pieces: one H-float row per 64-entry chunk, cdiv(n_c, 64) <= Mp / 64
  CHECK(region_bytes(L, L.ohcont) >= (Mp / 64) * H * 4 && region_bytes(L, L.ohhead) >= (Mp / 64) * H * 4);
  // dHidden slabs: for every completion count the device may meet, splits x
  // align(n_c, 256) x H floats stay inside the 2 Mp x H floats of the region
  const int nkt_ref = (int)(align_up((size_t)std::min(V, L.chunk_tiles * gemm::BN), gemm::BN) / gemm::BK);
  const size_t slab_floats = region_bytes(L, L.dhpart) / 4;
  CHECK(slab_floats >= 2 * Mp * H);
  const int grids[] = {1, 8, 80, 256, 304};
  const size_t step = std::max<size_t>(1, Mp / 97);
  for (size_t n_c = 0; n_c <= Mp; n_c += (n_c < 1024 ? 1 : step)) {
    for (int grid : grids) {
      const int s = gemm::dh_splits((int)n_c, H, nkt_ref, grid, 4, L.Mp);
      CHECK(s >= 1 && s <= 4);
      CHECK((size_t)s * gemm::dh_slab((int)n_c, H) <= slab_floats);
    }
  }
}

static void check_layouts() {
  const int ops[] = {DPO_OP_SEQ_LOGPS, DPO_OP_REF_SCORE, DPO_OP_HEAD_BACKWARD, DPO_OP_LOGITS_SEQ_LOGPS,
                     DPO_OP_LOGITS_BACKWARD, DPO_OP_SHARD_COMBINE, DPO_OP_SEQ_LOGPS_METRICS};
  struct Shape {
    int rows, T, H, V;
  };
  const Shape shapes[] = {{2, 1, 64, 8},        {4, 64, 256, 1024},     {8, 2048, 4096, 128256},
                          {128, 1024, 4096, 128256}, {4, 4096, 2048, 151936}, {8, 2048, 4096, 32064},
                          {2, 5, 64, 8},        {6, 300, 192, 1000},    {2, 8191, 320, 4104},
                          {2, 65536, 16320, 64}, {1024, 1024, 64, 1024}};
  for (int op : ops)
    for (const Shape& s : shapes) {
      const int H = op_needs_h(op) ? s.H : 0;
      if (!shape_ok(s.rows, s.T, H, s.V, op_needs_h(op)) || !backward_addressable(op, s.rows, s.T, H, s.V)) {
        CHECK(dpo_workspace_bytes(op, s.rows, s.T, H, s.V) == 0);
        continue;
      }
      check_layout(op, s.rows, s.T, H, s.V);
    }
}

// Entry points refuse bad arguments on the host, before any launch.  The
// pointers below are never dereferenced by host code.
static void check_validation() {
  char* const P = (char*)0x100000;          // 16-byte aligned stand-in
  char* const Q = (char*)0x100008;          // misaligned stand-in
  uint8_t* const M = (uint8_t*)0x200000;
  int32_t* const I = (int32_t*)0x300000;
  const size_t big = (size_t)1 << 40;
  // dpo_seq_logps
  CHECK(dpo_seq_logps(nullptr, (dpo_bf16*)P, I, M, 8, 64, 256, 1024, (float*)P, nullptr, nullptr, nullptr, P, big,
                      nullptr) == DPO_ERR_NULL);
  CHECK(dpo_seq_logps((dpo_bf16*)P, (dpo_bf16*)P, I, M, 7, 64, 256, 1024, (float*)P, nullptr, nullptr, nullptr, P,
                      big, nullptr) == DPO_ERR_SHAPE);
  CHECK(dpo_seq_logps((dpo_bf16*)P, (dpo_bf16*)P, I, M, 8, 64, 250, 1024, (float*)P, nullptr, nullptr, nullptr, P,
                      big, nullptr) == DPO_ERR_SHAPE);
  CHECK(dpo_seq_logps((dpo_bf16*)Q, (dpo_bf16*)P, I, M, 8, 64, 256, 1024, (float*)P, nullptr, nullptr, nullptr, P,
                      big, nullptr) == DPO_ERR_ALIGN);
  CHECK(dpo_seq_logps((dpo_bf16*)P, (dpo_bf16*)P, I, M, 8, 64, 256, 1024, (float*)P, nullptr, nullptr, nullptr, P,
                      16, nullptr) == DPO_ERR_WORKSPACE);
  // dpo_head_backward
  CHECK(dpo_head_backward((dpo_bf16*)P, (dpo_bf16*)P, I, M, 8, 64, 256, 1024, (float*)P, (float*)P, (float*)P,
                          (float*)P, 2, P, big, nullptr) == DPO_ERR_LAYOUT);
  CHECK(dpo_head_backward((dpo_bf16*)P, (dpo_bf16*)P, I, M, 8, 64, 256, 1024, (float*)P, (float*)P, (float*)Q,
                          (float*)P, 0, P, big, nullptr) == DPO_ERR_ALIGN);
  CHECK(dpo_head_backward((dpo_bf16*)P, (dpo_bf16*)P, I, M, 2, 1 << 22, 64, 1024, (float*)P, (float*)P,
                          (float*)P, (float*)P, 0, P, big, nullptr) == DPO_ERR_SHAPE);
  // dpo_loss / dpo_loss_ex
  CHECK(dpo_loss((double*)P, (float*)P, 4, 0.0, 0, (float*)P, (float*)P, nullptr, nullptr, nullptr, nullptr) ==
        DPO_ERR_BETA);
  CHECK(dpo_loss((double*)P, (float*)P, 4, 0.1, 7, (float*)P, (float*)P, nullptr, nullptr, nullptr, nullptr) ==
        DPO_ERR_LAYOUT);
  CHECK(dpo_loss((double*)P, (float*)P, 0, 0.1, 0, (float*)P, (float*)P, nullptr, nullptr, nullptr, nullptr) ==
        DPO_ERR_SHAPE);
  CHECK(dpo_loss_ex((double*)P, (float*)P, I, 4, 0.1, 0, 4, 0.0, (float*)P, (float*)P, nullptr, nullptr, nullptr,
                    nullptr, nullptr) == DPO_ERR_LAYOUT);
  CHECK(dpo_loss_ex((double*)P, (float*)P, I, 4, 0.1, 0, 0, -1.0, (float*)P, (float*)P, nullptr, nullptr, nullptr,
                    nullptr, nullptr) == DPO_ERR_ALPHA);
  CHECK(dpo_loss_ex((double*)P, nullptr, nullptr, 4, 0.1, 0, DPO_LOSS_LENGTH_NORM, 0.0, (float*)P, (float*)P,
                    nullptr, nullptr, nullptr, nullptr, nullptr) == DPO_ERR_NULL);
  // streaming entry points, shards, no-allocation forward
  CHECK(dpo_logits_seq_logps((dpo_bf16*)P, I, M, 8, 64, 1020, (float*)P, nullptr, nullptr, nullptr, P, big,
                             nullptr) == DPO_ERR_SHAPE);
  CHECK(dpo_logits_backward((dpo_bf16*)P, I, M, 8, 64, 1024, (float*)P, (float*)P, (dpo_bf16*)Q, P, big,
                            nullptr) == DPO_ERR_ALIGN);
  CHECK(dpo_seq_logps_shard((dpo_bf16*)P, (dpo_bf16*)P, I, M, 8, 64, 256, 256, 900, 1024, (float*)P, (float*)P,
                            (float*)P, P, big, nullptr) == DPO_ERR_SHAPE);
  CHECK(dpo_shard_combine((float*)P, (float*)P, (float*)P, 0, I, M, 8, 64, 1024, (float*)P, nullptr, nullptr,
                          nullptr, P, big, nullptr) == DPO_ERR_SHAPE);
  CHECK(dpo_logits_seq_logps_noalloc((dpo_bf16*)P, I, M, 2, (1 << 19) + 1, 8, (float*)P, nullptr, nullptr, nullptr,
                                     I, nullptr) == DPO_ERR_SCRATCH);
  CHECK(dpo_logits_seq_logps_noalloc((dpo_bf16*)P, I, M, 2, 16, 8, (float*)P, nullptr, nullptr, nullptr, nullptr,
                                     nullptr) == DPO_ERR_NULL);
  CHECK(dpo_logits_mean((double*)P, I, 4, 1024, 3, (float*)P, nullptr) == DPO_ERR_LAYOUT);
  // workspace sizes: unknown op, bad shapes
  CHECK(dpo_workspace_bytes(99, 8, 64, 256, 1024) == 0);
  CHECK(dpo_workspace_bytes(DPO_OP_SEQ_LOGPS, 8, 64, 256, 1020) == 0);
  CHECK(dpo_workspace_bytes(DPO_OP_SEQ_LOGPS, 2, 1 << 30, 64, 1024) == 0);
  // status strings and the host-only timing calls
  for (int c = 1; c >= -12; --c) CHECK(dpo_strerror(c) != nullptr);
  CHECK(dpo_profile_select("fwd_gemm") == DPO_OK && dpo_profile_select(nullptr) == DPO_OK);
  CHECK(dpo_profile_enable(0) == DPO_OK && dpo_profile_count() == 0);
  const char* name = nullptr;
  CHECK(dpo_profile_entry(0, &name, nullptr, nullptr) == DPO_ERR_SHAPE);
}

int main() {
  check_layouts();
  check_validation();
  printf("host checks: %d checks, %d failures\n", g_checks, g_failures);
  return g_failures ? 1 : 0;
}
