// Host-side checks of libgqa, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitize.py).
// Nothing here launches a kernel: every entry-point call either fails its
// argument checks, which run before any HIP call, or describes an empty
// problem, which returns before one. The planner of causal grids is plain C++
// and is run over many shapes, its output checked for consistency.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "gqa.h"
#include "plan.h"

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "check failed (line %d): %s; last error: %s\n", line, what, gqa_last_error());
    ++g_fail;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void* const P = reinterpret_cast<void*>(0x100000);  // aligned stand-in, never dereferenced
void* const M = reinterpret_cast<void*>(0x100004);  // misaligned stand-in
int32_t* const PI = static_cast<int32_t*>(P);
float* const PF = static_cast<float*>(P);

void check_entry_points() {
  // gqa_prefill
  EXPECT(gqa_prefill(P, P, P, P, 1, 6, 4, 16, 16, GQA_F32, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_last_error()[0] != '\0');
  EXPECT(gqa_prefill(P, P, P, P, -1, 4, 2, 16, 16, GQA_F32, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(P, P, P, P, 1, 4, 2, 16, 16, GQA_F32, GQA_F32, 0.0f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(P, P, P, P, 1, 4, 2, 16, 16, GQA_F32, GQA_F32, 0.25f, 3, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(P, P, P, M, 1, 4, 2, 16, 16, GQA_F32, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(nullptr, P, P, P, 1, 4, 2, 16, 16, GQA_F32, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(P, P, P, P, 1, 4, 2, 16, 48, GQA_BF16, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_prefill(P, P, P, P, 1, 4, 2, 16, 16, (gqa_dtype)9, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(P, P, P, P, 1, 1 << 20, 1, 1 << 12, 16, GQA_F32, GQA_F32, 0.25f, 1, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prefill(nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 16, 16, GQA_F32, GQA_F32, 0.25f, 1, nullptr) == GQA_OK);
  EXPECT(gqa_prefill(nullptr, nullptr, nullptr, nullptr, 2, 4, 2, 0, 16, GQA_BF16, GQA_F32, 0.25f, 1, nullptr) == GQA_OK);
  // gqa_decode
  const size_t ws = gqa_decode_workspace_bytes(4, 32, 8, 8192, 128);
  EXPECT(ws > 0);
  EXPECT(gqa_decode_workspace_bytes(0, 32, 8, 0, 128) == ws);
  EXPECT(gqa_decode_workspace_bytes(4, 32, 7, 8192, 128) == 0);
  EXPECT(gqa_decode_workspace_bytes(-1, 32, 8, 8192, 128) == 0);
  EXPECT(gqa_decode(P, P, P, PI, P, 4, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f, P, ws - 1, nullptr) == GQA_ERR_WORKSPACE);
  EXPECT(gqa_decode(P, P, P, PI, P, 4, 32, 8, 8192, 128, GQA_F32, GQA_BF16, 0.1f, P, ws, nullptr) == GQA_ERR_NO_DEVICE);
  EXPECT(gqa_decode(P, P, P, PI, P, 4, 32, 8, 8192, 128, (gqa_dtype)9, GQA_BF16, 0.1f, P, ws, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_decode(P, P, P, PI, P, 4, 32, 8, 8192, 48, GQA_BF16, GQA_BF16, 0.1f, P, ws, nullptr) == GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_decode(P, P, P, nullptr, P, 4, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f, P, ws, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_decode(P, P, P, PI, P, 4, 32, 8, -1, 128, GQA_BF16, GQA_BF16, 0.1f, P, ws, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_decode(P, P, P, PI, P, 4, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f, M, ws, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_decode(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f,
                    nullptr, 0, nullptr) == GQA_OK);
  // gqe_routed_decode
  EXPECT(gqe_routed_decode(P, P, P, PI, PF, 0, P, PI, PF, 4, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f, P, ws,
                           nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_routed_decode(P, P, P, PI, PF, 5, P, PI, PF, 4, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f, P, ws,
                           nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_routed_decode(P, P, P, PI, nullptr, 1, P, PI, PF, 4, 32, 8, 8192, 128, GQA_BF16, GQA_BF16, 0.1f, P,
                           ws, nullptr) == GQA_ERR_INVALID_ARG);
  // gqe_routed_prefill and its workspace query
  EXPECT(gqe_workspace_bytes(2, 32, 8, 4096, 128, 0) == 0);
  EXPECT(gqe_workspace_bytes(2, 32, 8, 4096, 48, 1) == 0);
  EXPECT(gqe_workspace_bytes(-2, 32, 8, 4096, 128, 1) == 0);
  for (int T : {1, 31, 32, 33, 100, 2048, 4096, 65536})
    for (int k : {1, 2, 4}) (void)gqe_workspace_bytes(2, 32, 8, T, 128, k);
  EXPECT(gqe_routed_prefill(P, P, P, PF, 0, P, PI, PF, 2, 32, 8, 64, 128, GQA_BF16, GQA_BF16, 0.1f, 1, nullptr, 0,
                            nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_routed_prefill(P, P, P, PF, 1, P, PI, PF, 2, 32, 8, 64, 128, GQA_BF16, GQA_BF16, 0.1f, 1, M, 1 << 20,
                            nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_routed_prefill(P, P, P, nullptr, 1, P, PI, PF, 2, 32, 8, 64, 128, GQA_BF16, GQA_BF16, 0.1f, 1, nullptr,
                            0, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_routed_prefill(P, P, P, PF, 1, P, PI, PF, 1, 256, 2, 64, 128, GQA_BF16, GQA_BF16, 0.1f, 1, nullptr, 0,
                            nullptr) == GQA_ERR_UNSUPPORTED);
  // gqe_prefill_build, gqe_router
  EXPECT(gqe_prefill_build(P, P, P, P, PF, 1, 8, P, P, P, PI, PF, 1, 16, 8, 64, 128, GQA_BF16, GQA_BF16, 0.1f, 1,
                           nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_prefill_build(P, P, P, P, PF, 1, 0, P, P, P, PI, PF, 1, 16, 8, 64, 128, GQA_F32, GQA_BF16, 0.1f, 1,
                           nullptr) == GQA_ERR_UNSUPPORTED);
  EXPECT(gqe_router(P, P, 1, nullptr, PI, PF, 64, 100, 32, 8, GQA_BF16, nullptr) == GQA_ERR_UNSUPPORTED);
  EXPECT(gqe_router(P, P, 5, nullptr, PI, PF, 64, 128, 32, 8, GQA_BF16, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_router(M, P, 1, nullptr, PI, PF, 64, 128, 32, 8, GQA_BF16, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqe_router(nullptr, nullptr, 1, nullptr, nullptr, nullptr, 0, 128, 32, 8, GQA_BF16, nullptr) == GQA_OK);
  // peaks, sizes, strings
  EXPECT(gqa_peak_hbm_read(P, 17, static_cast<uint32_t*>(P), nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_peak_hbm_read(P, 0, nullptr, nullptr) == GQA_OK);
  double fl = 0.0;
  EXPECT(gqa_peak_mfma_bf16(P, 0, PF, &fl, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_cache_bytes(32, 8, 16384, 128, GQA_BF16) == 2ull * 8 * 128 * 16384 * 2 * 32);
  EXPECT(gqa_kv_cache_bytes(-1, 8, 16384, 128, GQA_BF16) == 0);
  for (int s = -1; s < 8; ++s) EXPECT(gqa_status_string(static_cast<gqa_status>(s)) != nullptr);
  EXPECT(gqa_abi_version() >= 2);
}

// Every band appears once, whole, or twice as the two parts of a split at one
// key tile inside its range; split tiles are numbered 0 .. n_split-1.
void check_plan(const gqa::OrderShape& s) {
  const std::vector<gqa::Slot> v = gqa::plan_order(s);
  EXPECT((int)v.size() <= gqa::kMaxOrder);
  std::vector<int> whole(s.n_bands, 0), p1(s.n_bands, 0), p2(s.n_bands, 0), sp(s.n_bands, -1), sb(s.n_bands, -1);
  std::set<int> sbis;
  for (const gqa::Slot& x : v) {
    EXPECT(x.tile < s.n_bands);
    if (x.tile >= s.n_bands) continue;
    EXPECT(x.part <= 2);
    if (x.part == 0) {
      ++whole[x.tile];
      continue;
    }
    (x.part == 1 ? p1 : p2)[x.tile]++;
    const gqa::BandKeys k = gqa::band_keys(x.tile, s.rows, s.R, s.T, s.kBN);
    EXPECT(x.split >= 1 && x.split < k.n_tiles && x.split <= k.split);
    if (sp[x.tile] >= 0) EXPECT(sp[x.tile] == x.split && sb[x.tile] == x.sbi);
    sp[x.tile] = x.split;
    sb[x.tile] = x.sbi;
    sbis.insert(x.sbi);
  }
  int n_split = 0;
  for (int i = 0; i < s.n_bands; ++i) {
    EXPECT((whole[i] == 1 && p1[i] == 0 && p2[i] == 0) || (whole[i] == 0 && p1[i] == 1 && p2[i] == 1));
    n_split += p1[i];
  }
  EXPECT(n_split <= s.max_split);
  EXPECT((int)sbis.size() == n_split);
  for (int x : sbis) EXPECT(x < n_split);
}

void check_planner() {
  int n = 0;
  for (int T : {1, 33, 100, 2000, 2048, 4096, 8192})
    for (int R : {1, 2, 4})
      for (int rows : {256, 384})
        for (int kBN : {32, 64})
          for (int BG : {1, 16, 64})
            for (int B_sh : {0, 2})
              for (int n_cu : {80, 256}) {
                const int n_bands = (T * R + rows - 1) / rows;
                if (n_bands < 2 || n_bands > gqa::kMaxOrder) continue;
                const int cap = B_sh ? 0 : gqa::split_cap(n_bands, rows, R, T, kBN, BG, n_cu);
                EXPECT(cap >= 0 && cap <= gqa::kMaxOrder - n_bands);
                EXPECT((long long)cap * BG < n_cu);  // waiting second parts never hold every CU
                check_plan(gqa::OrderShape{n_bands, rows, R, T, kBN, BG, B_sh, n_cu, cap});
                ++n;
              }
  std::printf("planner: %d shapes checked\n", n);
}

}  // namespace

int main() {
  check_entry_points();
  check_planner();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
