// Host-only driver of the C ABI for the sanitizer test: every call here is
// rejected (or answered) by the host-side validation layer before any device
// work, so it runs on a machine without a GPU.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code; exits nonzero on a wrong status.
#include <cstdint>
#include <cstdio>
#include <climits>

#include "dsa.h"

static int failures = 0;

static void expect(const char* what, long long got, long long want) {
  if (got != want) {
    std::printf("FAIL %s: got %lld want %lld\n", what, got, want);
    ++failures;
  }
}

int main() {
  alignas(256) static unsigned char buf[4096];
  void* p = buf;
  const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
  const float* fp = reinterpret_cast<const float*>(buf);
  int32_t* op = reinterpret_cast<int32_t*>(buf);
  const int64_t big = INT64_MAX, ibig = INT32_MAX;

  for (int s = -10; s <= 1; ++s) {
    const char* m = dsa_status_string(s);
    if (!m || !m[0]) ++failures;
  }
  expect("version", dsa_version() > 0, 1);

  // windows
  expect("windows n_seqs 0", dsa_row_windows(ip, ip, 0, 4, 1, op, op, nullptr), DSA_ERR_INVALID_ARG);
  expect("windows null", dsa_row_windows(nullptr, ip, 1, 4, 1, op, op, nullptr), DSA_ERR_INVALID_ARG);
  expect("windows huge rows", dsa_row_windows(ip, ip, 1, big, 1, op, op, nullptr), DSA_ERR_INVALID_ARG);

  // workspace queries: extreme sizes must not overflow (the answer is either a
  // size or SIZE_MAX, never a wrapped small value)
  const size_t ws1 = dsa_topk_workspace_size(big, big, INT32_MAX);
  const size_t ws2 = dsa_topk_workspace_size(ibig, ibig, 65536);
  const size_t ws3 = dsa_indexer_topk_workspace_size(big, big, 64, 128, 1, INT32_MAX);
  const size_t ws4 = dsa_indexer_topk_workspace_size(ibig, ibig, 64, 128, 0, 2048);
  const size_t ws5 = dsa_sparse_mla_workspace_size(big, INT32_MAX, 576, 512, INT32_MAX, 1);
  const size_t ws6 = dsa_sparse_mla_workspace_size(ibig, 128, 576, 512, 2048, 2);
  const size_t ws7 = dsa_sparse_mla_workspace_size(1, INT32_MAX, 576, 512, INT32_MAX, 1);
  expect("topk ws extreme", ws1 == SIZE_MAX, 1);
  expect("indexer_topk ws extreme", ws3 == SIZE_MAX, 1);
  expect("mla ws extreme", ws5 == SIZE_MAX, 1);
  expect("topk ws large", ws2 >= (size_t(1) << 20) || ws2 == 0, 1);
  expect("indexer_topk ws large", ws4 > (size_t(ibig) * 4), 1);
  std::printf("ws: %zu %zu %zu %zu %zu %zu %zu\n", ws1, ws2, ws3, ws4, ws5, ws6, ws7);
  expect("ws small", dsa_topk_workspace_size(0, 10, 4) == 0, 1);

  // top-k
  expect("topk k 0", dsa_topk(fp, 16, ip, ip, 4, 16, 0, op, p, 0, nullptr), DSA_ERR_INVALID_ARG);
  expect("topk ld", dsa_topk(fp, 8, ip, ip, 4, 16, 4, op, p, 0, nullptr), DSA_ERR_INVALID_ARG);
  expect("topk huge", dsa_topk(fp, big, ip, ip, big, big, 4, op, p, 0, nullptr), DSA_ERR_INVALID_ARG);
  expect("topk k big", dsa_topk(fp, 16, ip, ip, 4, 16, 1 << 20, op, p, 0, nullptr), DSA_ERR_UNSUPPORTED);
  expect("topk null out", dsa_topk(fp, 16, ip, ip, 4, 16, 4, nullptr, p, 0, nullptr), DSA_ERR_INVALID_ARG);

  // indexer
  expect("idx dtype", dsa_indexer_scores(p, p, nullptr, fp, ip, ip, 4, 16, 4, 128, 9, nullptr, 16, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("idx heads", dsa_indexer_scores(p, p, nullptr, fp, ip, ip, 4, 16, 65, 128, 1, reinterpret_cast<float*>(buf), 16, nullptr),
         DSA_ERR_UNSUPPORTED);
  expect("idx fp8 no scale", dsa_indexer_scores(p, p, nullptr, fp, ip, ip, 4, 16, 4, 128, 2, reinterpret_cast<float*>(buf), 16, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("idx huge", dsa_indexer_scores(p, p, nullptr, fp, ip, ip, big, big, 4, 128, 1, reinterpret_cast<float*>(buf), big, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("idx ld", dsa_indexer_scores(p, p, nullptr, fp, ip, ip, 4, 16, 4, 128, 1, reinterpret_cast<float*>(buf), 8, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("idx_topk ws", dsa_indexer_topk(p, p, nullptr, fp, ip, ip, 4, 100000, 64, 128, 1, 2048, op, nullptr, 0, nullptr),
         DSA_ERR_WORKSPACE);
  expect("idx_topk k0", dsa_indexer_topk(p, p, nullptr, fp, ip, ip, 4, 16, 64, 128, 1, 0, op, p, 0, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("noalloc over", dsa_indexer_topk_noalloc(p, p, nullptr, fp, ip, ip, 256, 100000, 64, 128, 1, 2048, op, nullptr),
         DSA_ERR_WORKSPACE);

  // prep and inserts
  expect("prep rope odd", dsa_indexer_prep(fp, fp, fp, ip, ip, 4, 4, 2, 128, 63, 64, 1e4f, 1e-6f, 1,
                                           p, p, reinterpret_cast<float*>(buf), nullptr, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("k insert dtype", dsa_indexer_k_insert(p, 2, nullptr, nullptr, 1e-6f, reinterpret_cast<const int64_t*>(buf),
                                                4, 128, buf, reinterpret_cast<float*>(buf), 8, nullptr),
         DSA_ERR_UNSUPPORTED);
  expect("k insert eps", dsa_indexer_k_insert(p, 1, nullptr, nullptr, -1.0f, reinterpret_cast<const int64_t*>(buf),
                                              4, 128, buf, reinterpret_cast<float*>(buf), 8, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("mla insert dim", dsa_mla_kv_insert(p, 1, reinterpret_cast<const int64_t*>(buf), 4, 512, buf, 8, nullptr),
         DSA_ERR_UNSUPPORTED);
  expect("mla insert null", dsa_mla_kv_insert(nullptr, 1, reinterpret_cast<const int64_t*>(buf), 4, 576, buf, 8, nullptr),
         DSA_ERR_INVALID_ARG);

  // sparse MLA
  expect("mla dv", dsa_sparse_mla_fwd(p, p, ip, 4, 16, 128, 576, 600, 2048, 0.04f, 1, p, nullptr, nullptr, 0, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("mla heads", dsa_sparse_mla_fwd(p, p, ip, 4, 16, 100, 576, 512, 2048, 0.04f, 1, p, nullptr, nullptr, 0, nullptr),
         DSA_ERR_UNSUPPORTED);
  expect("mla ws", dsa_sparse_mla_fwd(p, p, ip, 4, 16, 128, 576, 512, 2048, 0.04f, 1, p, nullptr, nullptr, 0, nullptr),
         DSA_ERR_WORKSPACE);
  expect("mla fp8 ws", dsa_sparse_mla_fwd(p, p, ip, 4, 16, 128, 576, 512, 2048, 0.04f, 2, p, nullptr, nullptr, 0, nullptr),
         DSA_ERR_WORKSPACE);
  expect("mla huge", dsa_sparse_mla_fwd(p, p, ip, big, big, 128, 576, 512, 2048, 0.04f, 1, p, nullptr, nullptr, 0, nullptr),
         DSA_ERR_INVALID_ARG);
  expect("mla huge heads k", dsa_sparse_mla_fwd(p, p, ip, 4, 16, INT32_MAX, 576, 512, INT32_MAX, 0.04f, 1, p, nullptr, nullptr, 0, nullptr),
         DSA_ERR_UNSUPPORTED);

  std::printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
