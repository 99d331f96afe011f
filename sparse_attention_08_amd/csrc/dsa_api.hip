// C ABI of the DSA hot path: host-side validation and dispatch.  Every check
// runs before anything is enqueued, so a rejected call touches no buffer.
#include <climits>
#include <cstdint>

#include "dsa.h"
#include "dsa_launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int32_t kMaxK = 65536;          // index_topk limit of every entry point
constexpr int32_t kMaxMlaHeads = 65536;   // sparse MLA heads

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

int check_indexer(const void* q, const void* k, const float* k_scale, const float* w,
                  const int32_t* rs, const int32_t* re, int64_t n_q, int64_t n_k,
                  int32_t n_heads, int32_t head_dim, int32_t dtype) {
  if (n_q < 0 || n_k < 0 || n_k > INT32_MAX || n_q > INT32_MAX) return DSA_ERR_INVALID_ARG;
  if (dtype < DSA_DTYPE_F32 || dtype > DSA_DTYPE_MXFP4) return DSA_ERR_INVALID_ARG;
  if (n_heads < 1 || head_dim < 1) return DSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q || !w || !rs || !re)) return DSA_ERR_INVALID_ARG;
  if (n_q > 0 && n_k > 0 && !k) return DSA_ERR_INVALID_ARG;
  if (dtype == DSA_DTYPE_FP8_E4M3 || dtype == DSA_DTYPE_MXFP4) {
    if (n_q > 0 && n_k > 0 && !k_scale) return DSA_ERR_INVALID_ARG;
  } else if (k_scale) {
    return DSA_ERR_INVALID_ARG;
  }
  if (n_heads > 64) return DSA_ERR_UNSUPPORTED;
  if (dtype == DSA_DTYPE_F32) {
    if (head_dim > 256 || int64_t(n_heads) * head_dim > 8192) return DSA_ERR_UNSUPPORTED;
  } else {
    if (head_dim != 128) return DSA_ERR_UNSUPPORTED;
    // MXFP4 tokens are n_heads * 68 bytes: 16-byte fragments need n_heads % 4 == 0
    if (dtype == DSA_DTYPE_MXFP4 && (n_heads % 4) != 0) return DSA_ERR_UNSUPPORTED;
    const uintptr_t al = dtype == DSA_DTYPE_FP8_E4M3 ? 32 : 16;
    if (!aligned(q, al) || !aligned(k, al)) return DSA_ERR_UNSUPPORTED;
    if (dtype == DSA_DTYPE_MXFP4 && !aligned(k_scale, 4)) return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

int check_topk(const float* scores, int64_t ld, const int32_t* rs, const int32_t* re,
               int64_t n_q, int64_t n_cols, int32_t K, const int32_t* out) {
  if (n_q < 0 || n_cols < 0 || n_cols > INT32_MAX || n_q > INT32_MAX) return DSA_ERR_INVALID_ARG;
  if (K < 1) return DSA_ERR_INVALID_ARG;
  if (ld < n_cols) return DSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!scores || !rs || !re || !out)) return DSA_ERR_INVALID_ARG;
  if (K > kMaxK) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// Many rows (prefill): four rows per workgroup share each key chunk and keep
// their candidates in LDS; few rows (decode) split each window over workgroups.
bool fused_rows(int64_t n_q, int32_t dtype, int32_t K) {
  return n_q > 256 && dsa::indexer_topk_rows_applies(dtype, K);
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape, dtype or alignment";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int dsa_version(void) { return kVersion; }

int dsa_row_windows(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t n_seqs,
                    int64_t n_rows, int32_t causal, int32_t* row_starts, int32_t* row_ends,
                    void* stream) {
  if (n_seqs < 1 || n_rows < 0 || n_rows > INT32_MAX) return DSA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return DSA_ERR_INVALID_ARG;
  if (n_rows > 0 && (!cu_seqlens_q || !cu_seqlens_k || !row_starts || !row_ends))
    return DSA_ERR_INVALID_ARG;
  return launch_status(dsa::launch_row_windows(cu_seqlens_q, cu_seqlens_k, n_seqs, n_rows,
                                               causal, row_starts, row_ends, as_stream(stream)));
}

int dsa_indexer_prep(const float* q_raw, const float* k_raw, const float* w,
                     const int32_t* pos_q, const int32_t* pos_k, int64_t n_q, int64_t n_k,
                     int32_t n_heads, int32_t head_dim, int32_t rope_dim, int32_t rope_main_dim,
                     float rope_theta, float eps, int32_t dtype, void* q_out, void* k_out,
                     float* w_out, float* k_scale_out, void* stream) {
  if (n_q < 0 || n_k < 0 || n_heads < 1 || head_dim < 1) return DSA_ERR_INVALID_ARG;
  if (dtype < DSA_DTYPE_F32 || dtype > DSA_DTYPE_MXFP4) return DSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_raw || !w || !q_out || !w_out)) return DSA_ERR_INVALID_ARG;
  if (n_k > 0 && (!k_raw || !k_out)) return DSA_ERR_INVALID_ARG;
  if ((dtype == DSA_DTYPE_FP8_E4M3 || dtype == DSA_DTYPE_MXFP4) && n_k > 0 && !k_scale_out)
    return DSA_ERR_INVALID_ARG;
  // MXFP4 keys go through the fused insert path of the pages, which has no index rope
  if (dtype == DSA_DTYPE_MXFP4 && (rope_dim != 0 || head_dim % 64 != 0))
    return DSA_ERR_UNSUPPORTED;
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > head_dim) return DSA_ERR_INVALID_ARG;
  if (rope_dim > 0) {
    if (rope_main_dim < rope_dim || !(rope_theta > 0.0f)) return DSA_ERR_INVALID_ARG;
    if ((n_q > 0 && !pos_q) || (n_k > 0 && !pos_k)) return DSA_ERR_INVALID_ARG;
  }
  if (!(eps >= 0.0f)) return DSA_ERR_INVALID_ARG;
  if (head_dim > 256 || (head_dim & 1)) return DSA_ERR_UNSUPPORTED;
  return launch_status(dsa::launch_indexer_prep(q_raw, k_raw, w, pos_q, pos_k, n_q, n_k, n_heads,
                                                head_dim, rope_dim, rope_main_dim, rope_theta,
                                                eps, dtype, q_out, k_out, w_out, k_scale_out,
                                                as_stream(stream)));
}

int dsa_indexer_k_insert(const void* k_raw, int32_t k_dtype, const float* norm_weight,
                         const float* norm_bias, float eps, const int64_t* slot_mapping,
                         int64_t n_tokens, int32_t head_dim, uint8_t* k_cache,
                         float* k_scale_cache, int64_t n_slots, void* stream) {
  if (n_tokens < 0 || n_slots < 0 || head_dim < 1) return DSA_ERR_INVALID_ARG;
  if (k_dtype != DSA_DTYPE_F32 && k_dtype != DSA_DTYPE_BF16) {
    if (k_dtype == DSA_DTYPE_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    return DSA_ERR_INVALID_ARG;
  }
  if (!(eps >= 0.0f)) return DSA_ERR_INVALID_ARG;
  if (n_tokens > 0 && (!k_raw || !slot_mapping)) return DSA_ERR_INVALID_ARG;
  if (n_slots > 0 && (!k_cache || !k_scale_cache)) return DSA_ERR_INVALID_ARG;
  if (head_dim > 256 || (head_dim > 128 ? head_dim % 4 : head_dim % 2) != 0)
    return DSA_ERR_UNSUPPORTED;
  return launch_status(dsa::launch_indexer_k_insert(k_raw, k_dtype, norm_weight, norm_bias, eps,
                                                    slot_mapping, n_tokens, head_dim, k_cache,
                                                    k_scale_cache, n_slots, as_stream(stream)));
}

int dsa_mla_kv_insert(const void* kv, int32_t kv_dtype, const int64_t* slot_mapping,
                      int64_t n_tokens, int32_t d_qk, uint8_t* kv_cache, int64_t n_slots,
                      void* stream) {
  if (n_tokens < 0 || n_slots < 0 || d_qk < 1) return DSA_ERR_INVALID_ARG;
  if (kv_dtype != DSA_DTYPE_F32 && kv_dtype != DSA_DTYPE_BF16) {
    if (kv_dtype == DSA_DTYPE_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    return DSA_ERR_INVALID_ARG;
  }
  if (n_tokens > 0 && (!kv || !slot_mapping)) return DSA_ERR_INVALID_ARG;
  if (n_slots > 0 && !kv_cache) return DSA_ERR_INVALID_ARG;
  if (d_qk != 576) return DSA_ERR_UNSUPPORTED;
  if (!aligned(kv, 16) || !aligned(kv_cache, 16)) return DSA_ERR_UNSUPPORTED;
  return launch_status(dsa::launch_mla_kv_insert(kv, kv_dtype, slot_mapping, n_tokens, kv_cache,
                                                 n_slots, as_stream(stream)));
}

int dsa_indexer_scores(const void* q, const void* k, const float* k_scale, const float* w,
                       const int32_t* row_starts, const int32_t* row_ends, int64_t n_q,
                       int64_t n_k, int32_t n_heads, int32_t head_dim, int32_t dtype,
                       float* scores, int64_t ld_scores, void* stream) {
  int st = check_indexer(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, head_dim,
                         dtype);
  if (st != DSA_OK) return st;
  if (ld_scores < n_k || (n_q > 0 && !scores)) return DSA_ERR_INVALID_ARG;
  return launch_status(dsa::launch_indexer_scores(q, k, k_scale, w, row_starts, row_ends, n_q,
                                                  n_k, n_heads, head_dim, dtype, scores,
                                                  ld_scores, as_stream(stream)));
}

size_t dsa_topk_workspace_size(int64_t n_q, int64_t n_cols, int32_t index_topk) {
  if (n_q <= 0 || n_cols < 0 || index_topk < 1) return 0;
  if (n_q > INT32_MAX || n_cols > INT32_MAX || index_topk > kMaxK) return SIZE_MAX;
  return dsa::topk_workspace_bytes(n_q, n_cols, index_topk);
}

int dsa_topk(const float* scores, int64_t ld_scores, const int32_t* row_starts,
             const int32_t* row_ends, int64_t n_q, int64_t n_cols, int32_t index_topk,
             int32_t* topk_idx, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_topk(scores, ld_scores, row_starts, row_ends, n_q, n_cols, index_topk, topk_idx);
  if (st != DSA_OK) return st;
  const size_t need = dsa_topk_workspace_size(n_q, n_cols, index_topk);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return DSA_ERR_WORKSPACE;
  return launch_status(dsa::launch_topk(scores, ld_scores, row_starts, row_ends, n_q, n_cols,
                                        index_topk, topk_idx, workspace, as_stream(stream)));
}

size_t dsa_indexer_topk_workspace_size(int64_t n_q, int64_t n_k, int32_t n_heads,
                                       int32_t head_dim, int32_t dtype, int32_t index_topk) {
  (void)n_heads;
  (void)head_dim;
  if (n_q <= 0 || n_k <= 0 || index_topk < 1) return 0;
  if (n_q > INT32_MAX || n_k > INT32_MAX || index_topk > kMaxK) return SIZE_MAX;
  if (fused_rows(n_q, dtype, index_topk)) return 0;
  if (dsa::indexer_topk_fused(n_q, dtype, index_topk))
    return n_k > 8192 ? dsa::indexer_topk_fused_workspace_bytes(n_q, index_topk) : 0;
  // the score matrix, then the top-k's own workspace (256-byte aligned); at the
  // largest sizes the sum no longer fits in size_t
  size_t scores = 0, total = 0;
  if (__builtin_mul_overflow(size_t(n_q) * sizeof(float), size_t(n_k), &scores) ||
      __builtin_add_overflow(scores, size_t(255), &scores))
    return SIZE_MAX;
  scores &= ~size_t(255);
  if (__builtin_add_overflow(scores, dsa::topk_workspace_bytes(n_q, n_k, index_topk), &total))
    return SIZE_MAX;
  return total;
}

int dsa_indexer_topk(const void* q, const void* k, const float* k_scale, const float* w,
                     const int32_t* row_starts, const int32_t* row_ends, int64_t n_q,
                     int64_t n_k, int32_t n_heads, int32_t head_dim, int32_t dtype,
                     int32_t index_topk, int32_t* topk_idx, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_indexer(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, head_dim,
                         dtype);
  if (st != DSA_OK) return st;
  if (index_topk < 1 || (n_q > 0 && !topk_idx)) return DSA_ERR_INVALID_ARG;
  if (index_topk > kMaxK) return DSA_ERR_UNSUPPORTED;
  const size_t need =
      dsa_indexer_topk_workspace_size(n_q, n_k, n_heads, head_dim, dtype, index_topk);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return DSA_ERR_WORKSPACE;
  if (n_q == 0) return DSA_OK;
  hipStream_t s = as_stream(stream);
  if (fused_rows(n_q, dtype, index_topk))
    return launch_status(dsa::launch_indexer_topk_rows(q, k, k_scale, w, row_starts, row_ends,
                                                       n_q, n_k, n_heads, dtype, index_topk,
                                                       topk_idx, s));
  if (dsa::indexer_topk_fused(n_q, dtype, index_topk))
    return launch_status(dsa::launch_indexer_topk_fused(q, k, k_scale, w, row_starts, row_ends,
                                                        n_q, n_k, n_heads, dtype, index_topk,
                                                        topk_idx, workspace, s));
  float* scores = static_cast<float*>(workspace);
  hipError_t e = dsa::launch_indexer_scores(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                            n_heads, head_dim, dtype, scores, n_k, s);
  if (e != hipSuccess) return DSA_ERR_LAUNCH;
  void* topk_ws = static_cast<uint8_t*>(workspace) +
                  ((size_t(n_q) * size_t(n_k) * sizeof(float) + 255) & ~size_t(255));
  return launch_status(dsa::launch_topk(scores, n_k, row_starts, row_ends, n_q, n_k, index_topk,
                                        topk_idx, topk_ws, s));
}

size_t dsa_sparse_mla_workspace_size(int64_t n_q, int32_t n_heads, int32_t d_qk, int32_t d_v,
                                     int32_t index_topk, int32_t dtype) {
  if (n_q <= 0 || n_heads < 1 || index_topk < 1) return 0;
  if (n_q > INT32_MAX || n_heads > kMaxMlaHeads || index_topk > kMaxK) return SIZE_MAX;
  return dsa::mla_workspace_bytes(n_q, n_heads, d_qk, d_v, index_topk, dtype);
}

int dsa_sparse_mla_fwd(const void* q, const void* kv, const int32_t* topk_idx, int64_t n_q,
                       int64_t n_kv, int32_t n_heads, int32_t d_qk, int32_t d_v,
                       int32_t index_topk, float sm_scale, int32_t dtype, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (n_q < 0 || n_kv < 0 || n_q > INT32_MAX || n_kv > INT32_MAX) return DSA_ERR_INVALID_ARG;
  if (n_heads < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk || index_topk < 1)
    return DSA_ERR_INVALID_ARG;
  if (n_heads > kMaxMlaHeads || index_topk > kMaxK) return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_DTYPE_F32 && dtype != DSA_DTYPE_BF16 && dtype != DSA_DTYPE_FP8_E4M3)
    return DSA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q || !topk_idx || !out)) return DSA_ERR_INVALID_ARG;
  if (n_q > 0 && n_kv > 0 && !kv) return DSA_ERR_INVALID_ARG;
  if (dtype == DSA_DTYPE_BF16) {
    if (d_qk != 576 || d_v != 512 || (n_heads % 32) != 0) return DSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 4)) return DSA_ERR_UNSUPPORTED;
  } else if (dtype == DSA_DTYPE_FP8_E4M3) {
    if (d_qk != 576 || d_v != 512) return DSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 8)) return DSA_ERR_UNSUPPORTED;
  } else {
    if (d_qk > 256 || int64_t(index_topk) > 8192) return DSA_ERR_UNSUPPORTED;
  }
  const size_t need =
      dsa_sparse_mla_workspace_size(n_q, n_heads, d_qk, d_v, index_topk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return DSA_ERR_WORKSPACE;
  return launch_status(dsa::launch_sparse_mla(q, kv, topk_idx, n_q, n_kv, n_heads, d_qk, d_v,
                                              index_topk, sm_scale, dtype, out, lse, workspace,
                                              as_stream(stream)));
}

}  // extern "C"
