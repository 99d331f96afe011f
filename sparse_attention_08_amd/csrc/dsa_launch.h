// Internal launchers (host side) of the DSA kernels.  Argument validation is
// done by the C-ABI layer (dsa_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

hipError_t launch_row_windows(const int32_t* cu_q, const int32_t* cu_k, int32_t n_seqs,
                              int64_t n_rows, int32_t causal, int32_t* row_starts,
                              int32_t* row_ends, hipStream_t stream);

hipError_t launch_indexer_prep(const float* q_raw, const float* k_raw, const float* w,
                               const int32_t* pos_q, const int32_t* pos_k, int64_t n_q,
                               int64_t n_k, int32_t n_heads, int32_t head_dim,
                               int32_t rope_dim, int32_t rope_main_dim, float theta,
                               float eps, int32_t dtype, void* q_out, void* k_out,
                               float* w_out, float* k_scale_out, hipStream_t stream);

hipError_t launch_mla_kv_insert(const void* kv, int32_t kv_dtype, const int64_t* slot_mapping,
                                int64_t n_tokens, uint8_t* kv_cache, int64_t n_slots,
                                hipStream_t stream);
hipError_t launch_indexer_k_insert(const void* k_raw, int32_t k_dtype, const float* weight,
                                   const float* bias, float eps, const int64_t* slot_mapping,
                                   int64_t n_tokens, int32_t head_dim, uint8_t* k_cache,
                                   float* k_scale_cache, int64_t n_slots, hipStream_t stream);

size_t topk_workspace_bytes(int64_t n_q, int64_t n_cols, int32_t K);

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_starts,
                       const int32_t* row_ends, int64_t n_q, int64_t n_cols, int32_t K,
                       int32_t* out, void* workspace, hipStream_t stream);

// Final phase of the split top-k: merge the per-chunk candidates in the
// workspace (laid out as topksel::Candidates) into topk_idx.
hipError_t launch_topk_merge(const int32_t* row_starts, const int32_t* row_ends, int64_t n_q,
                             int64_t n_cols, int32_t K, int32_t* out, void* workspace,
                             hipStream_t stream);

hipError_t launch_indexer_scores(const void* q, const void* k, const float* k_scale,
                                 const float* w, const int32_t* row_starts,
                                 const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                 int32_t n_heads, int32_t head_dim, int32_t dtype,
                                 float* scores, int64_t ld, hipStream_t stream);

// Fused indexer + top-k (few rows over long windows): whether it applies, its
// workspace (the split top-k's candidates), and the launch.
bool indexer_topk_fused(int64_t n_q, int32_t dtype, int32_t K);
size_t indexer_topk_fused_workspace_bytes(int64_t n_q, int32_t K);
hipError_t launch_indexer_topk_fused(const void* q, const void* k, const float* k_scale,
                                     const float* w, const int32_t* row_starts,
                                     const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                     int32_t n_heads,
                                     int32_t dtype, int32_t K, int32_t* out, void* workspace,
                                     hipStream_t stream);

// Fused indexer + top-k for many rows (prefill): the rows' candidates stay in
// LDS, no workspace.
bool indexer_topk_rows_applies(int32_t dtype, int32_t K);
hipError_t launch_indexer_topk_rows(const void* q, const void* k, const float* k_scale,
                                    const float* w, const int32_t* row_starts,
                                    const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                    int32_t n_heads, int32_t dtype, int32_t K, int32_t* out,
                                    hipStream_t stream);

size_t mla_workspace_bytes(int64_t n_q, int32_t n_heads, int32_t d_qk, int32_t d_v,
                           int32_t index_topk, int32_t dtype);

hipError_t launch_sparse_mla(const void* q, const void* kv, const int32_t* idx,
                             int64_t n_q, int64_t n_kv, int32_t n_heads, int32_t d_qk,
                             int32_t d_v, int32_t K, float sm_scale, int32_t dtype,
                             void* out, float* lse, void* workspace, hipStream_t stream);

}  // namespace dsa
