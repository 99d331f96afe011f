/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD
 * Instinct MI355X (gfx950): lightning indexer -> per-row top-k -> sparse MLA.
 *
 * Sources.  The method is described on three pages: the vime docs page
 * "Day-0 Model Plugins", vime pull request #502 with its review comments, and
 * the vLLM API page "vllm.models.kimi_k3.nvidia.dsa" (classes KimiK3DSAAttention,
 * KimiK3DSAIndexer, KimiK3DSAIndexerKNorm).  Each entry point below names the
 * passage that defines its operation.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory), row-major and
 *     densely packed unless a leading dimension (ld_*) is given.  The caller owns
 *     every buffer; the library never allocates, frees or retains memory.
 *   - Packed (THD) sequences: the tokens of several sequences are concatenated;
 *     key indices are global positions in the packed key buffer.
 *   - A row's key window is the half-open range [row_starts[t], row_ends[t]).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream: no host synchronisation, no host<->device
 *     copies, no device-dependent host control flow, so the calls can be captured
 *     in a HIP graph.  The library holds no state and is safe to call from
 *     several host threads.
 *   - Every call returns DSA_OK (0) or a negative dsa_status.  Arguments are
 *     validated on the host before anything is enqueued; on error nothing is
 *     enqueued and no output is touched.
 *   - Size limits of every entry point: row and key counts <= INT32_MAX,
 *     1 <= index_topk <= 65536 (sparse MLA also n_heads <= 65536).  A
 *     workspace-size query returns 0 for an empty problem and SIZE_MAX for sizes
 *     beyond these limits (or whose workspace does not fit in size_t), which no
 *     workspace satisfies; the call itself rejects such sizes.
 *   - Device-side values are never trusted for addressing: every kernel clamps
 *     a window to [0, n_k] (a window that ends before it starts is empty), and
 *     the attention skips an index outside [0, n_kv) exactly like -1.  A NaN
 *     score inside a window is a precondition violation that gives an
 *     unspecified selection, still inside the buffers described here.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1, /* null pointer, negative size, ld too small ... */
  DSA_ERR_UNSUPPORTED = -2, /* shape / dtype combination without a kernel    */
  DSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required    */
  DSA_ERR_LAUNCH = -4,      /* the HIP runtime rejected a kernel launch      */
} dsa_status;

typedef enum dsa_dtype {
  DSA_DTYPE_F32 = 0,      /* float32                                    */
  DSA_DTYPE_BF16 = 1,     /* bfloat16                                   */
  DSA_DTYPE_FP8_E4M3 = 2, /* OCP float8 e4m3fn (max 448), one byte each */
  DSA_DTYPE_MXFP4 = 3,    /* OCP MXFP4: e2m1 values, two per byte (even
                             element in the low nibble), one E8M0 scale
                             byte (2^(byte - 127)) per 32 values       */
} dsa_dtype;

/* Human-readable name of a status code (static string). */
const char* dsa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int dsa_version(void);

/*
 * dsa_row_windows -- per-row key windows of packed sequences.
 *
 * Passage: the window rule of the fallback top-k in review comment 3 of vime
 * pull request #502 (column c of a row is valid when row_starts <= c < row_ends),
 * combined with the packed-position rebase of review comment 1 (indices are
 * offsets into the packed key buffer, sample offsets advance by the sample's
 * full token length).
 *
 *   cu_seqlens_q, cu_seqlens_k  int32 [n_seqs + 1], exclusive prefix sums of the
 *                               query and key counts of each sequence.  The
 *                               queries of sequence b are its LAST q_len tokens.
 *   n_rows                      = cu_seqlens_q[n_seqs] (passed by the caller so
 *                               that no device value is read on the host).
 *   causal                      1: the query at local position p of sequence b
 *                               sees keys [cu_k[b], cu_k[b] + k_len - q_len + p + 1)
 *                               (every key up to and including its own token;
 *                               prefill q_len == k_len gives end = t + 1, decode
 *                               q_len == 1 gives the whole cache).  0: the whole
 *                               sequence [cu_k[b], cu_k[b+1]).
 *   row_starts, row_ends        int32 [n_rows] outputs.
 * A causal window that would end before it starts (k_len < q_len) is empty.
 */
int dsa_row_windows(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t n_seqs, int64_t n_rows, int32_t causal,
                    int32_t* row_starts, int32_t* row_ends, void* stream);

/*
 * dsa_indexer_prep -- prepare indexer operands from raw projections.
 *
 * Passages (vLLM API page "vllm.models.kimi_k3.nvidia.dsa"):
 *   KimiK3DSAIndexerKNorm          LayerNorm of the shared index key, weight 1,
 *                                  bias 0, computed in fp32, cast to the output type;
 *   KimiK3DSAIndexer._apply_index_rope
 *                                  RoPE on the leading rope_dim dims of every head
 *                                  (q) and of the key, half-split pairing (dim i
 *                                  with dim i + rope_dim/2), after the key norm,
 *                                  frequencies = the leading rope_dim/2 frequencies
 *                                  theta^(-2i/rope_main_dim) of the main cache;
 *   KimiK3DSAIndexer.__init__ / score
 *                                  power-of-two ("ue8m0") scales per head_dim block,
 *                                  read as fp32; the query scale is folded into the
 *                                  per-head weights.
 *
 *   q_raw   f32 [n_q, n_heads, head_dim]   k_raw f32 [n_k, head_dim]
 *   w       f32 [n_q, n_heads]             pos_q int32 [n_q], pos_k int32 [n_k]
 *           (positions inside each sequence; ignored when rope_dim == 0, may be NULL then)
 *   dtype   output type of q_out / k_out: F32, BF16, FP8_E4M3 or MXFP4.
 *   q_out   [n_q, n_heads, head_dim] of dtype;  k_out [n_k, head_dim] of dtype.
 *   w_out   f32 [n_q, n_heads]: w (F32/BF16/MXFP4) or w * q_scale (FP8_E4M3).
 *   k_scale_out  f32 [n_k]: the key scale for FP8_E4M3; for MXFP4 the E8M0
 *           scale bytes [n_k, head_dim / 32]; else ignored (may be NULL).
 * Scale rule (FP8_E4M3): s = the smallest power of two with amax <= 448 * s
 * (s = 1 for an all-zero block); codes = round-to-nearest-even(x / s).
 * MXFP4 (the "MXFP4 keys with MXFP4 queries" indexer of KimiK3DSAIndexer.__init__,
 * scales not foldable into the per-head weights): the OCP microscaling
 * conversion per 32 values -- X = 2^(floor(log2 amax) - 2), codes =
 * round-to-nearest-even(x / X) on the e2m1 grid, saturating at 6; q_out holds,
 * per token, the n_heads rows of head_dim / 2 code bytes followed by the
 * n_heads scale groups of head_dim / 32 bytes; k_out [n_k, head_dim / 2] code
 * bytes.  MXFP4 requires rope_dim == 0 (on the page the fp4 keys need the
 * fused key insert, which runs without index rope) and head_dim % 64 == 0.
 * n_k may be 0 (queries only, e.g. a decode step over a key cache).
 * Supported: head_dim <= 256 and even; rope_dim even and <= head_dim.
 */
int dsa_indexer_prep(const float* q_raw, const float* k_raw, const float* w,
                     const int32_t* pos_q, const int32_t* pos_k,
                     int64_t n_q, int64_t n_k, int32_t n_heads, int32_t head_dim,
                     int32_t rope_dim, int32_t rope_main_dim, float rope_theta,
                     float eps, int32_t dtype,
                     void* q_out, void* k_out, float* w_out, float* k_scale_out,
                     void* stream);

/*
 * dsa_indexer_k_insert -- write new index keys into the fp8 index-key cache.
 *
 * Passage: KimiK3DSAIndexer._fused_k_insert and KimiK3DSAIndexer.__init__ on the
 * vLLM API page "vllm.models.kimi_k3.nvidia.dsa": the new tokens' index keys go
 * through the key LayerNorm (the norm's weight, bias and eps; this fused path
 * is the one used without index rope), are quantised to fp8 with one
 * power-of-two ("ue8m0", rounded at write) scale per index_head_dim block, and
 * are written to the cache at the tokens' slots.
 *
 *   k_raw          [n_tokens, head_dim] of k_dtype (F32 or BF16): the key
 *                  projection before the norm
 *   norm_weight    f32 [head_dim] or NULL (1);  norm_bias f32 [head_dim] or NULL (0)
 *   slot_mapping   int64 [n_tokens]: the cache row of each token; a negative
 *                  slot (padding) or one >= n_slots writes nothing
 *   k_cache        OCP e4m3fn [n_slots, head_dim] (uint8): row `slot` gets the
 *                  codes; k_scale_cache f32 [n_slots]: row `slot` gets the scale.
 *                  Together they are the k / k_scale operands of
 *                  dsa_indexer_scores and dsa_indexer_topk with FP8_E4M3 (132
 *                  bytes read per key), so a decode step scores the cache in place.
 * Other slots are left untouched.  Two tokens must not share a slot.  Scale
 * rule as dsa_indexer_prep: the smallest power of two s with amax <= 448 * s
 * (1 for an all-zero row), codes = round-to-nearest-even(y / s); the norm is
 * computed in fp32.  Supported: even head_dim <= 128, or a multiple of 4 up to
 * 256.
 */
int dsa_indexer_k_insert(const void* k_raw, int32_t k_dtype, const float* norm_weight,
                         const float* norm_bias, float eps, const int64_t* slot_mapping,
                         int64_t n_tokens, int32_t head_dim, uint8_t* k_cache,
                         float* k_scale_cache, int64_t n_slots, void* stream);

/*
 * dsa_mla_kv_insert -- write new latent rows into the fp8 MLA cache.
 *
 * Passage: KimiK3DSAAttention.__init__ on the vLLM API page
 * "vllm.models.kimi_k3.nvidia.dsa" (kv_cache_dtype "fp8_ds_mla": the latent
 * cache holds fp8 latent values with per-tile scales and the rope part
 * unquantised).
 *
 *   kv            [n_tokens, d_qk] of kv_dtype (F32 or BF16): the new rows, 512
 *                 latent dims then 64 rope dims (16-byte aligned)
 *   slot_mapping  int64 [n_tokens]: the cache row of each token; a negative slot
 *                 or one >= n_slots writes nothing
 *   kv_cache      uint8 [n_slots, 656] (16-byte aligned), the FP8_E4M3 kv
 *                 operand of dsa_sparse_mla_fwd: row `slot` gets, per 128
 *                 latent dims, the smallest power of two s with amax <= 448 s (1
 *                 for an all-zero tile) at bytes 512 + 4 b (fp32) and the codes
 *                 round-to-nearest-even(x / s) at bytes 128 b ..; then the rope
 *                 dims rounded to bf16 at bytes 528 .. 655.
 * Other slots are left untouched; two tokens must not share a slot.
 * Supported: d_qk == 576.
 */
int dsa_mla_kv_insert(const void* kv, int32_t kv_dtype, const int64_t* slot_mapping,
                      int64_t n_tokens, int32_t d_qk, uint8_t* kv_cache, int64_t n_slots,
                      void* stream);

/*
 * dsa_indexer_scores -- lightning-indexer scores over each row's window.
 *
 * Passage: the operands KimiK3DSAIndexer.forward and .score build on the vLLM API
 * page "vllm.models.kimi_k3.nvidia.dsa" (per-head queries, one shared key per
 * token, per-head weights with the query scale folded in, fp32 key scales), scored
 * with the DSA lightning-indexer formula
 *     score[t, s] = k_scale[s] * sum_h w[t, h] * max(0, q[t, h, :] . k[s, :])
 * for row_starts[t] <= s < row_ends[t].
 *
 *   q        [n_q, n_heads, head_dim] of dtype (MXFP4: the layout of
 *            dsa_indexer_prep's q_out, n_heads * (head_dim / 2 + head_dim / 32)
 *            bytes per token)
 *   k        [n_k, head_dim] of dtype (MXFP4: head_dim / 2 code bytes per key)
 *   k_scale  f32 [n_k] (FP8_E4M3), or the E8M0 bytes [n_k, head_dim / 32]
 *            (MXFP4, 4-byte aligned); must be NULL otherwise
 *   w        f32 [n_q, n_heads]
 * MXFP4: score = sum_h w * max(0, sum over the 32-value blocks b of
 * 2^(sq_b - 127) 2^(sk_b - 127) sum_{d in b} q4 k4) -- the matrix core applies
 * both block scales (v_mfma_scale_f32_32x32x64_f8f6f4 with e2m1 operands).
 *   scores   f32 [n_q, ld_scores], ld_scores >= n_k.  ONLY in-window entries are
 *            written; everything else is left untouched (it may hold garbage).
 * Accumulation is fp32.  Supported: BF16, FP8_E4M3 and MXFP4 with head_dim ==
 * 128 and 1 <= n_heads <= 64 (MXFP4: n_heads % 4 == 0) (matrix-core path); F32
 * with head_dim <= 256, n_heads <= 64 and n_heads * head_dim <= 8192.
 */
int dsa_indexer_scores(const void* q, const void* k, const float* k_scale,
                       const float* w, const int32_t* row_starts,
                       const int32_t* row_ends, int64_t n_q, int64_t n_k,
                       int32_t n_heads, int32_t head_dim, int32_t dtype,
                       float* scores, int64_t ld_scores, void* stream);

/*
 * dsa_topk -- per-row top-k of a score matrix, with windows and -1 padding.
 *
 * Passage: the fallback top-k of review comment 3 of vime pull request #502
 * (torch_dsa_topk with the suggested window mask): columns outside
 * [row_starts, row_ends) are never selected; k_eff = min(index_topk, number of
 * selectable columns); the remaining slots are -1.  Readings fixed here: ties go
 * to the lowest column; -inf is never selected (+inf is); -0.0 equals +0.0; the
 * selected columns are written in ASCENDING column order, then the -1 padding.
 *
 *   scores    f32 [n_q, ld_scores]; only in-window entries are read.
 *   topk_idx  int32 [n_q, index_topk], every entry written (global columns).
 *   workspace at least dsa_topk_workspace_size(...) bytes, 256-byte aligned, or
 *             NULL when that size is 0.  It is nonzero for few rows over many
 *             columns (n_q <= 1024, n_cols > 8192, index_topk <= 2048), where
 *             each row's window is selected in up to 16 chunks whose candidates
 *             (key, column) are merged: n_q * 16 * index_topk * 8 + n_q * 64
 *             bytes.  Its contents on entry do not matter.
 * Bit-exact: the result is a function of the fp32 score bits only.
 * Supported: 1 <= index_topk <= 65536.  Windows are clamped to [0, n_cols].
 */
size_t dsa_topk_workspace_size(int64_t n_q, int64_t n_cols, int32_t index_topk);
int dsa_topk(const float* scores, int64_t ld_scores, const int32_t* row_starts,
             const int32_t* row_ends, int64_t n_q, int64_t n_cols,
             int32_t index_topk, int32_t* topk_idx, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_topk -- indexer scores followed by the top-k, one call.
 *
 * Passage: KimiK3DSAIndexer.score on the vLLM API page
 * "vllm.models.kimi_k3.nvidia.dsa", which scores the current rows and writes
 * their top-k into a caller-owned int32 index buffer in one op.  Same operands
 * and semantics as dsa_indexer_scores followed by dsa_topk; the score matrix is
 * not an output.  workspace: at least dsa_indexer_topk_workspace_size(...) bytes,
 * 256-byte aligned (NULL when that size is 0); its contents on entry do not
 * matter.
 * The scores never reach memory for bf16, fp8 and MXFP4 with index_topk <= 2048:
 *   More than 256 rows (prefill): fused, no workspace -- four rows per
 *   workgroup share each chunk of keys, and each row keeps its candidates
 *   (scores above a running floor, shrunk in place to their exact top k when
 *   full) in LDS.
 *   At most 256 rows (decode): fused -- scores are computed into LDS per (row,
 *   key chunk) and reduced there to candidates; the workspace holds the
 *   candidates (n_q * 16 * index_topk * 8 + n_q * 64 bytes, 0 when
 *   n_k <= 8192).
 * Otherwise (F32, or index_topk > 2048) the scores go through the workspace
 * (n_q * n_k * 4 bytes, plus dsa_topk's workspace).
 * In the bf16, fp8 and MXFP4 paths (index_topk <= 2048), a row whose window
 * holds at most index_topk keys and whose head weights are all >= 0 is written
 * as its whole window (columns a .. b-1, then -1) without being scored: none of
 * its scores can be -inf, so the selection is every key.  Key scales must be
 * positive, as dsa_indexer_prep and dsa_indexer_k_insert write them.
 */
size_t dsa_indexer_topk_workspace_size(int64_t n_q, int64_t n_k, int32_t n_heads,
                                       int32_t head_dim, int32_t dtype,
                                       int32_t index_topk);
int dsa_indexer_topk(const void* q, const void* k, const float* k_scale,
                     const float* w, const int32_t* row_starts,
                     const int32_t* row_ends, int64_t n_q, int64_t n_k,
                     int32_t n_heads, int32_t head_dim, int32_t dtype,
                     int32_t index_topk, int32_t* topk_idx, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_topk_noalloc -- dsa_indexer_topk without a workspace argument.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same operands,
 * semantics and kernels as dsa_indexer_topk; the workspace that call would
 * need comes from a device array inside the library, DSA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) on each GPU, held from library load until the process ends.  The
 * call allocates nothing.
 *   - The stream must belong to the current device (the array of that device
 *     is used; its address is looked up on the first call on each device).
 *   - Returns DSA_ERR_WORKSPACE, enqueueing nothing, when the workspace
 *     dsa_indexer_topk_workspace_size(...) reports exceeds the array (e.g. more
 *     than 255 rows of windows longer than 8192 keys at index_topk = 2048).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind (no call relies on them): calls that overlap in time on one GPU
 *     (two streams, two threads) race and give undefined results.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dsa_indexer_topk_noalloc(const void* q, const void* k, const float* k_scale,
                             const float* w, const int32_t* row_starts,
                             const int32_t* row_ends, int64_t n_q, int64_t n_k,
                             int32_t n_heads, int32_t head_dim, int32_t dtype,
                             int32_t index_topk, int32_t* topk_idx, void* stream);

/*
 * dsa_sparse_mla_fwd -- MLA attention over the selected latent rows only.
 *
 * Passage: the vLLM API page "vllm.models.kimi_k3.nvidia.dsa" (module text and
 * KimiK3DSAAttention): the MLA layers run with is_sparse=True so that the sparse
 * attention backend consumes the indexer's top-k indices; in the absorbed MLA
 * form every head reads the same latent row per key (kv_lora_rank latent dims
 * followed by the rope dims), and the value is the latent part.
 *
 * For query t, head h, with J = the entries of topk_idx[t] that are not -1:
 *   l_j = sm_scale * q[t, h, :d_qk] . kv[J_j, :d_qk]
 *   out[t, h, :] = sum_j softmax(l)_j * kv[J_j, :d_v],  lse[t, h] = logsumexp_j l_j
 * An all -1 row gives out = 0 and lse = -inf.  Duplicates count as listed.
 *
 *   q         [n_q, n_heads, d_qk] of dtype (F32 or BF16; BF16 for FP8_E4M3)
 *   kv        [n_kv, d_qk] of dtype; V = the first d_v columns of the same rows.
 *             FP8_E4M3 is the fp8 latent cache ("fp8_ds_mla", the kv_cache_dtype
 *             of KimiK3DSAAttention on the same page), 656 bytes per row: 512 OCP
 *             e4m3fn latent codes, 4 fp32 scales (latent dims 128 b .. 128 b + 127
 *             are code * scale[b]), then the 64 rope dims in bf16 -- the rows
 *             dsa_mla_kv_insert writes.  Its rows enter the kernel as those bf16
 *             values (exact for the power-of-two scales the insert writes).
 *   topk_idx  int32 [n_q, index_topk]; entries in [0, n_kv) or -1 (an entry
 *             outside [0, n_kv) is skipped like -1)
 *   out       [n_q, n_heads, d_v] of dtype (BF16 for FP8_E4M3);  lse f32
 *             [n_q, n_heads] or NULL
 *   workspace at least dsa_sparse_mla_workspace_size(...) bytes (may be 0).
 *   For few queries (BF16, FP8_E4M3) each row's keys are split over several
 *   workgroups;
 *   the workspace then holds their normalised partial outputs in bf16 and
 *   their partial LSEs in fp32, merged by a second kernel.
 * Softmax statistics and accumulation are fp32; probabilities enter the
 * value product in the input type (bf16 for FP8_E4M3).  Supported: BF16 with
 * d_qk == 576, d_v == 512, n_heads a multiple of 32; FP8_E4M3 with d_qk == 576,
 * d_v == 512 (q and kv 16-byte aligned, out 8-byte aligned); F32 with
 * d_qk <= 256, d_v <= d_qk.
 */
size_t dsa_sparse_mla_workspace_size(int64_t n_q, int32_t n_heads, int32_t d_qk,
                                     int32_t d_v, int32_t index_topk,
                                     int32_t dtype);
int dsa_sparse_mla_fwd(const void* q, const void* kv, const int32_t* topk_idx,
                       int64_t n_q, int64_t n_kv, int32_t n_heads, int32_t d_qk,
                       int32_t d_v, int32_t index_topk, float sm_scale,
                       int32_t dtype, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
