// Fused lightning indexer + top-k for few query rows over long key windows
// (decode), gfx950.  The scores never leave the chip.
//
// KimiK3DSAIndexer.score on the vLLM API page "vllm.models.kimi_k3.nvidia.dsa"
// scores the current rows and writes their top-k into a caller-owned index
// buffer in one op; the selection rule is the fallback top-k of review comment
// 3 of vime pull request #502 (window mask, -1 padding), ties to the lowest
// column, output in ascending column order.
//
// Workgroup (row t, chunk c) of 4 waves:
//   * windows of 8193 .. 131072 keys are cut into 16 chunks of at most 8192
//     keys (as on the split path of dsa_topk); the workgroup computes the
//     scores of its chunk (each wave streams 32-key tiles: bf16 keys over
//     33..64 heads through two private LDS buffers by LDS-DMA, other keys
//     straight into registers, the next tile in flight while the current one is on the
//     matrix core) straight into LDS as order-preserving keys, selects the
//     chunk's top-k and writes it as candidates (key, column); the merge kernel
//     of the split top-k then selects the row's top-k from the candidates;
//   * other windows are done whole by chunk 0, which streams the window
//     through LDS in pieces of 8192 keys, keeping the running top-k (at most k
//     candidates, in column order) in LDS, and writes the row's result.
// Exactness of both is the same argument: a key of the row's top-k is in the
// top-k of any subset of the row that contains it.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "indexer_core.h"
#include "topk_select.h"

namespace dsa {
namespace {

using namespace topksel;
using ixcore::kKeyTile;
using ixcore::OpBf16;
using ixcore::OpFp4;
using ixcore::OpFp8;
using ixcore::QueryRow;

// Per-wave LDS buffers of the key stream (LDS-DMA, one tile in flight): bf16
// keys over 33..64 heads only.  There the kernel's registers allow one wave per
// SIMD anyway, and the DMA stream beats direct fragment loads on 256-byte keys
// (decode: 0.357 -> 0.325 ms); it loses on the fp8 ones (0.203 -> 0.244 ms),
// and with up to 32 heads the 64 KB of buffers would halve the workgroups per
// CU, so those stream into registers.
template <class Op, int MT>
struct FusedBufs {
  static constexpr int kNB = Op::kRowBytes == 256 && MT == 2 ? 2 : 0;
  static constexpr int kBytes = kNB > 0 ? kNB * ixcore::LdsTile<Op, Op::kKeyScale>::kBytes : 16;
};

struct FusedShared {
  uint32_t keys[kMaxSplitK + kCap];  // running candidates [0, ncand), then new keys
  int32_t cols[kMaxSplitK];          // columns of the running candidates
  uint32_t tkey[kMaxSplitK];         // next running candidate set
  int32_t tcol[kMaxSplitK];
  SelectShared<kThreads> sel;
};

// Scores of keys [s_lo, s_lo + m) of row qr into out[0, m) as order-preserving
// keys; returns this thread's count of selectable keys.  Each wave streams its
// 32-key tiles (every 4th) with the next tile's loads in flight (into tbuf, the
// wave's LDS buffers, when FusedBufs gives it any).
template <class Op, int MT, bool kScaled>
__device__ __forceinline__ uint32_t score_range(const QueryRow<Op, MT>& qr,
                                                const uint8_t* __restrict__ k,
                                                const float* __restrict__ k_scale, int s_lo,
                                                int m, uint32_t* out, int lane, int wave,
                                                uint32_t& kmin, uint32_t& kmax, uint8_t* tbuf) {
  constexpr int NW = kThreads / kWave;
  const int nt = (m + kKeyTile - 1) / kKeyTile;
  const int hi = s_lo + m;
  uint32_t cnt = 0u;
  auto put = [&](int i, float p) {
    const int j = i * kKeyTile + (lane & 31);
    if (lane < 32 && j < m) {
      const uint32_t key = score_key(p);
      out[j] = key;
      if (key != 0u) {
        ++cnt;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  };
  constexpr int kNB = FusedBufs<Op, MT>::kNB;
  if constexpr (kNB > 0)
    ixcore::stream_tiles_lds<Op, MT, kScaled, kNB>(qr, k, k_scale, s_lo, hi, wave, NW, nt, lane,
                                                   tbuf, put);
  else
    ixcore::stream_tiles<Op, MT, kScaled>(qr, k, k_scale, s_lo, hi, wave, NW, nt, lane, put);
  return cnt;
}

template <class Op, int MT>
__global__ __launch_bounds__(kThreads) void indexer_topk_chunk_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int H,
    int n_k, int32_t K, int32_t* __restrict__ out, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_col, int32_t* __restrict__ cand_cnt) {
  constexpr bool kScaled = Op::kKeyScale;  // fp8 / fp4 keys carry a scale
  __shared__ FusedShared sh;
  constexpr int kTBytes = FusedBufs<Op, MT>::kBytes;
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[kThreads / kWave][kTBytes];
  const int64_t t = blockIdx.x;
  const int c = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int a = max(row_starts[t], 0);  // windows are clamped to the keys [0, n_k)
  const int b = min(row_ends[t], n_k);
  const int n = b > a ? b - a : 0;
  const int clen = split_chunk_len(n);
  if (clen == 0 && c != 0) return;
  if (n <= K && ixcore::row_weights_nonneg(w, t, H, lane)) {
    // the whole window is the top-k (row_weights_nonneg): written without scoring
    int32_t* dst = out + t * int64_t(K);
    for (int j = threadIdx.x; j < K; j += kThreads) dst[j] = j < n ? a + j : -1;
    return;
  }

  QueryRow<Op, MT> qr;
  qr.load(q, w, t, H, lane);

  if (clen > 0) {
    // one chunk of a split window -> candidates
    const int64_t slot = t * kMaxChunks + c;
    const int lo = c * clen;
    const int m = lo < n ? min(clen, n - lo) : 0;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    const uint32_t cnt = score_range<Op, MT, kScaled>(qr, k, k_scale, a + lo, m, sh.keys, lane,
                                                      wave, kmin, kmax, tbuf[wave]);
    KeyRange kr;
    const uint32_t n_sel =
        block_count_range<kThreads>(cnt, kmin, kmax, sh.sel, kr);  // also orders the LDS writes
    uint32_t* ck = cand_key + slot * K;
    int32_t* cc = cand_col + slot * K;
    select_topk<kThreads>(
        LdsKeys{sh.keys}, m, n_sel, K, sh.sel,
        [&](uint32_t p, int i, uint32_t key) {
          ck[p] = key;
          cc[p] = a + lo + i;
        },
        kr);
    if (threadIdx.x == 0) cand_cnt[slot] = int32_t(n_sel < uint32_t(K) ? n_sel : uint32_t(K));
    return;
  }

  // the whole window, streamed through LDS with a running top-k
  int32_t* dst = out + t * int64_t(K);
  uint32_t ncand = 0u;
  for (int lo = 0;; lo += kCap) {
    const int m = lo < n ? min(kCap, n - lo) : 0;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;  // not used: the running candidates join the keys
    const uint32_t cnt = score_range<Op, MT, kScaled>(qr, k, k_scale, a + lo, m, sh.keys + ncand,
                                                      lane, wave, kmin, kmax, tbuf[wave]);
    const uint32_t n_sel = ncand + block_sum<kThreads>(cnt, sh.sel.tmp);
    const int total = int(ncand) + m;
    const int nc = int(ncand);
    if (lo + m >= n) {
      select_topk<kThreads>(LdsKeys{sh.keys}, total, n_sel, K, sh.sel,
                            [&](uint32_t p, int i, uint32_t) {
                              dst[p] = i < nc ? sh.cols[i] : a + lo + (i - nc);
                            });
      const uint32_t k_eff = n_sel < uint32_t(K) ? n_sel : uint32_t(K);
      for (uint32_t p = k_eff + threadIdx.x; p < uint32_t(K); p += kThreads) dst[p] = -1;
      return;
    }
    select_topk<kThreads>(LdsKeys{sh.keys}, total, n_sel, K, sh.sel,
                          [&](uint32_t p, int i, uint32_t key) {
                            sh.tkey[p] = key;
                            sh.tcol[p] = i < nc ? sh.cols[i] : a + lo + (i - nc);
                          });
    __syncthreads();
    ncand = n_sel < uint32_t(K) ? n_sel : uint32_t(K);
    for (uint32_t p = threadIdx.x; p < ncand; p += kThreads) {
      sh.keys[p] = sh.tkey[p];
      sh.cols[p] = sh.tcol[p];
    }
    __syncthreads();
  }
}

template <class Op, int MT>
hipError_t launch_fused(const void* q, const void* k, const float* k_scale, const float* w,
                        const int32_t* rs, const int32_t* re, int64_t n_q, int64_t n_k, int H,
                        int32_t K, int32_t* out, void* workspace, hipStream_t stream) {
  const Candidates cd = Candidates::at(workspace, n_q, K);
  hipLaunchKernelGGL((indexer_topk_chunk_kernel<Op, MT>), dim3(unsigned(n_q), kMaxChunks),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(q),
                     static_cast<const uint8_t*>(k), k_scale, w, rs, re, H, int(n_k), K, out,
                     cd.key, cd.col, cd.cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(rs, re, n_q, n_k, K, out, workspace, stream);
}

}  // namespace

bool indexer_topk_fused(int64_t n_q, int32_t dtype, int32_t K) {
  return dtype != 0 && n_q <= kMaxSplitRows && K <= kMaxSplitK;
}

size_t indexer_topk_fused_workspace_bytes(int64_t n_q, int32_t K) {
  return Candidates::bytes(n_q, K);
}

hipError_t launch_indexer_topk_fused(const void* q, const void* k, const float* k_scale,
                                     const float* w, const int32_t* row_starts,
                                     const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                     int32_t n_heads, int32_t dtype, int32_t K, int32_t* out,
                                     void* workspace, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const bool one = n_heads <= 32;
  if (dtype == 1)
    return one ? launch_fused<OpBf16, 1>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k, n_heads,
                                         K, out, workspace, stream)
               : launch_fused<OpBf16, 2>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k, n_heads,
                                         K, out, workspace, stream);
  if (dtype == 3)
    return one ? launch_fused<OpFp4, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads,
                                        K, out, workspace, stream)
               : launch_fused<OpFp4, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads,
                                        K, out, workspace, stream);
  return one ? launch_fused<OpFp8, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, K,
                                      out, workspace, stream)
             : launch_fused<OpFp8, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, K,
                                      out, workspace, stream);
}

}  // namespace dsa
