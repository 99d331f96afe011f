// Per-row top-k over a window of an fp32 score matrix (gfx950).
//
// Semantics follow the fallback top-k of review comment 3 of vime pull request
// #502 (window mask, k = min(topk, n), -inf -> -1, -1 padding), with ties to the
// lowest column and the selected columns written in ascending order.
//
// Selection core (select_topk), run by one workgroup of 256 threads over n keys:
//   1. every score is mapped to an order-preserving u32 key (score_key; -inf ->
//      0 = not selectable) and the selectable keys are counted;
//   2. if more than k are selectable, the k-th largest key is found exactly with
//      MSB-first radix passes of at most 11 bits (2048-bin LDS histogram) that
//      start at the highest bit in which the selectable keys differ: after them
//      `thr` is the k-th key and `need_eq` says how many keys equal to it (the
//      lowest-indexed ones) belong to the selection;
//   3. ordered compaction: each wave owns a contiguous segment, counts its
//      (> thr) and (== thr) keys with ballots, the wave totals are scanned, and
//      a second ballot/mbcnt pass emits every selected key at output position
//      #gt_before + min(#eq_before, need_eq).
//
// Work layouts:
//   rows     one workgroup per row; windows of at most 8192 keys are held in
//            LDS, longer ones are re-read from global memory by each pass;
//   split    for few rows with long windows (decode): a row's window is cut into
//            up to 16 chunks of at most 8192 keys, each workgroup selects its
//            chunk's top-k into a candidate list (key, column) in the workspace,
//            and a merge workgroup per row selects the top-k of the candidates.
//            Exact: a key of the row's top-k (ties to the lowest column) is in
//            its chunk's top-k under the same rule, and the candidates of chunk
//            c precede those of chunk c+1, so the merged output stays ascending.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCap = 8192;        // keys held in LDS by one workgroup
constexpr int kBins = 2048;       // 11-bit digit
constexpr int kMaxChunks = 16;    // chunks per row on the split path
constexpr int kMaxSplitK = 2048;  // largest k on the split path
constexpr int kMergeCap = kMaxChunks * kMaxSplitK;  // candidates merged in LDS
constexpr int64_t kMaxSplitRows = 1024;
constexpr int kMergeThreads = 1024;

template <int NT>
struct SelectShared {
  static constexpr int kNW = NT / kWave;
  uint32_t hist[kBins];
  uint32_t tmp[2 * kNW];
  uint32_t seg_cnt[2 * kNW];
  uint32_t pick[2];
};

// Keys of a row held in LDS, or read (and mapped) from the fp32 scores.
struct LdsKeys {
  const uint32_t* keys;
  __device__ __forceinline__ uint32_t operator()(int i) const { return keys[i]; }
};
struct GlobalKeys {
  const float* src;
  __device__ __forceinline__ uint32_t operator()(int i) const { return score_key(src[i]); }
};

// Workgroup-wide min and max of u32 values.
template <int NT>
__device__ __forceinline__ void block_min_max(uint32_t& lo, uint32_t& hi, uint32_t* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    lo = min(lo, uint32_t(__shfl_xor(int(lo), o)));
    hi = max(hi, uint32_t(__shfl_xor(int(hi), o)));
  }
  if (lane == 0) {
    tmp[wave] = lo;
    tmp[NW + wave] = hi;
  }
  __syncthreads();
  lo = tmp[0];
  hi = tmp[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = min(lo, tmp[w]);
    hi = max(hi, tmp[NW + w]);
  }
  __syncthreads();
}

// Select the K largest of the n keys key(0..n-1) (n_sel of them are nonzero),
// ties to the lowest index, and call emit(p, i, key) for each selected index i
// in ascending order, p = its output slot in [0, min(K, n_sel)).  All NT threads
// of the workgroup call it.
//
// The radix passes start at the highest bit in which the row's selectable keys
// differ (the bits above are common to all of them), in digits of at most 11
// bits: close scores then spread over the histogram instead of piling into a
// few bins, and narrow ranges need fewer passes.
template <int NT, class Keys, class Emit>
__device__ __forceinline__ void select_topk(const Keys& key, int n, uint32_t n_sel, int K,
                                            SelectShared<NT>& sh, Emit emit) {
  constexpr int NW = NT / kWave;
  constexpr int kBPT = kBins / NT;  // histogram bins owned per thread in the scan
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  uint32_t thr = 0u, need_eq = 0u;
  if (n_sel > uint32_t(K)) {
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i = tid; i < n; i += NT) {
      const uint32_t k = key(i);
      if (k != 0u) {
        kmin = min(kmin, k);
        kmax = max(kmax, k);
      }
    }
    block_min_max<NT>(kmin, kmax, sh.tmp);
    const uint32_t diff = kmin ^ kmax;
    int shift = diff == 0u ? 0 : 32 - __builtin_clz(diff);  // varying bits [0, shift)
    uint32_t pmask = shift >= 32 ? 0u : ~((1u << shift) - 1u);
    uint32_t prefix = kmax & pmask;
    uint32_t remaining = uint32_t(K);
#pragma unroll 1
    while (shift > 0) {
      const int nb = shift < 11 ? shift : 11;
      shift -= nb;
      const uint32_t dmask = (1u << nb) - 1u;
      for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t k = key(i);
        if (k != 0u && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      // thread j owns the bins of slot (NT-1-j), so an exclusive prefix over
      // threads is the count of keys in higher bins
      const int base = (NT - 1 - tid) * kBPT;
      uint32_t local = 0u;
#pragma unroll
      for (int j = 0; j < kBPT; ++j) local += sh.hist[base + j];
      uint32_t total;
      const uint32_t above = block_exclusive_sum<NT>(local, sh.tmp, total);
      if (above < remaining && above + local >= remaining) {
        uint32_t c = above;
        for (int j = kBPT - 1; j >= 0; --j) {
          const uint32_t h = sh.hist[base + j];
          if (c + h >= remaining) {
            sh.pick[0] = uint32_t(base + j);
            sh.pick[1] = remaining - c;
            break;
          }
          c += h;
        }
      }
      __syncthreads();
      prefix |= sh.pick[0] << shift;
      pmask |= dmask << shift;
      remaining = sh.pick[1];
      __syncthreads();
    }
    thr = prefix;
    need_eq = remaining;
  }

  // ordered compaction
  const int seg = ((n + NW - 1) / NW + kWave - 1) & ~(kWave - 1);
  const int s_lo = wave * seg;
  const int s_hi = min(n, s_lo + seg);
  uint32_t gt = 0u, eq = 0u;
  for (int base = s_lo; base < s_hi; base += kWave) {
    const int i = base + lane;
    const uint32_t k = i < s_hi ? key(i) : 0u;
    gt += __popcll(__ballot(k > thr));
    eq += __popcll(__ballot(i < s_hi && k == thr));
  }
  if (lane == 0) {
    sh.seg_cnt[wave] = gt;
    sh.seg_cnt[NW + wave] = eq;
  }
  __syncthreads();
  uint32_t gt_before = 0u, eq_before = 0u;
  for (int w = 0; w < wave; ++w) {
    gt_before += sh.seg_cnt[w];
    eq_before += sh.seg_cnt[NW + w];
  }
  const uint64_t lt = lanemask_lt();
  for (int base = s_lo; base < s_hi; base += kWave) {
    const int i = base + lane;
    const uint32_t k = i < s_hi ? key(i) : 0u;
    const bool is_gt = k > thr;
    const bool is_eq = i < s_hi && k == thr;
    const uint64_t mgt = __ballot(is_gt);
    const uint64_t meq = __ballot(is_eq);
    const uint32_t eq_rank = eq_before + uint32_t(__popcll(meq & lt));
    if (is_gt || (is_eq && eq_rank < need_eq)) {
      const uint32_t pos = gt_before + uint32_t(__popcll(mgt & lt)) + min(eq_rank, need_eq);
      if (pos < uint32_t(K)) emit(pos, i, k);
    }
    gt_before += uint32_t(__popcll(mgt));
    eq_before += uint32_t(__popcll(meq));
  }
}

// Keys of scores[a .. a+n) into LDS (n <= kCap); returns the selectable count.
__device__ __forceinline__ uint32_t load_keys(const float* src, int n, uint32_t* keys,
                                              SelectShared<kThreads>& sh) {
  uint32_t cnt = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const uint32_t k = score_key(src[i]);
    keys[i] = k;
    cnt += (k != 0u);
  }
  return block_sum<kThreads>(cnt, sh.tmp);  // also orders the LDS writes
}

// Whole row by one workgroup; writes topk_idx[row] including the -1 padding.
__device__ __forceinline__ void row_topk(const float* __restrict__ scores, int64_t ld,
                                         int64_t row, int a, int b, int32_t K,
                                         int32_t* __restrict__ out, uint32_t* keys,
                                         SelectShared<kThreads>& sh) {
  const int n = b > a ? b - a : 0;
  const float* src = scores + row * ld + a;
  int32_t* dst = out + row * int64_t(K);
  uint32_t n_sel;
  auto emit = [&](uint32_t p, int i, uint32_t) { dst[p] = a + i; };
  if (n <= kCap) {
    n_sel = load_keys(src, n, keys, sh);
    select_topk<kThreads>(LdsKeys{keys}, n, n_sel, K, sh, emit);
  } else {
    uint32_t cnt = 0;
    for (int i = threadIdx.x; i < n; i += kThreads) cnt += (score_key(src[i]) != 0u);
    n_sel = block_sum<kThreads>(cnt, sh.tmp);
    select_topk<kThreads>(GlobalKeys{src}, n, n_sel, K, sh, emit);
  }
  const uint32_t k_eff = n_sel < uint32_t(K) ? n_sel : uint32_t(K);
  for (uint32_t p = k_eff + threadIdx.x; p < uint32_t(K); p += kThreads) dst[p] = -1;
}

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ row_ends, int32_t K, int32_t* __restrict__ out) {
  __shared__ uint32_t keys[kCap];
  __shared__ SelectShared<kThreads> sh;
  const int64_t row = blockIdx.x;
  row_topk(scores, ld, row, row_starts[row], row_ends[row], K, out, keys, sh);
}

// Chunk length of a window on the split path (multiple of 64), or 0 when the
// row is handled whole by chunk 0 (short windows, and windows too long for 16
// LDS-resident chunks).
__device__ __forceinline__ int split_chunk_len(int n) {
  if (n <= kCap || n > kMaxChunks * kCap) return 0;
  const int c = (n + kMaxChunks - 1) / kMaxChunks;
  return (c + kWave - 1) & ~(kWave - 1);
}

// Split path, phase 1: workgroup (row, c) selects the top-k of chunk c.
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ row_ends, int32_t K, int32_t* __restrict__ out,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_col,
    int32_t* __restrict__ cand_cnt) {
  __shared__ uint32_t keys[kCap];
  __shared__ SelectShared<kThreads> sh;
  const int64_t row = blockIdx.x;
  const int c = blockIdx.y;
  const int a = row_starts[row];
  const int b = row_ends[row];
  const int n = b > a ? b - a : 0;
  const int clen = split_chunk_len(n);
  if (clen == 0) {
    if (c == 0) row_topk(scores, ld, row, a, b, K, out, keys, sh);
    return;
  }
  const int64_t slot = row * kMaxChunks + c;
  const int lo = c * clen;
  const int m = lo < n ? min(clen, n - lo) : 0;
  const uint32_t n_sel = load_keys(scores + row * ld + a + lo, m, keys, sh);
  uint32_t* ck = cand_key + slot * K;
  int32_t* cc = cand_col + slot * K;
  select_topk<kThreads>(LdsKeys{keys}, m, n_sel, K, sh, [&](uint32_t p, int i, uint32_t k) {
    ck[p] = k;
    cc[p] = a + lo + i;
  });
  if (threadIdx.x == 0) cand_cnt[slot] = int32_t(n_sel < uint32_t(K) ? n_sel : uint32_t(K));
}

// Split path, phase 2: merge the candidates of a row (chunk order = column
// order) and write the row's top-k with its -1 padding.
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int32_t K,
    int32_t* __restrict__ out, const uint32_t* __restrict__ cand_key,
    const int32_t* __restrict__ cand_col, const int32_t* __restrict__ cand_cnt) {
  __shared__ uint32_t keys[kMergeCap];
  __shared__ int off[kMaxChunks + 1];
  __shared__ SelectShared<kMergeThreads> sh;
  const int64_t row = blockIdx.x;
  const int n_win = row_ends[row] - row_starts[row];
  if (split_chunk_len(n_win) == 0) return;  // written whole by phase 1
  if (threadIdx.x == 0) {
    int o = 0;
    for (int c = 0; c < kMaxChunks; ++c) {
      off[c] = o;
      o += cand_cnt[row * kMaxChunks + c];
    }
    off[kMaxChunks] = o;
  }
  __syncthreads();
  const int n = off[kMaxChunks];
  for (int c = 0; c < kMaxChunks; ++c) {
    const uint32_t* ck = cand_key + (row * kMaxChunks + c) * int64_t(K);
    for (int i = threadIdx.x; i < off[c + 1] - off[c]; i += kMergeThreads)
      keys[off[c] + i] = ck[i];
  }
  __syncthreads();
  int32_t* dst = out + row * int64_t(K);
  // every candidate is selectable (-inf never becomes one)
  select_topk<kMergeThreads>(LdsKeys{keys}, n, uint32_t(n), K, sh,
                             [&](uint32_t p, int i, uint32_t) {
    int c = 0;
    while (off[c + 1] <= i) ++c;
    dst[p] = cand_col[(row * kMaxChunks + c) * int64_t(K) + (i - off[c])];
  });
  for (int p = (n < K ? n : K) + threadIdx.x; p < K; p += kMergeThreads) dst[p] = -1;
}

bool use_split(int64_t n_q, int64_t n_cols, int32_t K) {
  return n_cols > kCap && K <= kMaxSplitK && n_q <= kMaxSplitRows;
}

}  // namespace

size_t topk_workspace_bytes(int64_t n_q, int64_t n_cols, int32_t K) {
  if (n_q <= 0 || !use_split(n_q, n_cols, K)) return 0;
  const size_t slots = size_t(n_q) * kMaxChunks;
  return slots * size_t(K) * (sizeof(uint32_t) + sizeof(int32_t)) + slots * sizeof(int32_t);
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_starts,
                       const int32_t* row_ends, int64_t n_q, int64_t n_cols, int32_t K,
                       int32_t* out, void* workspace, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  if (!use_split(n_q, n_cols, K)) {
    hipLaunchKernelGGL(topk_rows_kernel, dim3(unsigned(n_q)), dim3(kThreads), 0, stream, scores,
                       ld, row_starts, row_ends, K, out);
    return hipGetLastError();
  }
  const size_t slots = size_t(n_q) * kMaxChunks;
  uint32_t* cand_key = static_cast<uint32_t*>(workspace);
  int32_t* cand_col = reinterpret_cast<int32_t*>(cand_key + slots * K);
  int32_t* cand_cnt = cand_col + slots * K;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(unsigned(n_q), kMaxChunks), dim3(kThreads), 0,
                     stream, scores, ld, row_starts, row_ends, K, out, cand_key, cand_col,
                     cand_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(n_q)), dim3(kMergeThreads), 0, stream,
                     row_starts, row_ends, K, out, cand_key, cand_col, cand_cnt);
  return hipGetLastError();
}

}  // namespace dsa
