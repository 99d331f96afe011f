// Per-row top-k over a window of an fp32 score matrix (gfx950).
//
// Semantics follow the fallback top-k of review comment 3 of vime pull request
// #502 (window mask, k = min(topk, n), -inf -> -1, -1 padding), with ties to the
// lowest column and the selected columns written in ascending order.
//
// One workgroup (256 threads, 4 waves) per row:
//   1. map every in-window score to an order-preserving u32 key (score_key) and
//      count the selectable ones; rows of at most kCap keys are held in LDS, longer
//      rows are re-read from global memory (L2) by each pass;
//   2. if more than k are selectable, find the k-th largest key exactly with three
//      MSB-first radix passes (11 + 11 + 10 bits, 2048-bin LDS histogram): after
//      them `thr` is the k-th key and `need_eq` says how many keys equal to it
//      (the lowest-indexed ones) belong to the selection;
//   3. ordered compaction: each wave owns a contiguous segment of the window,
//      counts its (> thr) and (== thr) keys with ballots, the 4 wave totals are
//      scanned, and a second ballot/mbcnt pass writes every selected column at
//      position  #gt_before + min(#eq_before, need_eq);
//   4. the slots after min(k, #selectable) get -1.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCap = 8192;    // keys held in LDS
constexpr int kBins = 2048;   // 11-bit digit

struct RowKeys {
  const float* src;
  const uint32_t* lds;
  bool in_lds;
  __device__ __forceinline__ uint32_t operator()(int i) const {
    return in_lds ? lds[i] : score_key(src[i]);
  }
};

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ row_ends, int32_t K, int32_t* __restrict__ out) {
  __shared__ uint32_t keys[kCap];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[kWaves];
  __shared__ uint32_t seg_cnt[2 * kWaves];
  __shared__ uint32_t pick[2];

  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  const int a = row_starts[row];
  const int b = row_ends[row];
  const int n = b > a ? b - a : 0;
  const float* src = scores + row * ld + a;
  int32_t* dst = out + row * int64_t(K);
  const bool in_lds = n <= kCap;
  const RowKeys key{src, keys, in_lds};

  // 1. keys + number of selectable entries
  uint32_t cnt = 0;
  for (int i = tid; i < n; i += kThreads) {
    const uint32_t k = score_key(src[i]);
    if (in_lds) keys[i] = k;
    cnt += (k != 0u);
  }
  const uint32_t n_sel = block_sum<kThreads>(cnt, tmp);  // also orders the LDS writes

  // 2. exact k-th largest key
  uint32_t thr = 0u, need_eq = 0u;
  if (n_sel > uint32_t(K)) {
    uint32_t prefix = 0u, pmask = 0u, remaining = uint32_t(K);
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += kThreads) {
        const uint32_t k = key(i);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      // thread j owns the 8 bins of slot (kThreads-1-j), so an exclusive prefix
      // over threads is the count of keys in higher bins
      const int base = (kThreads - 1 - tid) * (kBins / kThreads);
      uint32_t local = 0u;
#pragma unroll
      for (int j = 0; j < kBins / kThreads; ++j) local += hist[base + j];
      uint32_t total;
      const uint32_t above = block_exclusive_sum<kThreads>(local, tmp, total);
      if (above < remaining && above + local >= remaining) {
        uint32_t c = above;
        for (int j = kBins / kThreads - 1; j >= 0; --j) {
          const uint32_t h = hist[base + j];
          if (c + h >= remaining) {
            pick[0] = uint32_t(base + j);
            pick[1] = remaining - c;
            break;
          }
          c += h;
        }
      }
      __syncthreads();
      prefix |= pick[0] << shift;
      pmask |= dmask << shift;
      remaining = pick[1];
      __syncthreads();
    }
    thr = prefix;
    need_eq = remaining;
  }

  // 3. ordered compaction
  const int seg = ((n + kWaves - 1) / kWaves + kWave - 1) & ~(kWave - 1);
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
    seg_cnt[wave] = gt;
    seg_cnt[kWaves + wave] = eq;
  }
  __syncthreads();
  uint32_t gt_before = 0u, eq_before = 0u;
  for (int w = 0; w < wave; ++w) {
    gt_before += seg_cnt[w];
    eq_before += seg_cnt[kWaves + w];
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
      if (pos < uint32_t(K)) dst[pos] = a + i;
    }
    gt_before += uint32_t(__popcll(mgt));
    eq_before += uint32_t(__popcll(meq));
  }

  // 4. -1 padding
  const uint32_t k_eff = n_sel < uint32_t(K) ? n_sel : uint32_t(K);
  for (uint32_t p = k_eff + tid; p < uint32_t(K); p += kThreads) dst[p] = -1;
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_starts,
                       const int32_t* row_ends, int64_t n_q, int32_t K, int32_t* out,
                       hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(unsigned(n_q)), dim3(kThreads), 0, stream,
                     scores, ld, row_starts, row_ends, K, out);
  return hipGetLastError();
}

}  // namespace dsa
