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
//      MSB-first radix passes of at most 11 bits (a 2048-bin LDS histogram; 10
//      bits and 1024 bins in the rows kernels, for the LDS it frees) that
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
//            registers, longer ones are re-read from global memory by each
//            pass (the split path's chunks hold theirs in LDS);
//   stream   many rows over more than 8192 columns: the rows kernel takes the
//            windows of at most 8192 keys, and a second kernel streams each
//            longer window through LDS with its running top-k;
//   split    for few rows with long windows (decode): a row's window is cut into
//            up to 16 chunks of at most 8192 keys, each workgroup selects its
//            chunk's top-k into a candidate list (key, column) in the workspace,
//            and a merge workgroup per row selects the top-k of the candidates.
//            Exact: a key of the row's top-k (ties to the lowest column) is in
//            its chunk's top-k under the same rule, and the candidates of chunk
//            c precede those of chunk c+1, so the merged output stays ascending.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "topk_select.h"

namespace dsa {
namespace {

using namespace topksel;

// The selection state of the rows and chunk kernels: a 1024-bin histogram
// (10-bit digits) and up to 704 boundary-digit keys refined on their own take
// 7.7 KB instead of 13.4 KB (with keys in LDS this made room for six
// workgroups per CU beside 4096 keys instead of five: 30.2 -> 28.5 us at
// prefill4k, 434 -> 397 us at THD).
using RowSel = SelectShared<kThreads, 1024, 704>;

constexpr int kShortRow = 2048;  // windows of at most this many keys and k: no selection

// A window of at most min(k, kShortRow) keys: every selectable key is
// selected.  The ordered compaction straight from the scores in registers (wave
// w: its contiguous segment, lane-strided), one barrier for the wave totals, no
// LDS copy of the keys.
__device__ __forceinline__ void row_topk_short(const float* __restrict__ src, int n, int a,
                                               int32_t K, int32_t* __restrict__ dst,
                                               RowSel& sh) {
  constexpr int kPer = kShortRow / kThreads;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t lt = lanemask_lt();
  int s_lo, s_hi;
  select_segment<kThreads>(n, s_lo, s_hi);  // at most kShortRow / kWaves keys
  float x[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = s_lo + j * kWave + lane;
    x[j] = i < s_hi ? src[i] : -INFINITY;
  }
  uint64_t m[kPer];
  uint32_t cnt = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    m[j] = __ballot(score_key(x[j]) != 0u);
    cnt += uint32_t(__popcll(m[j]));
  }
  if (lane == 0) sh.seg_cnt[wave] = cnt;
  __syncthreads();
  uint32_t base = 0u, total = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = sh.seg_cnt[w];
    base += w < wave ? c : 0u;
    total += c;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if ((m[j] >> lane) & 1ull)
      dst[base + uint32_t(__popcll(m[j] & lt))] = a + s_lo + j * kWave + lane;
    base += uint32_t(__popcll(m[j]));
  }
  for (uint32_t p = total + threadIdx.x; p < uint32_t(K); p += kThreads) dst[p] = -1;
}

// A window too long for the keys to be held: every pass re-reads (and maps)
// the scores from global memory.  Returns the selectable count; the caller
// writes the -1 padding.
__device__ __forceinline__ uint32_t row_topk_global(const float* __restrict__ src, int n, int a,
                                                    int32_t K, int32_t* __restrict__ dst,
                                                    RowSel& sh) {
  uint32_t cnt = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) cnt += (score_key(src[i]) != 0u);
  const uint32_t n_sel = block_sum<kThreads>(cnt, sh.tmp);
  select_topk<kThreads>(GlobalKeys{src}, n, n_sel, K, sh,
                        [&](uint32_t p, int i, uint32_t) { dst[p] = a + i; });
  return n_sel;
}

// The n keys of scores src[0 .. n) into registers, in the layout of the
// ordered compaction: thread (wave w, lane l) holds key s_lo + j * 64 + l of
// its wave's segment [s_lo, s_hi) in k[j] (key 0 past s_hi; n <= PER * kThreads).
// Every load is issued before any is used.  Returns the selectable count and
// the range of the selectable keys.
template <int PER>
__device__ __forceinline__ uint32_t load_keys_regs(const float* __restrict__ src, int n,
                                                   uint32_t (&k)[PER], int& s_lo, RowSel& sh,
                                                   KeyRange& kr) {
  const int lane = threadIdx.x & (kWave - 1);
  int s_hi;
  select_segment<kThreads>(n, s_lo, s_hi);  // at most PER * kWave keys per wave
  {
    float x[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = s_lo + j * kWave + lane;
      x[j] = i < s_hi ? src[i] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) k[j] = score_key(x[j]);  // -inf -> 0: not selectable
  }
  uint32_t cnt = 0, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (k[j] != 0u) {
      ++cnt;
      lo = min(lo, k[j]);
      hi = max(hi, k[j]);
    }
  }
  return block_count_range<kThreads>(cnt, lo, hi, sh, kr);
}

// Whole row [a, a + n) by one workgroup; writes dst[0 .. K) including the -1
// padding.  A window of at most min(k, kShortRow) keys takes the short path;
// one of at most CAP keys keeps them in registers (CAP / kThreads per thread),
// so none of the selection's passes reads LDS and the selection state is the
// only LDS a row takes; a longer one re-reads the scores from memory per pass.
template <int CAP>
__device__ __forceinline__ void row_topk(const float* __restrict__ src, int n, int a, int32_t K,
                                         int32_t* __restrict__ dst, RowSel& sh) {
  static_assert(CAP % kThreads == 0, "whole keys per thread");
  uint32_t n_sel;
  if (n <= K && n <= kShortRow) {
    row_topk_short(src, n, a, K, dst, sh);
    return;
  }
  if (n <= CAP) {
    uint32_t k[CAP / kThreads];
    int s_lo;
    KeyRange kr;
    n_sel = load_keys_regs(src, n, k, s_lo, sh, kr);
    select_topk<kThreads>(RegKeys<CAP / kThreads>{k, s_lo}, n, n_sel, K, sh,
                          [&](uint32_t p, int i, uint32_t) { dst[p] = a + i; }, kr);
  } else {
    n_sel = row_topk_global(src, n, a, K, dst, sh);
  }
  const uint32_t k_eff = n_sel < uint32_t(K) ? n_sel : uint32_t(K);
  for (uint32_t p = k_eff + threadIdx.x; p < uint32_t(K); p += kThreads) dst[p] = -1;
}

// Rows whose window is longer than CAP (skip_long) or at most `skip_below`
// keys are left to another launch.  The keys of a window stay in registers
// (CAP / kThreads per thread: 76 VGPRs at 4096, six workgroups per CU; 108 at
// 8192, four), and the selection state is the only LDS (7.7 KB): against
// holding the keys in LDS, 28.8 -> 27.4 us at prefill4k and 387 -> 354 us at
// THD, the same output.  Windows too long for the registers (possible only
// when k is past the stream path's limit) re-read the scores from memory.
template <int CAP>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ row_ends, int n_cols, int32_t K, int32_t* __restrict__ out,
    int skip_long, int skip_below) {
  __shared__ RowSel sh;
  // last rows first: in a causal prefill they hold the longest windows, and
  // starting them first leaves the short ones for the end of the launch
  const int64_t row = int64_t(gridDim.x) - 1 - blockIdx.x;
  const int a = max(row_starts[row], 0);  // windows are clamped to the columns [0, n_cols)
  const int b = min(row_ends[row], n_cols);
  const int n = b > a ? b - a : 0;
  if ((skip_long && n > CAP) || n <= skip_below) return;
  row_topk<CAP>(scores + row * ld + a, n, a, K, out + row * int64_t(K), sh);
}

// Split path, phase 1: workgroup (row, c) selects the top-k of chunk c.
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ row_ends, int n_cols, int32_t K, int32_t* __restrict__ out,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_col,
    int32_t* __restrict__ cand_cnt) {
  __shared__ RowSel sh;
  const int64_t row = blockIdx.x;
  const int c = blockIdx.y;
  const int a = max(row_starts[row], 0);  // clamped to the columns
  const int b = min(row_ends[row], n_cols);
  const int n = b > a ? b - a : 0;
  const int clen = split_chunk_len(n);
  if (clen == 0) {
    if (c == 0) row_topk<kCap>(scores + row * ld + a, n, a, K, out + row * int64_t(K), sh);
    return;
  }
  const int64_t slot = row * kMaxChunks + c;
  const int lo = c * clen;
  const int m = lo < n ? min(clen, n - lo) : 0;  // at most kCap
  uint32_t k[kCap / kThreads];
  int s_lo;
  KeyRange kr;
  const uint32_t n_sel = load_keys_regs(scores + row * ld + a + lo, m, k, s_lo, sh, kr);
  uint32_t* ck = cand_key + slot * K;
  int32_t* cc = cand_col + slot * K;
  select_topk<kThreads>(
      RegKeys<kCap / kThreads>{k, s_lo}, m, n_sel, K, sh,
      [&](uint32_t p, int i, uint32_t k) {
        ck[p] = k;
        cc[p] = a + lo + i;
      },
      kr);
  if (threadIdx.x == 0) cand_cnt[slot] = int32_t(n_sel < uint32_t(K) ? n_sel : uint32_t(K));
}

// Split path, phase 2: merge candidate slots (slot order = column order), in
// two levels so that the whole GPU takes part.  Level 1 (kFinal = false):
// workgroup (row, g) merges the kGroup slots from g * kGroup and writes its
// top-k back as the candidates of slot g * kGroup (every slot it reads is read
// before any is written, and no other workgroup reads them).  Level 2 (kFinal):
// one workgroup per row merges the slots 0, kStride, 2 kStride, ... and writes
// the row's top-k with its -1 padding.
template <int kGroup, int kStride, bool kFinal>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int n_cols,
    int32_t K, int32_t* __restrict__ out, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_col, int32_t* __restrict__ cand_cnt) {
  __shared__ uint32_t keys[kGroup * kMaxSplitK];
  __shared__ int sel[kMaxSplitK];  // selected candidate positions, then (level 1) their columns
  __shared__ uint32_t skey[kFinal ? 1 : kMaxSplitK];
  __shared__ int off[kGroup + 1];
  __shared__ SelectShared<kMergeThreads> sh;
  const int64_t row = blockIdx.x;
  // the window as phase 1 clamped it
  const int n_win = max(min(row_ends[row], n_cols) - max(row_starts[row], 0), 0);
  if (split_chunk_len(n_win) == 0) return;  // written whole by phase 1
  const int64_t slot0 = row * kMaxChunks + int64_t(blockIdx.y) * kGroup * kStride;
  if (threadIdx.x == 0) {
    int o = 0;
    for (int m = 0; m < kGroup; ++m) {
      off[m] = o;
      o += cand_cnt[slot0 + m * kStride];
    }
    off[kGroup] = o;
  }
  __syncthreads();
  const int n = off[kGroup];
  // every thread issues all its candidate loads before storing any of them:
  // slot s of member m for s = tid, tid + kMergeThreads (k <= 2048)
  constexpr int kPer = kMaxSplitK / kMergeThreads;
  {
    uint32_t v[kGroup][kPer];
#pragma unroll
    for (int m = 0; m < kGroup; ++m) {
      const uint32_t* ck = cand_key + (slot0 + m * kStride) * int64_t(K);
      const int cnt = off[m + 1] - off[m];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int sl = int(threadIdx.x) + j * kMergeThreads;
        v[m][j] = sl < cnt ? ck[sl] : 0u;
      }
    }
#pragma unroll
    for (int m = 0; m < kGroup; ++m) {
      const int cnt = off[m + 1] - off[m];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int sl = int(threadIdx.x) + j * kMergeThreads;
        if (sl < cnt) keys[off[m] + sl] = v[m][j];
      }
    }
  }
  __syncthreads();
  // every candidate is selectable (-inf never becomes one); the selection is
  // recorded as candidate positions first, so that the column loads below are
  // independent of each other instead of one per step of the compaction
  select_topk<kMergeThreads>(LdsKeys{keys}, n, uint32_t(n), K, sh,
                             [&](uint32_t p, int i, uint32_t) { sel[p] = i; });
  __syncthreads();
  const int k_eff = n < K ? n : K;
  auto column = [&](int i) {
    int m = 0;
    while (off[m + 1] <= i) ++m;
    return cand_col[(slot0 + m * kStride) * int64_t(K) + (i - off[m])];
  };
  if constexpr (kFinal) {
    int32_t* dst = out + row * int64_t(K);
    for (int p = threadIdx.x; p < K; p += kMergeThreads) dst[p] = p < k_eff ? column(sel[p]) : -1;
  } else {
    // gather the selection in LDS (its columns read from every member slot)
    // before slot0 is overwritten
    int cv[kPer];
    uint32_t kv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = int(threadIdx.x) + j * kMergeThreads;
      if (p < k_eff) {
        const int i = sel[p];
        cv[j] = column(i);
        kv[j] = keys[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = int(threadIdx.x) + j * kMergeThreads;
      if (p < k_eff) {
        sel[p] = cv[j];
        skey[p] = kv[j];
      }
    }
    __syncthreads();
    uint32_t* ck = cand_key + slot0 * int64_t(K);
    int32_t* cc = cand_col + slot0 * int64_t(K);
    for (int p = threadIdx.x; p < k_eff; p += kMergeThreads) {
      ck[p] = skey[p];
      cc[p] = sel[p];
    }
    if (threadIdx.x == 0) cand_cnt[slot0] = k_eff;
  }
}

// Many rows over more than 8192 columns (k <= 2048): a row is streamed through
// LDS in pieces of kPiece keys.  The keys that can still be in the top-k are
// held in LDS with their columns, in column order; a new key enters only if it
// is above the floor (a key not above it has at least k keys above it, or is
// the k-th key of everything seen with an older, lower-column tie).  When a
// piece's survivors do not fit, the floor is raised and the held keys are
// compacted: one histogram pass over them (the first digit of the exact
// search) finds the digit that holds their k-th key, every key below that digit
// goes, and when that leaves room for a piece the held keys above the floor are
// compacted in place; otherwise (a crowded digit: many equal keys) they are
// shrunk in place to their exact top k.  The scores are read once.  The held
// keys carry their offsets in the window: 16-bit for windows of at most 65536
// keys (38.8 KB of LDS, at most 128 VGPRs: four workgroups per CU, which the
// per-piece barriers need more than anything else), else 32-bit (47.2 KB: three).
constexpr int kPiece = 2048;
constexpr int kSlack = 128;  // held keys past k that the histogram shrink may keep
constexpr int kHeldCap = kMaxSplitK + kPiece + kSlack;

template <typename ColT>
struct StreamShared {
  uint32_t keys[kHeldCap];
  ColT cols[kHeldCap];  // offset of each held key in the row's window
  uint32_t wcnt[2 * kWaves];
  SelectShared<kThreads> sel;
};

template <typename ColT>
__global__ __launch_bounds__(kThreads, sizeof(ColT) == 2 ? 4 : 1) void topk_stream_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ row_ends, int n_cols, int32_t K, int32_t* __restrict__ out) {
  __shared__ StreamShared<ColT> sh;
  constexpr int kPer = kPiece / kThreads;  // keys per thread per piece
  const int64_t row = int64_t(gridDim.x) - 1 - blockIdx.x;  // last (causal: longest) rows first
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int a = max(row_starts[row], 0);  // clamped to the columns
  const int b = min(row_ends[row], n_cols);
  const int n = b > a ? b - a : 0;
  const float* src = scores + row * ld + a;
  int32_t* dst = out + row * int64_t(K);
  if (n <= kCap) return;  // held whole by the rows kernel of the same launch
  const uint64_t lt = lanemask_lt();

  int ncand = 0;           // keys held in LDS (the running set, then survivors)
  uint32_t floor_key = 0;  // keys <= floor_key cannot enter (0: not selectable)
  // wave w owns keys [w*kPiece/4, (w+1)*kPiece/4) of a piece, lane-strided; the
  // next piece's scores are loaded while the current one is processed
  auto load_piece = [&](int lo, float (&f)[kPer]) {
    const int m = lo < n ? min(kPiece, n - lo) : 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = wave * (kPiece / kWaves) + j * kWave + lane;
      f[j] = i < m ? src[lo + i] : -INFINITY;
    }
  };
  // In-place ordered compaction of the held keys: those > thr and the first
  // need_eq of those == thr (in column order) stay.  Every wave reads its
  // segment into registers and counts (barrier), then writes its kept keys at
  // their new positions (barrier); all reads precede all writes.
  auto compact_held = [&](uint32_t thr, uint32_t need_eq, int cnt) {
    constexpr int kHeldPer = (kHeldCap + kThreads - 1) / kThreads;
    int s_lo, s_hi;
    select_segment<kThreads>(cnt, s_lo, s_hi);
    uint32_t hk[kHeldPer];
    ColT hc[kHeldPer];
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int j = 0; j < kHeldPer; ++j) {
      const int i = s_lo + j * kWave + lane;
      hk[j] = i < s_hi ? sh.keys[i] : 0u;
      hc[j] = i < s_hi ? sh.cols[i] : ColT(0);
    }
#pragma unroll
    for (int j = 0; j < kHeldPer; ++j) {
      gt += __popcll(__ballot(hk[j] > thr));
      eq += __popcll(__ballot(hk[j] == thr && s_lo + j * kWave + lane < s_hi));
    }
    if (lane == 0) {
      sh.wcnt[wave] = gt;
      sh.wcnt[kWaves + wave] = eq;
    }
    __syncthreads();
    uint32_t gt_before = 0u, eq_before = 0u;
    for (int w = 0; w < wave; ++w) {
      gt_before += sh.wcnt[w];
      eq_before += sh.wcnt[kWaves + w];
    }
#pragma unroll
    for (int j = 0; j < kHeldPer; ++j) {
      const bool is_gt = hk[j] > thr;
      const bool is_eq = hk[j] == thr && s_lo + j * kWave + lane < s_hi;
      const uint64_t mgt = __ballot(is_gt);
      const uint64_t meq = __ballot(is_eq);
      const uint32_t eq_rank = eq_before + uint32_t(__popcll(meq & lt));
      if (is_gt || (is_eq && eq_rank < need_eq)) {
        const uint32_t at = gt_before + uint32_t(__popcll(mgt & lt)) + min(eq_rank, need_eq);
        sh.keys[at] = hk[j];
        sh.cols[at] = hc[j];
      }
      gt_before += uint32_t(__popcll(mgt));
      eq_before += uint32_t(__popcll(meq));
    }
    __syncthreads();
  };
  float fnext[kPer];
  load_piece(0, fnext);
  for (int lo = 0;; lo += kPiece) {
    const int m = lo < n ? min(kPiece, n - lo) : 0;
    uint32_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = score_key(fnext[j]);  // -inf -> 0: not selectable
    load_piece(lo + kPiece, fnext);
    auto survivors = [&]() {  // survivors of this wave's part (uniform per wave)
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) c += __popcll(__ballot(v[j] > floor_key));
      if (lane == 0) sh.wcnt[wave] = c;
      __syncthreads();
      int tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += int(sh.wcnt[w]);
      return tot;
    };
    int s_all = survivors();
    if (ncand + s_all > kHeldCap) {
      // no room: raise the floor from the first digit of the held keys' k-th key
      bool shrunk = false;
      {
        RadixSearch<kThreads> rs{sh.sel};
        rs.init(LdsKeys{sh.keys}, ncand, K, KeyRange{});
        if (rs.shift > 0) {
          const uint32_t in_bin = rs.pass(LdsKeys{sh.keys}, ncand);
          // keys whose d has the picked digit or a higher one: at least k
          const uint32_t keep = uint32_t(K) - rs.remaining + in_bin;
          if (keep <= uint32_t(kMaxSplitK + kSlack)) {
            // every key <= f is below all of those keys
            const uint32_t f = rs.kmin + rs.prefix - 1u;
            compact_held(f, 0u, ncand);
            ncand = int(keep);
            floor_key = f;
            shrunk = true;
          }
        }
      }
      if (!shrunk) {
        // a crowded digit: shrink the held keys in place to their exact top k
        const SelectThreshold r =
            select_search<kThreads>(LdsKeys{sh.keys}, ncand, uint32_t(ncand), K, sh.sel);
        compact_held(r.thr, r.need_eq, ncand);
        ncand = K;
        floor_key = r.thr;  // the k-th key of everything seen so far
      }
      s_all = survivors();
    }
    // ordered compaction of the survivors behind the held keys
    int base = ncand;
    for (int w = 0; w < wave; ++w) base += int(sh.wcnt[w]);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool keep = v[j] > floor_key;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int at = base + __popcll(bal & lt);
        sh.keys[at] = v[j];
        sh.cols[at] = ColT(lo + wave * (kPiece / kWaves) + j * kWave + lane);
      }
      base += __popcll(bal);
    }
    ncand += s_all;
    __syncthreads();
    if (lo + m >= n) {
      select_topk<kThreads>(LdsKeys{sh.keys}, ncand, uint32_t(ncand), K, sh.sel,
                            [&](uint32_t p, int i, uint32_t) { dst[p] = a + int(sh.cols[i]); });
      for (int p = (ncand < K ? ncand : K) + tid; p < K; p += kThreads) dst[p] = -1;
      return;
    }
  }
}

bool use_split(int64_t n_q, int64_t n_cols, int32_t K) {
  return n_cols > kCap && K <= kMaxSplitK && n_q <= kMaxSplitRows;
}

}  // namespace

size_t topk_workspace_bytes(int64_t n_q, int64_t n_cols, int32_t K) {
  if (n_q <= 0 || !use_split(n_q, n_cols, K)) return 0;
  return Candidates::bytes(n_q, K);
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_starts,
                       const int32_t* row_ends, int64_t n_q, int64_t n_cols, int32_t K,
                       int32_t* out, void* workspace, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  if (!use_split(n_q, n_cols, K)) {
    // windows of at most kCap keys: held whole in LDS by the rows kernel; longer
    // ones (only possible when n_cols > kCap) streamed by the stream kernel
    const bool stream_long = n_cols > kCap && K <= kMaxSplitK;
    // windows of at most 4096 keys: the 4096-key instance; longer ones up to
    // kCap (and, without the stream kernel, all longer ones): the kCap instance
    hipLaunchKernelGGL(topk_rows_kernel<4096>, dim3(unsigned(n_q)), dim3(kThreads), 0, stream,
                       scores, ld, row_starts, row_ends, int(n_cols), K, out, 1, -1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (n_cols > 4096) {
      hipLaunchKernelGGL(topk_rows_kernel<kCap>, dim3(unsigned(n_q)), dim3(kThreads), 0, stream,
                         scores, ld, row_starts, row_ends, int(n_cols), K, out, int(stream_long),
                         4096);
      e = hipGetLastError();
    }
    if (e != hipSuccess || !stream_long) return e;
    // windows are clamped to the columns, so n_cols bounds every offset
    if (n_cols <= 65536)
      hipLaunchKernelGGL(topk_stream_kernel<uint16_t>, dim3(unsigned(n_q)), dim3(kThreads), 0,
                         stream, scores, ld, row_starts, row_ends, int(n_cols), K, out);
    else
      hipLaunchKernelGGL(topk_stream_kernel<uint32_t>, dim3(unsigned(n_q)), dim3(kThreads), 0,
                         stream, scores, ld, row_starts, row_ends, int(n_cols), K, out);
    return hipGetLastError();
  }
  const Candidates cd = Candidates::at(workspace, n_q, K);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(unsigned(n_q), kMaxChunks), dim3(kThreads), 0,
                     stream, scores, ld, row_starts, row_ends, int(n_cols), K, out, cd.key, cd.col,
                     cd.cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(row_starts, row_ends, n_q, n_cols, K, out, workspace, stream);
}

hipError_t launch_topk_merge(const int32_t* row_starts, const int32_t* row_ends, int64_t n_q,
                             int64_t n_cols, int32_t K, int32_t* out, void* workspace,
                             hipStream_t stream) {
  const Candidates cd = Candidates::at(workspace, n_q, K);
  constexpr int kGroup = 4;  // slots per level-1 merge
  static_assert(kMaxChunks == kGroup * kGroup, "two levels of kGroup-way merges");
  hipLaunchKernelGGL((topk_merge_kernel<kGroup, 1, false>), dim3(unsigned(n_q), kGroup),
                     dim3(kMergeThreads), 0, stream, row_starts, row_ends, int(n_cols), K, out,
                     cd.key, cd.col, cd.cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_merge_kernel<kGroup, kGroup, true>), dim3(unsigned(n_q), 1),
                     dim3(kMergeThreads), 0, stream, row_starts, row_ends, int(n_cols), K, out,
                     cd.key, cd.col, cd.cnt);
  return hipGetLastError();
}

}  // namespace dsa
