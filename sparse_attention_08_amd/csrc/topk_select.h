// Exact per-row top-k selection in LDS (gfx950), shared by the top-k kernels
// and the fused indexer + top-k kernel.  See topk.hip for the method.
#pragma once

#include "dsa_device.h"

namespace dsa {
namespace topksel {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCap = 8192;        // keys held in LDS by one workgroup
constexpr int kBins = 2048;       // 11-bit digit
constexpr int kMaxChunks = 16;    // chunks per row on the split path
constexpr int kMaxSplitK = 2048;  // largest k on the split path
constexpr int64_t kMaxSplitRows = 1024;
constexpr int kMergeThreads = 1024;
constexpr int kCandCap = 1024;   // boundary-bin keys refined on their own
constexpr int kRankMax = 128;    // up to this many: refined by counting ranks

// BINS: histogram bins (a power of two, at most 2^11: the radix digit); CC: keys
// of the boundary digit refined on their own.  Smaller values take less LDS.
template <int NT, int BINS = kBins, int CC = kCandCap>
struct SelectShared {
  static constexpr int kNW = NT / kWave;
  static constexpr int kDigitBits = __builtin_ctz(BINS);
  static_assert((BINS & (BINS - 1)) == 0 && BINS <= 2048 && BINS % NT == 0, "histogram bins");
  uint32_t hist[BINS];
  uint32_t tmp[3 * kNW];
  uint32_t seg_cnt[2 * kNW];
  uint32_t wsum[kNW];  // radix pass: wave totals of the bin counts
  uint32_t pick[3];    // radix pass: the digit, the rank left, the digit's count
  uint32_t ccount;     // boundary-bin keys gathered
  alignas(16) uint32_t ckey[CC + 4];  // the boundary bin's keys (4 zero keys after the last) ...
  uint8_t cwave[CC];                  // ... and the wave whose segment each came from
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

// The key loops below read kBatch keys before they use any of them: a loop that
// uses each key as it is read waits a full LDS (or memory) round trip per key.
constexpr int kBatch = 8;

// f(i, key(i)) for this thread's keys i = tid, tid + NT, ... < n, in that order.
template <int NT, class Keys, class F>
__device__ __forceinline__ void for_keys(const Keys& key, int n, F f) {
  for (int base = int(threadIdx.x); base < n; base += NT * kBatch) {
    uint32_t k[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * NT;
      k[u] = i < n ? key(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * NT;
      if (i < n) f(i, k[u]);
    }
  }
}

// f(i, key) for i = s_lo + lane, s_lo + lane + 64, ... over the wave's segment
// [s_lo, s_hi) (s_lo a multiple of 64): every lane of the wave calls f the same
// number of times (key 0 past the end), so f may use wave-wide ballots.
template <class Keys, class F>
__device__ __forceinline__ void for_segment(const Keys& key, int s_lo, int s_hi, int lane, F f) {
  for (int base = s_lo; base < s_hi; base += kWave * kBatch) {
    uint32_t k[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * kWave + lane;
      k[u] = i < s_hi ? key(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (base + u * kWave < s_hi) f(base + u * kWave + lane, k[u]);
    }
  }
}

// A row's keys held in registers: thread (wave w, lane l) holds key
// s_lo + j * 64 + l of its wave's compaction segment [s_lo, s_hi) in k[j]
// (key 0 past s_hi), so the passes below read no LDS.  The overloads of
// for_keys and for_segment visit this thread's registers.
template <int PER>
struct RegKeys {
  const uint32_t (&k)[PER];
  int s_lo;
};
// all of this thread's keys (0 past the segment: never counted)
template <int NT, int PER, class F>
__device__ __forceinline__ void for_keys(const RegKeys<PER>& key, int, F f) {
#pragma unroll
  for (int j = 0; j < PER; ++j) f(key.s_lo + j * kWave + int(threadIdx.x & (kWave - 1)), key.k[j]);
}
template <int PER, class F>
__device__ __forceinline__ void for_segment(const RegKeys<PER>& key, int s_lo, int s_hi, int lane,
                                            F f) {
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (s_lo + j * kWave < s_hi) f(s_lo + j * kWave + lane, key.k[j]);
  }
}

// Radix search for the k-th largest selectable key.  init() takes the min and
// max of the selectable keys (and clears the histogram, ordered by its
// barriers); the digits are then taken from d = key - kmin over the bits of
// kmax - kmin, most significant first, at most 11 at a time.  After each pass()
// `prefix` holds the digits of d picked so far (the bits under pmask), the
// k-th largest key lies among the keys whose d has that prefix, and it is the
// `remaining`-th largest of them.
// The smallest and largest selectable (nonzero) key of a row, when the caller
// already has them (the keys were mapped in registers on their way to LDS);
// `known` is uniform over the workgroup.
struct KeyRange {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  bool known = false;
};

// Count, smallest and largest selectable key over the workgroup in one
// reduction of per-thread values (two barriers: the first also orders the
// caller's earlier LDS writes, the second the reuse of tmp).  Returns the count
// and fills kr.
template <int NT, int B, int C>
__device__ __forceinline__ uint32_t block_count_range(uint32_t cnt, uint32_t lo, uint32_t hi,
                                                      SelectShared<NT, B, C>& sh, KeyRange& kr) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    cnt += uint32_t(__shfl_xor(int(cnt), o));
    lo = min(lo, uint32_t(__shfl_xor(int(lo), o)));
    hi = max(hi, uint32_t(__shfl_xor(int(hi), o)));
  }
  if (lane == 0) {
    sh.tmp[wave] = cnt;
    sh.tmp[NW + wave] = lo;
    sh.tmp[2 * NW + wave] = hi;
  }
  __syncthreads();
  cnt = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    cnt += sh.tmp[w];
    lo = min(lo, sh.tmp[NW + w]);
    hi = max(hi, sh.tmp[2 * NW + w]);
  }
  __syncthreads();
  kr.lo = lo;
  kr.hi = hi;
  kr.known = true;
  return cnt;
}

template <int NT, int B = kBins, int C = kCandCap>
struct RadixSearch {
  SelectShared<NT, B, C>& sh;
  uint32_t kmin = 0u;
  int shift = 0;        // d's bits below the digits picked so far
  uint32_t pmask = 0u;
  uint32_t prefix = 0u;
  uint32_t remaining = 0u;

  template <class Keys>
  __device__ __forceinline__ void init(const Keys& key, int n, int K, const KeyRange& kr) {
    for (int i = int(threadIdx.x); i < B; i += NT) sh.hist[i] = 0u;
    uint32_t lo = kr.lo, hi = kr.hi;
    if (kr.known) {
      __syncthreads();  // orders the clears before the first pass's counts
    } else {
      for_keys<NT>(key, n, [&](int, uint32_t k) {
        if (k != 0u) {
          lo = min(lo, k);
          hi = max(hi, k);
        }
      });
      block_min_max<NT>(lo, hi, sh.tmp);  // its barrier also orders the clears
    }
    kmin = lo;
    const uint32_t range = hi - lo;  // d in [0, range]
    shift = range == 0u ? 0 : 32 - __builtin_clz(range);
    pmask = shift >= 32 ? 0u : ~((1u << shift) - 1u);
    prefix = 0u;
    remaining = uint32_t(K);
  }

  // One radix pass over keys(0..cnt-1): histogram (barrier); every thread reads
  // its bins into registers and clears them, wave prefix sums by DPP, wave
  // totals (barrier); the thread whose bins hold the k-th key picks the digit
  // (barrier).  The wave totals are read before the third barrier and written
  // again only before the next pass's second; the pick is read after the third
  // and written again only after the next pass's second.  Returns the number of
  // keys with the picked digit.
  template <class Keys>
  __device__ __forceinline__ uint32_t pass(const Keys& keys, int cnt) {
    constexpr int NW = NT / kWave;
    constexpr int kBPT = B / NT;  // histogram bins owned per thread in the scan
    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    constexpr int kDig = SelectShared<NT, B, C>::kDigitBits;
    const int nb = shift < kDig ? shift : kDig;
    shift -= nb;
    const uint32_t dmask = (1u << nb) - 1u;
    const uint32_t km = kmin, pm = pmask, pf = prefix;
    const int sh_ = shift;
    for_keys<NT>(keys, cnt, [&](int, uint32_t k) {
      const uint32_t d = k - km;
      if (k != 0u && (d & pm) == pf) atomicAdd(&sh.hist[(d >> sh_) & dmask], 1u);
    });
    __syncthreads();
    // thread j owns the bins of slot (NT-1-j), so an exclusive prefix over
    // threads is the count of keys in higher bins
    const int base = (NT - 1 - tid) * kBPT;
    uint32_t h[kBPT];
    uint32_t local = 0u;
#pragma unroll
    for (int j = 0; j < kBPT; ++j) {
      h[j] = sh.hist[base + j];
      local += h[j];
    }
#pragma unroll
    for (int j = 0; j < kBPT; ++j) sh.hist[base + j] = 0u;  // for the next pass
    const uint32_t incl = wave_inclusive_sum(local);
    if (lane == kWave - 1) sh.wsum[wave] = incl;
    __syncthreads();
    uint32_t above = incl - local;
#pragma unroll
    for (int w = 0; w < NW; ++w) above += w < wave ? sh.wsum[w] : 0u;
    if (above < remaining && above + local >= remaining) {
      uint32_t c = above;
#pragma unroll
      for (int j = kBPT - 1; j >= 0; --j) {
        if (c < remaining && c + h[j] >= remaining) {
          sh.pick[0] = uint32_t(base + j);
          sh.pick[1] = remaining - c;
          sh.pick[2] = h[j];
        }
        c += h[j];
      }
    }
    __syncthreads();
    prefix |= sh.pick[0] << shift;
    pmask |= dmask << shift;
    remaining = sh.pick[1];
    return sh.pick[2];
  }
};

// Select the K largest of the n keys key(0..n-1) (n_sel of them are nonzero),
// ties to the lowest index, and call emit(p, i, key) for each selected index i
// in ascending order, p = its output slot in [0, min(K, n_sel)).  All NT threads
// of the workgroup call it.
//
// The radix passes run on key - kmin (kmin = the smallest selectable key; an
// order-preserving shift) from the highest bit of kmax - kmin down, in digits of
// at most 11 bits: the first digit then cuts the row's actual key range into
// equal parts (close scores spread over the histogram instead of piling into a
// few bins, also across a power of two), and narrow ranges need fewer passes.
// After the first pass every key
// outside the boundary digit is decided; when that digit holds at most CC
// keys they are gathered (with the wave whose segment they came from) in one
// more pass over the keys, and the rest of the search runs on them alone: by
// counting ranks for at most kRankMax of them, else by radix passes over the
// gathered keys.  The same pass counts, per wave segment, the keys above the
// boundary digit, so that the compaction needs no counting pass of its own.  A
// larger boundary digit (many equal scores) takes the radix passes over all keys.
// The selection as a threshold: the k-th largest key `thr` and how many of the
// keys equal to it (the lowest-indexed ones) are selected; with n_sel <= K,
// thr = 0 and need_eq = 0 (every selectable key).  When `counted`, gt and eq
// are the counts of keys > thr and == thr in this wave's compaction segment.
struct SelectThreshold {
  uint32_t thr = 0u, need_eq = 0u;
  uint32_t gt = 0u, eq = 0u;
  bool counted = false;
};

// Wave w's contiguous segment [s_lo, s_hi) of n keys in the ordered compaction.
template <int NT>
__device__ __forceinline__ void select_segment(int n, int& s_lo, int& s_hi) {
  constexpr int NW = NT / kWave;
  const int seg = ((n + NW - 1) / NW + kWave - 1) & ~(kWave - 1);
  s_lo = int(threadIdx.x / kWave) * seg;
  s_hi = min(n, s_lo + seg);
}

template <int NT, class Keys, int B, int C>
__device__ __forceinline__ SelectThreshold select_search(const Keys& key, int n, uint32_t n_sel,
                                                         int K, SelectShared<NT, B, C>& sh,
                                                         const KeyRange& kr = KeyRange{}) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint64_t lt = lanemask_lt();
  int s_lo, s_hi;
  select_segment<NT>(n, s_lo, s_hi);

  uint32_t thr = 0u, need_eq = 0u;
  uint32_t gt = 0u, eq = 0u;  // this wave's segment: keys > thr, keys == thr
  bool counted = false;
  if (n_sel > uint32_t(K)) {
    if (tid == 0) sh.ccount = 0u;  // ordered by the barriers of init
    RadixSearch<NT, B, C> rs{sh};
    rs.init(key, n, K, kr);
    const uint32_t in_bin = rs.shift > 0 ? rs.pass(key, n) : 0u;
    if (rs.shift > 0 && in_bin <= uint32_t(C)) {
      // gather the boundary digit's keys; count the keys above it per segment
      const uint32_t bin_max = rs.prefix | ~rs.pmask;  // largest d with the boundary digit
      const uint32_t kmin = rs.kmin, pmask = rs.pmask, prefix = rs.prefix;
      for_segment(key, s_lo, s_hi, lane, [&](int i, uint32_t k) {
        const uint32_t d = k - kmin;
        gt += __popcll(__ballot(k != 0u && d > bin_max));
        const bool take = k != 0u && (d & pmask) == prefix;
        const uint64_t b = __ballot(take);
        if (b != 0ull) {
          uint32_t at = 0u;
          if (lane == 0) at = atomicAdd(&sh.ccount, uint32_t(__popcll(b)));
          at = uint32_t(__shfl(int(at), 0)) + uint32_t(__popcll(b & lt));
          if (take) {
            sh.ckey[at] = k;
            sh.cwave[at] = uint8_t(wave);
          }
        }
        (void)i;
      });
      if (tid < 4) sh.ckey[in_bin + tid] = 0u;  // zero keys after the last: never counted
      __syncthreads();
      const int m = int(in_bin);
      if (m <= kRankMax) {
        // the remaining-th largest gathered key, by counting: key c is it when
        // #(keys > c) < remaining <= #(keys >= c)
        if (tid < m) {
          const uint32_t c = sh.ckey[tid];
          uint32_t ngt = 0u, nge = 0u;
          for (int j = 0; j < m; j += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(&sh.ckey[j]);
            ngt += uint32_t(v.x > c) + uint32_t(v.y > c) + uint32_t(v.z > c) + uint32_t(v.w > c);
            nge += uint32_t(v.x >= c) + uint32_t(v.y >= c) + uint32_t(v.z >= c) + uint32_t(v.w >= c);
          }
          if (ngt < rs.remaining && rs.remaining <= nge) {
            sh.pick[0] = c;
            sh.pick[1] = rs.remaining - ngt;
          }
        }
        __syncthreads();
        thr = sh.pick[0];
        need_eq = sh.pick[1];
      } else {
        const LdsKeys cand{sh.ckey};
        while (rs.shift > 0) rs.pass(cand, m);
        thr = rs.kmin + rs.prefix;
        need_eq = rs.remaining;
      }
      // the gathered keys of this wave's segment: > thr and == thr (gt so far is
      // the same in every lane: the keys above the boundary digit)
      uint32_t cgt = 0u, ceq = 0u;
      for (int j = lane; j < m; j += kWave) {
        if (sh.cwave[j] == uint8_t(wave)) {
          cgt += uint32_t(sh.ckey[j] > thr);
          ceq += uint32_t(sh.ckey[j] == thr);
        }
      }
      gt += wave_sum(cgt);
      eq = wave_sum(ceq);
      counted = true;
    } else {
      while (rs.shift > 0) rs.pass(key, n);
      thr = rs.kmin + rs.prefix;
      need_eq = rs.remaining;
    }
  }

  SelectThreshold r;
  r.thr = thr;
  r.need_eq = need_eq;
  r.gt = gt;
  r.eq = eq;
  r.counted = counted;
  return r;
}

template <int NT, class Keys, class Emit, int B, int C>
__device__ __forceinline__ void select_topk(const Keys& key, int n, uint32_t n_sel, int K,
                                            SelectShared<NT, B, C>& sh, Emit emit,
                                            const KeyRange& kr = KeyRange{}) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint64_t lt = lanemask_lt();
  int s_lo, s_hi;
  select_segment<NT>(n, s_lo, s_hi);
  const SelectThreshold r = select_search<NT>(key, n, n_sel, K, sh, kr);
  const uint32_t thr = r.thr, need_eq = r.need_eq;
  uint32_t gt = r.gt, eq = r.eq;
  // ordered compaction
  if (!r.counted) {
    for_segment(key, s_lo, s_hi, lane, [&](int i, uint32_t k) {
      gt += __popcll(__ballot(k > thr));
      eq += __popcll(__ballot(i < s_hi && k == thr));
    });
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
  for_segment(key, s_lo, s_hi, lane, [&](int i, uint32_t k) {
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
  });
}

// Chunk length of a window on the split path (multiple of 64), or 0 when the
// row is handled whole by chunk 0 (short windows, and windows too long for 16
// LDS-resident chunks).
__device__ __forceinline__ int split_chunk_len(int n) {
  if (n <= kCap || n > kMaxChunks * kCap) return 0;
  const int c = (n + kMaxChunks - 1) / kMaxChunks;
  return (c + kWave - 1) & ~(kWave - 1);
}

// Candidate workspace of the split path: per (row, chunk) slot up to k keys,
// their columns, and a count.
struct Candidates {
  uint32_t* key;
  int32_t* col;
  int32_t* cnt;
  __host__ __device__ static size_t bytes(int64_t n_q, int32_t K) {
    const size_t slots = size_t(n_q) * kMaxChunks;
    return slots * size_t(K) * (sizeof(uint32_t) + sizeof(int32_t)) + slots * sizeof(int32_t);
  }
  __host__ __device__ static Candidates at(void* ws, int64_t n_q, int32_t K) {
    const size_t slots = size_t(n_q) * kMaxChunks;
    uint32_t* k = static_cast<uint32_t*>(ws);
    int32_t* c = reinterpret_cast<int32_t*>(k + slots * K);
    return Candidates{k, c, c + slots * K};
  }
};

}  // namespace topksel
}  // namespace dsa
