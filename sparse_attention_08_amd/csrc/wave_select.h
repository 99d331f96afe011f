// Exact top-k over one row's candidates held in LDS by ONE wave (gfx950,
// wave64), with no workgroup barrier: the running candidate set of the fused
// prefill indexer + top-k, where every wave owns one query row.
//
// Candidates are order-preserving u32 keys (score_key: larger score, larger
// key; 0 = not selectable, never held) with their columns, kept in column
// order.  The rule is the top-k rule of the library: the k largest keys, ties
// to the lowest column, output in ascending column order, then -1.
//
// Every pass reads the held keys in blocks of 256, four consecutive keys per
// lane (one 16-byte LDS read), so that a pass costs n / 256 short steps instead
// of n / 64 dependent LDS round trips.  Order-dependent steps (the compaction)
// rank a lane's four keys after all keys of the lanes below it: a wave prefix
// sum of the per-lane counts plus the count among the lane's earlier keys.
//
// LDS ordering: the LDS executes one wave's DS instructions in issue order, so
// a lane's read after another lane's write of the same wave sees the write; the
// wavefront-scope fences below only keep the compiler from reordering them.
#pragma once

#include "dsa_device.h"

namespace dsa {
namespace wsel {

constexpr int kBins = 256;   // 8-bit radix digits; one histogram per wave
constexpr int kBlock = 256;  // keys per step: 4 per lane

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v = min(v, uint32_t(__shfl_xor(int(v), o)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), o)));
  return v;
}

// The four keys of this lane in block `base` (0 past n: never counted).
__device__ __forceinline__ void load4(const uint32_t* keys, int n, int base, int lane,
                                      uint32_t (&x)[4]) {
  const uint4 v = *reinterpret_cast<const uint4*>(keys + base + 4 * lane);
  const int i = base + 4 * lane;
  x[0] = i < n ? v.x : 0u;
  x[1] = i + 1 < n ? v.y : 0u;
  x[2] = i + 2 < n ? v.z : 0u;
  x[3] = i + 3 < n ? v.w : 0u;
}

// The k-th largest key and how many of the keys equal to it (the lowest-column
// ones) are selected, when n > k: the selection is {key > thr} plus the first
// need_eq keys == thr in column order.
struct Threshold {
  uint32_t thr;
  uint32_t need_eq;
};

// A radix search over d = key - kmin (kmin = the smallest held key) from the
// highest bit in which the held keys differ, 8 bits per pass.
struct Radix {
  uint32_t kmin = 0u;
  int shift = 0;         // d's bits below the digits picked so far
  uint32_t prefix = 0u;  // the digits picked so far (bits under pmask)
  uint32_t pmask = 0u;
  uint32_t remaining = 0u;  // rank of the k-th key among the keys with that prefix
  uint32_t in_bin = 0u;     // keys with that prefix

  __device__ __forceinline__ void init(const uint32_t* keys, int n, int k, int lane) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int base = 0; base < n; base += kBlock) {
      uint32_t x[4];
      load4(keys, n, base, lane, x);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (x[j] != 0u) lo = min(lo, x[j]);
        hi = max(hi, x[j]);
      }
    }
    kmin = wave_min_u32(lo);
    const uint32_t range = wave_max_u32(hi) - kmin;
    shift = range == 0u ? 0 : 32 - __builtin_clz(range);
    prefix = 0u;
    pmask = 0u;
    remaining = uint32_t(k);
    in_bin = uint32_t(n);
  }

  // One 8-bit digit: histogram of the keys with the current prefix, then the
  // bin that holds the remaining-th largest.
  __device__ __forceinline__ void pass(const uint32_t* keys, int n, uint32_t* hist, int lane) {
    const int nb = shift < 8 ? shift : 8;
    shift -= nb;
    const uint32_t dmask = (1u << nb) - 1u;
    *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    wave_fence();
    const uint32_t km = kmin, pm = pmask, pf = prefix;
    const int sh = shift;
    for (int base = 0; base < n; base += kBlock) {
      uint32_t x[4];
      load4(keys, n, base, lane, x);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t d = x[j] - km;
        if (x[j] != 0u && (d & pm) == pf) atomicAdd(&hist[(d >> sh) & dmask], 1u);
      }
    }
    wave_fence();
    // lane l owns bins 255-4l .. 252-4l (descending): an exclusive prefix over
    // lanes counts the keys in higher bins
    const uint4 h4 = *reinterpret_cast<const uint4*>(hist + kBins - 4 - 4 * lane);
    const uint32_t h[4] = {h4.w, h4.z, h4.y, h4.x};  // bins 255-4l, 254-4l, 253-4l, 252-4l
    const uint32_t local = h[0] + h[1] + h[2] + h[3];
    const uint32_t incl = wave_inclusive_sum(local);
    const uint32_t above = incl - local;
    uint32_t pick = 0u, rem = 0u, cnt = 0u;
    const bool mine = above < remaining && incl >= remaining;
    if (mine) {
      uint32_t c = above;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c < remaining && c + h[j] >= remaining) {
          pick = uint32_t(kBins - 1 - 4 * lane - j);
          rem = remaining - c;
          cnt = h[j];
        }
        c += h[j];
      }
    }
    const uint64_t who = __ballot(mine);
    const int src = who != 0ull ? __builtin_ctzll(who) : 0;  // one lane: the counts reach `remaining`
    pick = uint32_t(__builtin_amdgcn_readlane(int(pick), src));
    remaining = uint32_t(__builtin_amdgcn_readlane(int(rem), src));
    in_bin = uint32_t(__builtin_amdgcn_readlane(int(cnt), src));
    prefix |= pick << shift;
    pmask |= dmask << shift;
    wave_fence();  // the histogram reads are done before the next pass clears it
  }
};

__device__ __forceinline__ Threshold kth_largest(const uint32_t* keys, int n, int k,
                                                 uint32_t* hist, int lane) {
  Radix r;
  r.init(keys, n, k, lane);
  while (r.shift > 0) r.pass(keys, n, hist, lane);
  return Threshold{r.kmin + r.prefix, r.remaining};
}

// The four columns of this lane in block `base` (read together with its keys).
__device__ __forceinline__ void load4c(const uint16_t* cols, int base, int lane, uint32_t (&c)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(cols + base + 4 * lane);
  c[0] = v.x & 0xFFFFu;
  c[1] = v.x >> 16;
  c[2] = v.y & 0xFFFFu;
  c[3] = v.y >> 16;
}
__device__ __forceinline__ void load4c(const uint32_t* cols, int base, int lane, uint32_t (&c)[4]) {
  const uint4 v = *reinterpret_cast<const uint4*>(cols + base + 4 * lane);
  c[0] = v.x;
  c[1] = v.y;
  c[2] = v.z;
  c[3] = v.w;
}

// Visit the kept candidates of keys[0..n) in column order: those > t.thr and
// the first t.need_eq equal to it.  f(pos, key, col) gets the candidate's key
// and column and its position among the kept ones (ascending with the index).
// Returns the kept count.  A block's keys and columns are all read before any
// of its candidates is visited, and positions never pass indices, so f may
// store candidate i at slot pos in place.
template <class ColT, class F>
__device__ __forceinline__ int for_kept(const uint32_t* keys, const ColT* cols, int n,
                                        Threshold t, int lane, F f) {
  uint32_t gt_before = 0u, eq_before = 0u;
  for (int base = 0; base < n; base += kBlock) {
    uint32_t x[4], c[4];
    load4(keys, n, base, lane, x);
    load4c(cols, base, lane, c);
    uint32_t ngt = 0u, neq = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ngt += uint32_t(x[j] > t.thr);
      neq += uint32_t(x[j] == t.thr && base + 4 * lane + j < n);
    }
    const uint32_t gi = wave_inclusive_sum(ngt | (neq << 16));  // both counts < 2^16
    const uint32_t g_excl = (gi & 0xFFFFu) - ngt, e_excl = (gi >> 16) - neq;
    uint32_t gt_at = gt_before + g_excl, eq_at = eq_before + e_excl;
    wave_fence();  // every read of the block is issued before its first store
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool is_gt = x[j] > t.thr;
      const bool is_eq = x[j] == t.thr && base + 4 * lane + j < n;
      if (is_gt || (is_eq && eq_at < t.need_eq)) f(int(gt_at + min(eq_at, t.need_eq)), x[j], c[j]);
      gt_at += uint32_t(is_gt);
      eq_at += uint32_t(is_eq);
    }
    const uint32_t tot = uint32_t(__builtin_amdgcn_readlane(int(gi), kWave - 1));
    gt_before += tot & 0xFFFFu;
    eq_before += tot >> 16;
  }
  return int(gt_before + min(eq_before, t.need_eq));
}

// Make room in the held candidates (n > k): a shrink keeps at least k of them
// and returns the new floor -- a key arriving later (a higher column) can only
// enter above it.  One radix pass usually does: every key below the digit that
// holds the k-th key goes, and the floor is the top of the digit below (the
// keys kept are the k-th key's digit and everything above it).  When that
// would keep more than `keep_max` (a crowded digit: many close or equal keys),
// the held keys are cut to their exact top k and the floor is the k-th key
// (a later key equal to it has a higher column and loses the tie).
template <class ColT>
__device__ __forceinline__ uint32_t shrink(uint32_t* keys, ColT* cols, int& n, int k,
                                           int keep_max, uint32_t* hist, int lane) {
  Radix r;
  r.init(keys, n, k, lane);
  Threshold t;
  uint32_t floor_key;
  bool cut = false;
  if (r.shift > 0) {
    r.pass(keys, n, hist, lane);
    const uint32_t keep = uint32_t(k) - r.remaining + r.in_bin;  // keys at or above the digit
    if (keep <= uint32_t(keep_max)) {
      floor_key = r.kmin + r.prefix - 1u;  // every key at or below it is below the digit
      t = Threshold{floor_key, 0u};
      cut = true;
    }
  }
  if (!cut) {
    while (r.shift > 0) r.pass(keys, n, hist, lane);
    t = Threshold{r.kmin + r.prefix, r.remaining};
    floor_key = t.thr;
  }
  n = for_kept(keys, cols, n, t, lane, [&](int pos, uint32_t x, uint32_t c) {
    keys[pos] = x;
    cols[pos] = ColT(c);
  });
  wave_fence();
  return floor_key;
}

// The row's result: the top k of the held candidates in ascending column
// order (col_base + the held column), then -1 up to k.
template <class ColT>
__device__ __forceinline__ void emit(const uint32_t* keys, const ColT* cols, int n, int k,
                                     int col_base, int32_t* __restrict__ dst, uint32_t* hist,
                                     int lane) {
  Threshold t{0u, 0u};  // n <= k: every held key (all are > 0)
  if (n > k) t = kth_largest(keys, n, k, hist, lane);
  const int kept = for_kept(keys, cols, n, t, lane, [&](int pos, uint32_t, uint32_t c) {
    dst[pos] = col_base + int(c);
  });
  for (int p = kept + lane; p < k; p += kWave) dst[p] = -1;
}

}  // namespace wsel
}  // namespace dsa
