// Fused lightning indexer + top-k for many query rows (prefill), gfx950.  The
// score matrix never reaches memory: each row's candidates stay in LDS.
//
// KimiK3DSAIndexer.score on the vLLM API page "vllm.models.kimi_k3.nvidia.dsa"
// scores the current rows and writes their top-k into a caller-owned index
// buffer in one op; the selection rule is the fallback top-k of review comment
// 3 of vime pull request #502 (window mask, -1 padding), ties to the lowest
// column, output in ascending column order.
//
// Workgroup = 4 consecutive query rows and 8 waves: per row a scoring wave and
// a selecting wave, which the hardware places on one SIMD, so the selection's
// LDS and VALU work runs beside the matrix-core work of the scoring.
//   * keys: chunks of 32 KB (128 bf16 / 256 fp8 keys) staged in LDS by LDS-DMA
//     (issued by the scoring waves), one chunk ahead, shared by the four rows;
//     one workgroup barrier per chunk;
//   * scoring wave: the row's 32-key tiles in pairs on the matrix core, exactly
//     as the score kernel computes them (same operands, same accumulation
//     order, so the same fp32 scores), into the row's ring of scores in LDS;
//   * selecting wave, one chunk behind: the ring's scores above the row's floor
//     are appended to the row's held candidates (order-preserving keys with
//     their window offsets, in column order); when the next chunk might not
//     fit, the held set is shrunk in place -- to the k-th key's radix digit and
//     above, or to its exact top k -- and the floor rises; at the end the
//     wave selects the row's top k and writes it, ascending, then -1.
// Exact for the same reason as every streamed selection here: a key of the
// row's top k is in the top k of every prefix of the row that contains it.
#include <climits>
#include <type_traits>

#include "dsa_device.h"
#include "dsa_launch.h"
#include "indexer_core.h"
#include "wave_select.h"

namespace dsa {
namespace {

using ixcore::kKeyTile;
using ixcore::OpBf16;
using ixcore::OpFp4;
using ixcore::OpFp8;
using ixcore::PendingTile;
using ixcore::QueryRow;

constexpr int kFRows = 4;  // query rows per workgroup
constexpr int kFThreads = 2 * kFRows * kWave;  // a scoring and a selecting wave per row
constexpr int kFChunkBytes = 32768;
constexpr int kLdsBytes = 160 * 1024;
constexpr int kFMaxK = 2048;

template <class Op>
constexpr int chunk_keys() {
  return kFChunkBytes / Op::kRowBytes < 256 ? kFChunkBytes / Op::kRowBytes : 256;  // 128 bf16, 256 fp8 / fp4
}

// One row's state in LDS: the radix histogram, the ring of scores (the chunk
// being scored and the one being filtered: 2 * 256), then the held keys and
// their offsets from the window start (u16 when every window fits 65536 keys).
constexpr int kStage = 512;
template <class ColT>
struct Held {
  static constexpr int kBytes = (kLdsBytes - 2 * kFChunkBytes - 512) / kFRows;
  static constexpr int kCap =
      ((kBytes - (wsel::kBins + kStage) * 4) / int(sizeof(uint32_t) + sizeof(ColT))) &
      ~(wsel::kBlock - 1);
  uint32_t hist[wsel::kBins];
  float stage[kStage];
  uint32_t keys[kCap];
  ColT cols[kCap];
};
static_assert(sizeof(Held<uint16_t>) * kFRows + 2 * kFChunkBytes + 512 <= kLdsBytes, "LDS");
static_assert(sizeof(Held<uint32_t>) * kFRows + 2 * kFChunkBytes + 512 <= kLdsBytes, "LDS");
static_assert(Held<uint32_t>::kCap >= kFMaxK + 256 + kKeyTile + 1, "a chunk fits after a shrink");

__shared__ __attribute__((aligned(16))) uint8_t g_fb0[kFChunkBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_fb1[kFChunkBytes];

template <int kBuf>
__device__ __forceinline__ uint8_t* fbuf() {
  return kBuf == 0 ? g_fb0 : g_fb1;
}

// Append the scores of keys [from, to) of the row (staged in the ring at
// (key - lo) mod kStage) that lie above the floor to the held candidates, in
// column order: four consecutive keys per lane, ranked after the keys of the
// lanes below it (wave prefix sum).
template <class ColT>
__device__ __forceinline__ void append_staged(Held<ColT>& hd, int lo, int from, int to, int a,
                                              int& cnt, uint32_t floor_key, int lane) {
  for (int base = from; base < to; base += 4 * kWave) {
    const int s0 = base + 4 * lane;
    uint32_t key[4];
    uint32_t n = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = s0 + j;
      key[j] = s < to ? score_key(hd.stage[(s - lo) & (kStage - 1)]) : 0u;
      n += uint32_t(key[j] > floor_key);
    }
    const uint32_t incl = wave_inclusive_sum(n);
    int pos = cnt + int(incl - n);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (key[j] > floor_key) {
        hd.keys[pos] = key[j];
        hd.cols[pos] = ColT(s0 + j - a);
        ++pos;
      }
    }
    cnt += __builtin_amdgcn_readlane(int(incl), kWave - 1);
  }
}

// The selecting wave's step: filter the scores of keys [from, to) (all scored
// by now) into the held candidates, shrinking them first if they might not
// fit.  At most kChunkMax + 32 keys arrive per step.
template <class ColT>
__device__ __forceinline__ void select_step(Held<ColT>& hd, int lo, int from, int to, int a,
                                            int b, int& cnt, uint32_t& floor_key, int K,
                                            int lane) {
  from = max(from, a);  // a tile's keys outside the window are never candidates
  to = min(to, b);
  if (from >= to) return;
  constexpr int kRoom = Held<ColT>::kCap - 256 - kKeyTile;
  if (cnt > kRoom) {
    // a one-pass cut may keep up to halfway between k and the room; more (a
    // crowded digit) and the held set is cut to its exact top k
    floor_key = wsel::shrink(hd.keys, hd.cols, cnt, K, K + (kRoom - K) / 2, hd.hist, lane);
  }
  append_staged(hd, lo, from, to, a, cnt, floor_key, lane);
  wsel::wave_fence();
}

template <class Op, int MT, class ColT>
__global__ __launch_bounds__(kFThreads) void indexer_topk_rows_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int64_t n_q,
    int n_k, int H, int K, int32_t* __restrict__ out) {
  constexpr int CK = chunk_keys<Op>();
  static_assert(2 * CK <= kStage, "the ring holds the chunk scored and the one filtered");
  __shared__ int win[2 * kFRows];
  __shared__ int span[2];
  __shared__ int scored[kFRows];  // per row: every key before it is in the ring
  __shared__ bool trivial[kFRows];  // per row: its top-k is its whole window
  __shared__ __attribute__((aligned(16))) Held<ColT> held[kFRows];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool scorer = wave < kFRows;
  const int row = scorer ? wave : wave - kFRows;
  const int64_t nrb = (n_q + kFRows - 1) / kFRows;
  const int64_t t0 = (nrb - 1 - int64_t(blockIdx.x)) * kFRows;  // latest rows first

  if (tid < kFRows) {
    const int64_t t = t0 + tid;
    int a = 0, b = 0;
    if (t < n_q) {
      a = max(row_starts[t], 0);  // windows are clamped to the keys [0, n_k)
      b = min(row_ends[t], n_k);
      if (b < a) b = a;
    }
    win[tid] = a;
    win[kFRows + tid] = b;
    scored[tid] = a;
  }
  __syncthreads();
  // rows of at most k keys and no negative weight are their whole windows
  // (row_weights_nonneg); a workgroup whose rows all are returns before any load
  if (tid < kFRows * kWave) {
    const int r = tid / kWave;
    const int64_t t = t0 + r;
    const bool whole = t >= n_q || (win[kFRows + r] - win[r] <= K &&
                                    ixcore::row_weights_nonneg(w, t, H, lane));
    if (lane == 0) trivial[r] = whole;
  }
  if (tid == 0) {
    int lo = INT_MAX, hi = INT_MIN;
    for (int i = 0; i < kFRows; ++i)
      if (win[kFRows + i] > win[i]) {
        lo = min(lo, win[i]);
        hi = max(hi, win[kFRows + i]);
      }
    span[0] = lo;
    span[1] = hi;
  }
  __syncthreads();
  static_assert(kFRows == 4, "four rows per workgroup");
  if (trivial[0] && trivial[1] && trivial[2] && trivial[3]) {
    for (int r = 0; r < kFRows; ++r) {
      const int64_t t = t0 + r;
      if (t >= n_q) continue;
      const int a = win[r], n = win[kFRows + r] - a;
      for (int j = tid; j < K; j += kFThreads) out[t * int64_t(K) + j] = j < n ? a + j : -1;
    }
    return;
  }
  const int lo = __builtin_amdgcn_readfirstlane(span[0]);
  const int hi = __builtin_amdgcn_readfirstlane(span[1]);
  const int nchunks = hi > lo ? (hi - lo + CK - 1) / CK : 0;
  const int64_t t = t0 + row;
  const int a = win[row], b = win[kFRows + row];
  const bool active = b > a;
  Held<ColT>& hd = held[row];

  if (scorer) {
    const ixcore::ChunkDma<Op, kFRows, CK> dma(wave, lane);
    if (nchunks > 0) dma.issue(fbuf<0>(), k, lo, n_k, wave, lane);
    QueryRow<Op, MT> qr;
    if (active) qr.load(q, w, t, H, lane);
    PendingTile<Op, MT> pd;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) pd.acc[mt] = f32x16_t{};
    // lanes l and l + 32 both hold key s0 + l % 32 and store the same value to
    // the same slot
    auto put = [&](int s0, float p) {
      hd.stage[(s0 - lo + (lane & 31)) & (kStage - 1)] = p;
    };
    auto chunk = [&](int c, auto cur, auto nn) {
      constexpr int kCur = decltype(cur)::value, kNn = decltype(nn)::value;
      const int key0 = lo + c * CK;
      typename Op::kscale_t ksc[CK / kKeyTile];
      ixcore::chunk_key_scales<Op, CK>(k_scale, key0, hi, lane, ksc);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA pieces of chunk c landed
      __syncthreads();                // ... everyone's; chunk c-1 and its ring slots are free
      if (c + 1 < nchunks) dma.issue(fbuf<kNn>(), k, key0 + CK, n_k, wave, lane);
      if (!active || key0 >= b || key0 + CK <= a) return;
      ixcore::chunk_tile_pairs<Op, MT, CK>(fbuf<kCur>(), key0, a, b, qr, lane, ksc, pd, put);
      wsel::wave_fence();
      // every key before the pending tile is in the ring
      if (lane == 0) scored[row] = pd.live ? pd.s0 : min(b, key0 + CK);
    };
    for (int c = 0; c < nchunks; c += 2) {
      chunk(c, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      if (c + 1 >= nchunks) break;
      chunk(c + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
    }
    __syncthreads();  // the selecting wave has filtered everything before the pending tile
    if (pd.live) put(pd.s0, qr.epilogue(pd.acc) * Op::post(pd.ksc));
    wsel::wave_fence();
    if (lane == 0) scored[row] = b;
    __syncthreads();  // the row's last scores are in the ring
    return;
  }

  // selecting wave: one chunk behind the scoring wave of its row
  int cnt = 0;             // held candidates (wave-uniform)
  int done = a;            // keys before it are filtered
  uint32_t floor_key = 0;  // a key enters only above it (0: not selectable)
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();  // chunk c-1's scores are in the ring
    const int upto = __builtin_amdgcn_readfirstlane(scored[row]);
    select_step(hd, lo, done, upto, a, b, cnt, floor_key, K, lane);
    done = max(done, upto);
  }
  __syncthreads();
  {
    const int upto = __builtin_amdgcn_readfirstlane(scored[row]);
    select_step(hd, lo, done, upto, a, b, cnt, floor_key, K, lane);
    done = max(done, upto);
  }
  __syncthreads();
  select_step(hd, lo, done, b, a, b, cnt, floor_key, K, lane);
  if (t < n_q) wsel::emit(hd.keys, hd.cols, cnt, K, a, out + t * int64_t(K), hd.hist, lane);
}

template <class Op, int MT>
hipError_t launch_rows(const void* q, const void* k, const float* k_scale, const float* w,
                       const int32_t* rs, const int32_t* re, int64_t n_q, int64_t n_k, int H,
                       int32_t K, int32_t* out, hipStream_t stream) {
  const int64_t nrb = (n_q + kFRows - 1) / kFRows;
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const uint8_t* kb = static_cast<const uint8_t*>(k);
  if (n_k <= 65536)
    hipLaunchKernelGGL((indexer_topk_rows_kernel<Op, MT, uint16_t>), dim3(unsigned(nrb)),
                       dim3(kFThreads), 0, stream, qb, kb, k_scale, w, rs, re, n_q, int(n_k), H, K,
                       out);
  else
    hipLaunchKernelGGL((indexer_topk_rows_kernel<Op, MT, uint32_t>), dim3(unsigned(nrb)),
                       dim3(kFThreads), 0, stream, qb, kb, k_scale, w, rs, re, n_q, int(n_k), H, K,
                       out);
  return hipGetLastError();
}

}  // namespace

bool indexer_topk_rows_applies(int32_t dtype, int32_t K) {
  return dtype != 0 && K <= kFMaxK;
}

hipError_t launch_indexer_topk_rows(const void* q, const void* k, const float* k_scale,
                                    const float* w, const int32_t* row_starts,
                                    const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                    int32_t n_heads, int32_t dtype, int32_t K, int32_t* out,
                                    hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const bool one = n_heads <= 32;
  if (dtype == 1)
    return one ? launch_rows<OpBf16, 1>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k, n_heads,
                                        K, out, stream)
               : launch_rows<OpBf16, 2>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k, n_heads,
                                        K, out, stream);
  if (dtype == 3)
    return one ? launch_rows<OpFp4, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads,
                                       K, out, stream)
               : launch_rows<OpFp4, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads,
                                       K, out, stream);
  return one ? launch_rows<OpFp8, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, K,
                                     out, stream)
             : launch_rows<OpFp8, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, K,
                                     out, stream);
}

}  // namespace dsa
