// Lightning-indexer scores (gfx950).
//
//   score[t, s] = k_scale[s] * sum_h w[t, h] * max(0, q[t, h, :] . k[s, :])
//
// Matrix-core path (bf16 / fp8 e4m3, head_dim 128).  For one query row the
// q[t] block [H x 128] is the MFMA A operand (heads on M, in MT tiles of 32) and
// a tile of 32 keys [128 x 32] is the B operand (keys on N), so the 32x32 output
// of v_mfma_f32_32x32x16_bf16 (or v_mfma_f32_32x32x64_f8f6f4) holds, in lane l,
// 16 heads of key column l%32.  The ReLU and the weighted head sum happen in
// those registers; one cross-lane add (lane l + lane l^32) finishes the head sum,
// and lanes 0..31 store 32 consecutive scores (one 128-byte line).  The [H x T]
// logits never leave the registers.
//
// Two work layouts:
//   rows kernel (prefill)  8 waves = 8 consecutive query rows share each 32-key
//                          tile staged in LDS (padded rows: conflict-free b128
//                          reads); q and w of a row stay in registers for the
//                          whole key loop; row blocks are issued latest-first so
//                          the longest causal rows start first.
//   rowsplit kernel (decode) one long row per workgroup slice: each wave streams
//                          its own 32-key tiles straight from global memory (the
//                          keys are read once, so there is nothing to share).
// The fp32 path (small head dims) is a plain VALU kernel.
#include <climits>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

struct OpBf16 {
  typedef bf16x8_t frag_t;
  static constexpr int kRowBytes = 256;  // 128 bf16
  static constexpr int kFragBytes = 16;  // 8 bf16 per lane per K-step of 16
  static constexpr int kSteps = 8;
  __device__ static __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct OpFp8 {
  typedef i32x8_t frag_t;
  static constexpr int kRowBytes = 128;  // 128 e4m3
  static constexpr int kFragBytes = 32;  // 32 e4m3 per lane per K-step of 64
  static constexpr int kSteps = 2;
  __device__ static __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c) {
    // format 0 = e4m3 for both operands; block scales 127 = 2^0 (no scaling)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

constexpr int kKeyTile = 32;

// q[t] fragments and the matching head weights of one query row, per lane.
template <class Op, int MT>
struct QueryRow {
  typename Op::frag_t qa[MT][Op::kSteps];
  float wv[MT][16];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ q,
                                       const float* __restrict__ w, int64_t t, int H,
                                       int lane) {
    const int half = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 32 + (lane & 31);
      const bool ok = h < H;
      const uint8_t* base =
          q + (t * H + (ok ? h : 0)) * int64_t(Op::kRowBytes) + half * Op::kFragBytes;
#pragma unroll
      for (int st = 0; st < Op::kSteps; ++st) {
        typename Op::frag_t v = *reinterpret_cast<const typename Op::frag_t*>(
            base + st * 2 * Op::kFragBytes);
        qa[mt][st] = ok ? v : typename Op::frag_t{};
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hh = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        wv[mt][r] = hh < H ? w[t * H + hh] : 0.0f;
      }
    }
  }

  // Scores of the 32 keys whose fragments are in kb; lanes l and l^32 both end
  // with the score of key l%32.
  __device__ __forceinline__ float score(const typename Op::frag_t (&kb)[Op::kSteps]) const {
    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16_t{};
#pragma unroll
    for (int st = 0; st < Op::kSteps; ++st)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = Op::mfma(qa[mt][st], kb[st], acc[mt]);
    float p = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) p = fmaf(wv[mt][r], fmaxf(acc[mt][r], 0.0f), p);
    return p + __shfl_xor(p, 32);
  }
};

// ---------------------------------------------------------------------------
// prefill: 8 query rows per workgroup, key tiles shared through LDS
// ---------------------------------------------------------------------------
constexpr int kRowsPerBlock = 8;
constexpr int kRowsThreads = kRowsPerBlock * kWave;

template <class Op, int MT>
__global__ __launch_bounds__(kRowsThreads) void indexer_rows_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends,
    int64_t n_q, int H, float* __restrict__ scores, int64_t ld, int nsplit) {
  constexpr int kStride = Op::kRowBytes + 16;  // padded LDS row
  constexpr int kChunksPerKey = Op::kRowBytes / 16;
  constexpr int kChunks = kKeyTile * kChunksPerKey;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kKeyTile * kStride];
  __shared__ int win[2 * kRowsPerBlock];
  __shared__ int span[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t nrb = (n_q + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t t0 = (nrb - 1 - int64_t(blockIdx.x)) * kRowsPerBlock;

  if (tid < kRowsPerBlock) {
    const int64_t t = t0 + tid;
    int a = 0, b = 0;
    if (t < n_q) {
      a = row_starts[t];
      b = row_ends[t];
      if (b < a) b = a;
    }
    win[tid] = a;
    win[kRowsPerBlock + tid] = b;
  }
  __syncthreads();
  if (tid == 0) {
    int lo = INT_MAX, hi = INT_MIN;
    for (int i = 0; i < kRowsPerBlock; ++i)
      if (win[kRowsPerBlock + i] > win[i]) {
        lo = min(lo, win[i]);
        hi = max(hi, win[kRowsPerBlock + i]);
      }
    span[0] = lo;
    span[1] = hi;
  }
  __syncthreads();
  const int lo = span[0], hi = span[1];
  if (hi <= lo) return;
  const int ntiles = (hi - lo + kKeyTile - 1) / kKeyTile;
  const int i0 = int(int64_t(ntiles) * blockIdx.y / nsplit);
  const int i1 = int(int64_t(ntiles) * (blockIdx.y + 1) / nsplit);
  if (i0 >= i1) return;

  const int64_t t = t0 + wave;
  const int a = win[wave], b = win[kRowsPerBlock + wave];
  const bool active = b > a;
  QueryRow<Op, MT> qr;
  if (active) qr.load(q, w, t, H, lane);

  const int ck = tid / kChunksPerKey, cc = tid % kChunksPerKey;
  i32x4_t pre = {};
  auto fetch = [&](int i) {
    const int s = lo + i * kKeyTile + ck;
    i32x4_t v = {};
    if (tid < kChunks && s < hi)
      v = *reinterpret_cast<const i32x4_t*>(k + int64_t(s) * Op::kRowBytes + cc * 16);
    pre = v;
  };
  fetch(i0);
  const int half = lane >> 5;
  for (int i = i0; i < i1; ++i) {
    __syncthreads();
    if (tid < kChunks) *reinterpret_cast<i32x4_t*>(tile + ck * kStride + cc * 16) = pre;
    __syncthreads();
    if (i + 1 < i1) fetch(i + 1);
    const int s0 = lo + i * kKeyTile;
    if (active && s0 < b && s0 + kKeyTile > a) {
      typename Op::frag_t kb[Op::kSteps];
      const uint8_t* src = tile + (lane & 31) * kStride + half * Op::kFragBytes;
#pragma unroll
      for (int st = 0; st < Op::kSteps; ++st)
        kb[st] = *reinterpret_cast<const typename Op::frag_t*>(src + st * 2 * Op::kFragBytes);
      float p = qr.score(kb);
      const int s = s0 + lane;
      if (lane < 32 && s >= a && s < b) {
        if (k_scale) p *= k_scale[s];
        scores[t * ld + s] = p;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode: one long row split over workgroups; each wave streams its own tiles
// ---------------------------------------------------------------------------
constexpr int kSplitThreads = 256;

template <class Op, int MT>
__global__ __launch_bounds__(kSplitThreads) void indexer_rowsplit_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int H,
    float* __restrict__ scores, int64_t ld, int nsplit) {
  constexpr int kWaves = kSplitThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t = blockIdx.x;
  const int a = row_starts[t], b = row_ends[t];
  if (b <= a) return;
  const int ntiles = (b - a + kKeyTile - 1) / kKeyTile;
  const int i0 = int(int64_t(ntiles) * blockIdx.y / nsplit);
  const int i1 = int(int64_t(ntiles) * (blockIdx.y + 1) / nsplit);
  if (i0 + wave >= i1) return;

  QueryRow<Op, MT> qr;
  qr.load(q, w, t, H, lane);
  const int half = lane >> 5;
  for (int i = i0 + wave; i < i1; i += kWaves) {
    const int s = a + i * kKeyTile + (lane & 31);
    const bool ok = s < b;
    const uint8_t* src = k + int64_t(ok ? s : a) * Op::kRowBytes + half * Op::kFragBytes;
    typename Op::frag_t kb[Op::kSteps];
#pragma unroll
    for (int st = 0; st < Op::kSteps; ++st) {
      typename Op::frag_t v =
          *reinterpret_cast<const typename Op::frag_t*>(src + st * 2 * Op::kFragBytes);
      kb[st] = ok ? v : typename Op::frag_t{};
    }
    float p = qr.score(kb);
    if (lane < 32 && ok) {
      if (k_scale) p *= k_scale[s];
      scores[t * ld + s] = p;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: plain VALU kernel, one thread per (row, key)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void indexer_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int H,
    int D, float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sm[];  // q[t] (H*D) then w[t] (H)
  const int64_t t = blockIdx.x;
  const int a = row_starts[t], b = row_ends[t];
  const int s = a + int(blockIdx.y) * 256 + int(threadIdx.x);
  if (a + int(blockIdx.y) * 256 >= b) return;
  for (int i = threadIdx.x; i < H * D; i += 256) sm[i] = q[t * H * D + i];
  for (int i = threadIdx.x; i < H; i += 256) sm[H * D + i] = w[t * H + i];
  __syncthreads();
  if (s >= b) return;
  const float* kr = k + int64_t(s) * D;
  float tot = 0.0f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.0f;
    for (int d = 0; d < D; ++d) dot = fmaf(sm[h * D + d], kr[d], dot);
    tot = fmaf(sm[H * D + h], fmaxf(dot, 0.0f), tot);
  }
  scores[t * ld + s] = tot;
}

template <class Op, int MT>
hipError_t launch_mfma(const void* q, const void* k, const float* k_scale, const float* w,
                       const int32_t* rs, const int32_t* re, int64_t n_q, int64_t n_k,
                       int H, float* scores, int64_t ld, hipStream_t stream) {
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const uint8_t* kb = static_cast<const uint8_t*>(k);
  if (n_q <= 256) {
    // few long rows (decode): split every row's keys over workgroups
    int nsplit = int(2048 / n_q);
    nsplit = nsplit < 1 ? 1 : (nsplit > 128 ? 128 : nsplit);
    const int64_t max_tiles = (n_k + kKeyTile - 1) / kKeyTile;
    const int64_t per_wave = 4 * kSplitThreads / kWave;  // at least 4 tiles per wave
    while (nsplit > 1 && int64_t(nsplit) * per_wave > max_tiles) nsplit >>= 1;
    hipLaunchKernelGGL((indexer_rowsplit_kernel<Op, MT>), dim3(unsigned(n_q), nsplit),
                       dim3(kSplitThreads), 0, stream, qb, kb, k_scale, w, rs, re, H,
                       scores, ld, nsplit);
  } else {
    const int64_t nrb = (n_q + kRowsPerBlock - 1) / kRowsPerBlock;
    int nsplit = int((n_k + 2047) / 2048);
    nsplit = nsplit < 1 ? 1 : (nsplit > 8 ? 8 : nsplit);
    hipLaunchKernelGGL((indexer_rows_kernel<Op, MT>), dim3(unsigned(nrb), nsplit),
                       dim3(kRowsThreads), 0, stream, qb, kb, k_scale, w, rs, re, n_q, H,
                       scores, ld, nsplit);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const void* q, const void* k, const float* k_scale,
                                 const float* w, const int32_t* row_starts,
                                 const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                 int32_t n_heads, int32_t head_dim, int32_t dtype,
                                 float* scores, int64_t ld, hipStream_t stream) {
  if (n_q == 0 || n_k == 0) return hipSuccess;
  if (dtype == 0) {
    const unsigned gy = unsigned((n_k + 255) / 256);
    const size_t smem = size_t(n_heads) * (head_dim + 1) * sizeof(float);
    hipLaunchKernelGGL(indexer_f32_kernel, dim3(unsigned(n_q), gy), dim3(256), smem, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k), w,
                       row_starts, row_ends, n_heads, head_dim, scores, ld);
    return hipGetLastError();
  }
  const bool one = n_heads <= 32;
  if (dtype == 1)
    return one ? launch_mfma<OpBf16, 1>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k,
                                        n_heads, scores, ld, stream)
               : launch_mfma<OpBf16, 2>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k,
                                        n_heads, scores, ld, stream);
  return one ? launch_mfma<OpFp8, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                     n_heads, scores, ld, stream)
             : launch_mfma<OpFp8, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                     n_heads, scores, ld, stream);
}

}  // namespace dsa
