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
// and 32 consecutive scores leave as one 128-byte line.  The [H x T] logits
// never leave the registers.
//
// Two work layouts:
//   rows kernel (prefill)  8 waves = 8 consecutive query rows share 256-key
//                          chunks staged in LDS by LDS-DMA (XOR-swizzled rows:
//                          conflict-free b128 fragment reads); q and w of a row
//                          stay in registers for the whole key loop; each wave
//                          overlaps its tiles' MFMAs with its own epilogue (tile
//                          pairs with one tile pending); row blocks are issued
//                          latest-first so the longest causal rows start first.
//   rowsplit kernel (decode) one long row per workgroup slice: each wave streams
//                          its own 32-key tiles through private LDS buffers with
//                          contiguous 1 KB LDS-DMA loads (the keys are read once,
//                          so there is nothing to share).
// The fp32 path (small head dims) is a plain VALU kernel.
#include <climits>

#include "dsa_device.h"
#include "dsa_launch.h"
#include "indexer_core.h"

namespace dsa {
namespace {

using ixcore::OpBf16;
using ixcore::OpFp4;
using ixcore::OpFp8;
using ixcore::PendingTile;
using ixcore::QueryRow;
using ixcore::kKeyTile;

// ---------------------------------------------------------------------------
// prefill: 8 query rows per workgroup (one per wave), keys staged through LDS in
// chunks of 256 by LDS-DMA one chunk ahead (two buffers, one workgroup barrier
// per 8 tiles).  LDS rows are unpadded; 16-byte pieces are XOR-swizzled by the
// key so that the fragment reads are conflict-free.
// ---------------------------------------------------------------------------
constexpr int kRowsPerBlock = 8;
constexpr int kRowsThreads = kRowsPerBlock * kWave;
constexpr int kChunkKeys = 256;
constexpr int kChunkTiles = kChunkKeys / kKeyTile;
template <class Op>
using RowsDma = ixcore::ChunkDma<Op, kRowsPerBlock, kChunkKeys>;

// Two chunk buffers as separate LDS objects, so that the compiler can tell the
// in-flight LDS-DMA target apart from the buffer being read (it then inserts no
// wait for the DMA before those reads).
constexpr int kChunkBytesMax = kChunkKeys * 256;
__shared__ __attribute__((aligned(16))) uint8_t g_kb0[kChunkBytesMax];
__shared__ __attribute__((aligned(16))) uint8_t g_kb1[kChunkBytesMax];

template <int kBuf>
__device__ __forceinline__ uint8_t* kbuf() {
  return kBuf == 0 ? g_kb0 : g_kb1;
}

// The scores of the 32 keys s0 .. s0+31 (lanes l and l + 32 both hold key
// s0 + l % 32) into a row through a buffer resource whose size ends at the
// window end b, so keys past b are dropped by the hardware's range check;
// keys before a get an offset past any size.  Both lane halves store the same
// values to the same addresses.
__device__ __forceinline__ void store_scores(__amdgpu_buffer_rsrc_t row, int a, int s0, int lane,
                                             float p) {
  const int s = s0 + (lane & 31);
  const unsigned off = s >= a ? unsigned(s) * 4u : 0xFFFFFFF0u;
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p), row, off, 0, 0);
}

// Scores of one wave's row over chunk c (keys key0 .. key0+255), which sits in
// buffer kCur; the DMA of chunk c+1 goes to the other buffer kNn.
template <class Op, int MT, int kCur, int kNn>
__device__ __forceinline__ void rows_chunk(int c, int nchunks, int key0, int hi, int n_k,
                                           const uint8_t* __restrict__ k,
                                           const float* __restrict__ k_scale,
                                           const QueryRow<Op, MT>& qr, bool active, int a, int b,
                                           __amdgpu_buffer_rsrc_t srow, int wave, int lane,
                                           const RowsDma<Op>& dma, PendingTile<Op, MT>& pd) {
  typename Op::kscale_t ksc[kChunkTiles];
  ixcore::chunk_key_scales<Op, kChunkKeys>(k_scale, key0, hi, lane, ksc);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA pieces of chunk c landed
  __syncthreads();                // ... everyone's; all waves are done with chunk c-1
  if (c + 1 < nchunks) dma.issue(kbuf<kNn>(), k, key0 + kChunkKeys, n_k, wave, lane);
  if (!active || key0 >= b || key0 + kChunkKeys <= a) return;
  auto put = [&](int s0, float p) { store_scores(srow, a, s0, lane, p); };
  ixcore::chunk_tile_pairs<Op, MT, kChunkKeys>(kbuf<kCur>(), key0, a, b, qr, lane, ksc, pd, put);
}

template <class Op, int MT>
__global__ __launch_bounds__(kRowsThreads) void indexer_rows_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends,
    int64_t n_q, int n_k, int H, float* __restrict__ scores, int64_t ld) {
  __shared__ int win[2 * kRowsPerBlock];
  __shared__ int span[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t nrb = (n_q + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t t0 = (nrb - 1 - int64_t(blockIdx.x)) * kRowsPerBlock;  // latest rows first

  if (tid < kRowsPerBlock) {
    const int64_t t = t0 + tid;
    int a = 0, b = 0;
    if (t < n_q) {
      // windows are clamped to the keys [0, n_k)
      a = max(row_starts[t], 0);
      b = min(row_ends[t], n_k);
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
  const int lo = __builtin_amdgcn_readfirstlane(span[0]);
  const int hi = __builtin_amdgcn_readfirstlane(span[1]);
  if (hi <= lo) return;
  const int nchunks = (hi - lo + kChunkKeys - 1) / kChunkKeys;
  const RowsDma<Op> dma(wave, lane);
  dma.issue(kbuf<0>(), k, lo, n_k, wave, lane);

  const int64_t t = t0 + wave;
  const int a = win[wave], b = win[kRowsPerBlock + wave];
  const bool active = b > a;
  QueryRow<Op, MT> qr;
  if (active) qr.load(q, w, t, H, lane);
  // row t's scores, sized to end at its window end (empty for an idle wave)
  const __amdgpu_buffer_rsrc_t srow = __builtin_amdgcn_make_buffer_rsrc(
      scores + t * ld, 0, active ? b * 4 : 0, 0x00020000);
  PendingTile<Op, MT> pd;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) pd.acc[mt] = f32x16_t{};

  for (int c = 0; c < nchunks; c += 2) {
    rows_chunk<Op, MT, 0, 1>(c, nchunks, lo + c * kChunkKeys, hi, n_k, k, k_scale, qr, active,
                             a, b, srow, wave, lane, dma, pd);
    if (c + 1 >= nchunks) break;
    rows_chunk<Op, MT, 1, 0>(c + 1, nchunks, lo + (c + 1) * kChunkKeys, hi, n_k, k, k_scale, qr,
                             active, a, b, srow, wave, lane, dma, pd);
  }
  if (pd.live) store_scores(srow, a, pd.s0, lane, qr.epilogue(pd.acc) * Op::post(pd.ksc));
}

// ---------------------------------------------------------------------------
// decode: one long row split over workgroups; each wave streams its own tiles
// through its own LDS buffers
// ---------------------------------------------------------------------------
constexpr int kSplitThreads = 256;
constexpr int kSplitBufs = 2;  // LDS tile buffers per wave: one tile in flight

template <class Op, int MT>
__global__ __launch_bounds__(kSplitThreads) void indexer_rowsplit_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int H,
    int n_k, float* __restrict__ scores, int64_t ld, int nsplit) {
  constexpr int kWaves = kSplitThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t = blockIdx.x;
  const int a = max(row_starts[t], 0), b = min(row_ends[t], n_k);  // clamped to the keys
  if (b <= a) return;
  const int ntiles = (b - a + kKeyTile - 1) / kKeyTile;
  const int i0 = int(int64_t(ntiles) * blockIdx.y / nsplit);
  const int i1 = int(int64_t(ntiles) * (blockIdx.y + 1) / nsplit);
  if (i0 + wave >= i1) return;

  QueryRow<Op, MT> qr;
  qr.load(q, w, t, H, lane);
  constexpr bool kScaled = Op::kKeyScale;  // fp8 / fp4 keys carry a scale
  auto put = [&](int i, float p) {
    const int s = a + i * kKeyTile + (lane & 31);
    if (lane < 32 && s < b && i < i1) scores[t * ld + s] = p;
  };
  typedef ixcore::LdsTile<Op, kScaled> T;
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[kWaves][kSplitBufs * T::kBytes];
  ixcore::stream_tiles_lds<Op, MT, kScaled, kSplitBufs>(qr, k, k_scale, a, b, i0 + wave, kWaves,
                                                        i1, lane, tbuf[wave], put);
}

// ---------------------------------------------------------------------------
// fp32 inputs: plain VALU kernel, one thread per (row, key)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void indexer_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ row_ends, int H,
    int D, int n_k, float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sm[];  // q[t] (H*D) then w[t] (H)
  const int64_t t = blockIdx.x;
  const int a = max(row_starts[t], 0), b = min(row_ends[t], n_k);  // clamped to the keys
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
  // the rows kernel addresses a score row through a buffer resource of b * 4
  // bytes (an int); wider score rows, which no GPU holds for more than a few
  // hundred rows, take the row-split kernel
  constexpr int64_t kRowsMaxKeys = (int64_t(1) << 29) - 1;
  if (n_q <= 256 || n_k > kRowsMaxKeys) {
    // few long rows (decode): split every row's keys over workgroups
    int nsplit = int(2048 / n_q);
    nsplit = nsplit < 1 ? 1 : (nsplit > 128 ? 128 : nsplit);
    const int64_t max_tiles = (n_k + kKeyTile - 1) / kKeyTile;
    const int64_t per_wave = 4 * kSplitThreads / kWave;  // at least 4 tiles per wave
    while (nsplit > 1 && int64_t(nsplit) * per_wave > max_tiles) nsplit >>= 1;
    hipLaunchKernelGGL((indexer_rowsplit_kernel<Op, MT>), dim3(unsigned(n_q), nsplit),
                       dim3(kSplitThreads), 0, stream, qb, kb, k_scale, w, rs, re, H,
                       int(n_k), scores, ld, nsplit);
  } else {
    const int64_t nrb = (n_q + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((indexer_rows_kernel<Op, MT>), dim3(unsigned(nrb)), dim3(kRowsThreads), 0,
                       stream, qb, kb, k_scale, w, rs, re, n_q, int(n_k), H, scores, ld);
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
                       row_starts, row_ends, n_heads, head_dim, int(n_k), scores, ld);
    return hipGetLastError();
  }
  const bool one = n_heads <= 32;
  if (dtype == 1)
    return one ? launch_mfma<OpBf16, 1>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k,
                                        n_heads, scores, ld, stream)
               : launch_mfma<OpBf16, 2>(q, k, nullptr, w, row_starts, row_ends, n_q, n_k,
                                        n_heads, scores, ld, stream);
  if (dtype == 3)
    return one ? launch_mfma<OpFp4, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                       n_heads, scores, ld, stream)
               : launch_mfma<OpFp4, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                       n_heads, scores, ld, stream);
  return one ? launch_mfma<OpFp8, 1>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                     n_heads, scores, ld, stream)
             : launch_mfma<OpFp8, 2>(q, k, k_scale, w, row_starts, row_ends, n_q, n_k,
                                     n_heads, scores, ld, stream);
}

}  // namespace dsa
