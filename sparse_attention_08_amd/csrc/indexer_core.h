// Indexer building blocks shared by the score kernels and the fused indexer +
// top-k kernel (gfx950): operand traits of the bf16 and fp8 matrix-core paths
// and the per-row query state.
//
//   score[t, s] = k_scale[s] * sum_h w[t, h] * max(0, q[t, h, :] . k[s, :])
//
// For one query row the q[t] block [H x 128] is the MFMA A operand (heads on M,
// in MT tiles of 32) and a tile of 32 keys [128 x 32] is the B operand (keys on
// N), so the 32x32 output of v_mfma_f32_32x32x16_bf16 (or
// v_mfma_scale_f32_32x32x64_f8f6f4) holds, in lane l, 16 heads of key column
// l%32.  The ReLU and the weighted head sum happen in those registers; one
// cross-lane add (lane l + lane l^32) finishes the head sum.
#pragma once

#include "dsa_device.h"

namespace dsa {
namespace ixcore {

// Operand traits.  Keys of the fp8 and fp4 paths carry a 4-byte scale per key
// (kscale_t): fp8 one fp32 power of two that multiplies the score (post), fp4
// the four E8M0 bytes of its 32-dim blocks, which the matrix core applies
// itself (kMx: scaled MFMA with a per-lane scale on each operand).
struct OpBf16 {
  typedef bf16x8_t frag_t;
  typedef float kscale_t;
  static constexpr int kRowBytes = 256;  // 128 bf16
  static constexpr int kFragBytes = 16;  // 8 bf16 per lane per K-step of 16
  static constexpr int kSteps = 8;
  static constexpr bool kKeyScale = false, kMx = false;
  __device__ static __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c, int, int) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ kscale_t kscale_one() { return 1.0f; }
  __device__ static __forceinline__ kscale_t load_kscale(const float*, int64_t) { return 1.0f; }
  __device__ static __forceinline__ float post(kscale_t) { return 1.0f; }
};

struct OpFp8 {
  typedef i32x8_t frag_t;
  typedef float kscale_t;
  static constexpr int kRowBytes = 128;  // 128 e4m3
  static constexpr int kFragBytes = 32;  // 32 e4m3 per lane per K-step of 64
  static constexpr int kSteps = 2;
  static constexpr bool kKeyScale = true, kMx = false;
  __device__ static __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c, int, int) {
    // format 0 = e4m3 for both operands; block scales 127 = 2^0 (no scaling)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
  __device__ static __forceinline__ kscale_t kscale_one() { return 1.0f; }
  __device__ static __forceinline__ kscale_t load_kscale(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ float post(kscale_t ks) { return ks; }
};

// MXFP4 (OCP microscaling): 128 packed E2M1 values per row (64 bytes), one E8M0
// scale per 32 dims.  A K-step of the 32x32x64 MFMA gives each lane 32 values
// -- exactly one block -- of its row (lanes 0-31: dims 64 st .. +32, lanes
// 32-63: the next 32), so the block scale is the lane's scale operand.
struct OpFp4 {
  typedef i32x4_t frag_t;  // 32 e2m1 per lane per K-step of 64
  typedef uint32_t kscale_t;
  static constexpr int kRowBytes = 64;
  static constexpr int kFragBytes = 16;
  static constexpr int kSteps = 2;
  static constexpr bool kKeyScale = true, kMx = true;
  __device__ static __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c, int sa,
                                                  int sb) {
    // format 4 = e2m1 for both operands (the instruction reads four registers
    // of each: the upper half of the 8-register operand is not used)
    const i32x8_t a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3);
    const i32x8_t b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
  }
  __device__ static __forceinline__ kscale_t kscale_one() { return 0x7F7F7F7Fu; }  // 2^0 x 4
  __device__ static __forceinline__ kscale_t load_kscale(const float* p, int64_t i) {
    return reinterpret_cast<const uint32_t*>(p)[i];
  }
  __device__ static __forceinline__ float post(kscale_t) { return 1.0f; }
};

constexpr int kKeyTile = 32;

// A window of at most k keys selects every key whose score is not -inf.  With
// no negative head weight no score is: w * ReLU(x) is >= 0 or +inf (NaN, from
// an infinite weight against a zero logit, is not a valid score), and the key
// scales are positive.  True (uniform over the wave) when row t's H weights are
// all >= 0; such a row's top-k is its whole window and the fused kernels write
// it without scoring.
__device__ __forceinline__ bool row_weights_nonneg(const float* __restrict__ w, int64_t t, int H,
                                                   int lane) {
  bool ok = true;
  for (int h = lane; h < H; h += kWave) ok = ok && w[t * H + h] >= 0.0f;
  return __ballot(!ok) == 0ull;
}

// q[t] fragments and the matching head weights of one query row, per lane.
// MXFP4 queries: token t's H code rows (64 bytes each) are followed by its H
// scale quads (4 E8M0 bytes each), so a token takes H * 68 bytes.
template <class Op, int MT>
struct QueryRow {
  typename Op::frag_t qa[MT][Op::kSteps];
  float wv[MT][16];
  int qs[Op::kMx ? MT : 1][Op::kSteps];  // MXFP4: the lane's block scale per (tile, step)
  int kshift;                            // MXFP4: bit offset of the lane's key scale in step 0

  __device__ __forceinline__ void load(const uint8_t* __restrict__ q,
                                       const float* __restrict__ w, int64_t t, int H,
                                       int lane) {
    const int half = lane >> 5;
    constexpr int64_t kTok = Op::kMx ? int64_t(Op::kRowBytes + Op::kSteps * 2) : Op::kRowBytes;
    kshift = 8 * half;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 32 + (lane & 31);
      const bool ok = h < H;
      const uint8_t* base = Op::kMx ? q + t * H * kTok + (ok ? h : 0) * Op::kRowBytes +
                                          half * Op::kFragBytes
                                    : q + (t * H + (ok ? h : 0)) * int64_t(Op::kRowBytes) +
                                          half * Op::kFragBytes;
#pragma unroll
      for (int st = 0; st < Op::kSteps; ++st) {
        typename Op::frag_t v = *reinterpret_cast<const typename Op::frag_t*>(
            base + st * 2 * Op::kFragBytes);
        qa[mt][st] = ok ? v : typename Op::frag_t{};
        if constexpr (Op::kMx) {
          const uint8_t* sc = q + t * H * kTok + int64_t(H) * Op::kRowBytes +
                              (ok ? h : 0) * (Op::kSteps * 2) + 2 * st + half;
          qs[mt][st] = ok ? int(*sc) : 127;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hh = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        wv[mt][r] = hh < H ? w[t * H + hh] : 0.0f;
      }
    }
  }

  // Logits of the 32 keys whose fragments are in kb (heads on M, keys on N);
  // ks: the lane's key scale (MXFP4: its four block scales).
  __device__ __forceinline__ void mma(const typename Op::frag_t (&kb)[Op::kSteps],
                                      typename Op::kscale_t ks, f32x16_t (&acc)[MT]) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16_t{};
#pragma unroll
    for (int st = 0; st < Op::kSteps; ++st) {
      int sb = 0;
      if constexpr (Op::kMx) sb = int((uint32_t(ks) >> (kshift + 16 * st)) & 0xFFu);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = Op::mfma(qa[mt][st], kb[st], acc[mt], Op::kMx ? qs[Op::kMx ? mt : 0][st] : 0, sb);
    }
  }

  // ReLU, head weights and the head sum; lanes l and l^32 both end with the
  // score of key l%32.  ReLU is a signed-integer max on the float bits:
  // non-negative floats keep their bits, every negative float (and -0.0) has
  // negative bits and becomes +0.0 -- one v_max_i32 instead of the two VALU ops
  // of an IEEE fmaxf.
  __device__ __forceinline__ float epilogue(const f32x16_t (&acc)[MT]) const {
    float p = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p = fmaf(wv[mt][r], __int_as_float(max(__float_as_int(acc[mt][r]), 0)), p);
    // v_permlane32_swap: lanes 0-31 and 32-63 exchange this value
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p),
                                                     false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }

  // The tile's scores: epilogue times the key's post scale (fp8).
  __device__ __forceinline__ float score(const typename Op::frag_t (&kb)[Op::kSteps],
                                         typename Op::kscale_t ks) const {
    f32x16_t acc[MT];
    mma(kb, ks, acc);
    return epilogue(acc) * Op::post(ks);
  }
};


// Fragments of the 32-key tile starting at key s0, straight from global memory:
// lane l reads key s0 + l%32.  Lanes past the last key b-1 read key s0 instead
// (their score columns are discarded; a column of the MFMA output depends only
// on that column's key).
template <class Op>
__device__ __forceinline__ void load_key_tile(const uint8_t* __restrict__ k, int s0, int b,
                                              int lane, typename Op::frag_t (&kb)[Op::kSteps]) {
  const int s = s0 + (lane & 31);
  const uint8_t* src = k + int64_t(s < b ? s : s0) * Op::kRowBytes + (lane >> 5) * Op::kFragBytes;
#pragma unroll
  for (int st = 0; st < Op::kSteps; ++st)
    kb[st] = *reinterpret_cast<const typename Op::frag_t*>(src + st * 2 * Op::kFragBytes);
}

// A 32-key tile and the scale of the lane's key.
template <class Op, bool kScaled>
struct KeyTile {
  typename Op::frag_t kb[Op::kSteps];
  typename Op::kscale_t ks = Op::kscale_one();
  __device__ __forceinline__ void load(const uint8_t* __restrict__ k,
                                       const float* __restrict__ k_scale, int s0, int b,
                                       int lane) {
    load_key_tile<Op>(k, s0, b, lane, kb);
    if constexpr (kScaled) {
      const int s = s0 + (lane & 31);
      ks = Op::load_kscale(k_scale, s < b ? s : s0);
    }
  }
};

// Scores of the tiles i = first, first + step, ... < nt of one query row, with
// the next tile's loads in flight while a tile is on the matrix core.  Two
// tiles alternate between two register sets, and every load is issued
// unconditionally (past the last tile the last tile is reloaded and its score
// dropped), so each loop iteration has the same loads in the same order and
// the compiler's memory-counter waits stay exact instead of draining the
// prefetch.  put(i, score) receives each tile's scores, key scale applied
// (lanes l and l^32 both hold key l%32).
template <class Op, int MT, bool kScaled, class Put>
__device__ __forceinline__ void stream_tiles(const QueryRow<Op, MT>& qr,
                                             const uint8_t* __restrict__ k,
                                             const float* __restrict__ k_scale, int base, int b,
                                             int first, int step, int nt, int lane, Put put) {
  if (first >= nt) return;
  auto key0 = [&](int i) { return base + (i < nt ? i : nt - 1) * 32; };
  KeyTile<Op, kScaled> ta, tb;
  ta.load(k, k_scale, key0(first), b, lane);
  tb.load(k, k_scale, key0(first + step), b, lane);
  for (int i = first;; i += 2 * step) {
    const float pa = qr.score(ta.kb, ta.ks);
    ta.load(k, k_scale, key0(i + 2 * step), b, lane);
    put(i, pa);
    if (i + step >= nt) break;
    const float pb = qr.score(tb.kb, tb.ks);
    tb.load(k, k_scale, key0(i + 3 * step), b, lane);
    put(i + step, pb);
    if (i + 2 * step >= nt) break;
  }
}

// ---------------------------------------------------------------------------
// Key tiles staged through wave-private LDS buffers (few long rows: decode).
//
// A direct fragment load gives each lane 16 bytes of a different key, so one
// load instruction touches 32 key rows for 1 KB of data, and the misses the
// memory pipeline can keep in flight run out long before HBM is busy.  Here a
// wave copies each 32-key tile into its own LDS buffer with LDS-DMA loads that
// each move 1 KB of contiguous key rows, NB - 1 tiles ahead of the tile it
// computes, and reads the MFMA fragments from LDS.  The 16-byte pieces of a
// key are XOR-swizzled by the key (kswz) so that the fragment reads are free
// of bank conflicts.  fp8 keys bring their scales along (one 4-byte DMA load).
//
// The DMA is issued through inline asm: the compiler counts a DMA it issues
// itself on its LDS counter as well, and then waits for LDS reads only with a
// full drain.  Its one wait is the explicit vector-memory count below; the
// buffers are private to the wave, so no barrier is needed.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// LDS slot (in 16-byte pieces) of piece cc of tile-local key kl (an involution).
template <class Op>
__device__ __forceinline__ int kswz(int kl, int cc) {
  return Op::kRowBytes == 256   ? (cc ^ (kl & 15))
         : Op::kRowBytes == 128 ? (cc ^ ((kl >> 1) & 7))
                                : (cc ^ ((kl >> 2) & 3));
}

template <class Op, bool kScaled>
struct LdsTile {
  static constexpr int kKeyBytes = kKeyTile * Op::kRowBytes;      // 8 KB bf16, 4 KB fp8
  static constexpr int kBytes = kKeyBytes + (kScaled ? 256 : 0);  // + the scales (twice)
  static constexpr int kKeyLoads = kKeyBytes / 1024;              // 1 KB DMA loads per tile
  static constexpr int kLoads = kKeyLoads + (kScaled ? 1 : 0);

  // DMA of the tile whose first key is s0 into buf (keys past b - 1: key s0)
  __device__ static __forceinline__ void issue(uint8_t* buf, const uint8_t* __restrict__ k,
                                               const float* __restrict__ k_scale, int s0, int b,
                                               int lane) {
    constexpr int kPieces = Op::kRowBytes / 16;
    constexpr int kKeysPerLoad = kWave / kPieces;
    int l = lane;
    asm volatile("" : "+v"(l));  // recomputed here, not held in registers
#pragma unroll
    for (int j = 0; j < kKeyLoads; ++j) {
      const int kl = j * kKeysPerLoad + l / kPieces;
      const int key = s0 + kl < b ? s0 + kl : s0;
      const uint8_t* src = k + int64_t(key) * Op::kRowBytes + kswz<Op>(kl, l % kPieces) * 16;
      asm volatile("global_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "{m0}"(lds_addr(buf + j * 1024))
                   : "memory");
    }
    if constexpr (kScaled) {
      const int key = s0 + (l & 31) < b ? s0 + (l & 31) : s0;
      asm volatile("global_load_lds_dword %0, off"
                   :
                   : "v"(k_scale + key), "{m0}"(lds_addr(buf + kKeyBytes))
                   : "memory");
    }
  }

  // MFMA fragments (and the scale) of the lane's key l % 32
  __device__ static __forceinline__ void read(const uint8_t* buf, int lane,
                                              typename Op::frag_t (&kb)[Op::kSteps],
                                              typename Op::kscale_t& ks) {
    const int kl = lane & 31;
    const uint8_t* row = buf + kl * Op::kRowBytes;
    constexpr int kFragPieces = Op::kFragBytes / 16;
#pragma unroll
    for (int st = 0; st < Op::kSteps; ++st) {
      const int cc = (2 * st + (lane >> 5)) * kFragPieces;
      if constexpr (kFragPieces == 1) {
        kb[st] = *reinterpret_cast<const typename Op::frag_t*>(row + kswz<Op>(kl, cc) * 16);
      } else {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(row + kswz<Op>(kl, cc) * 16);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(row + kswz<Op>(kl, cc + 1) * 16);
        kb[st] = __builtin_bit_cast(typename Op::frag_t,
                                    __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    if constexpr (kScaled)
      ks = reinterpret_cast<const typename Op::kscale_t*>(buf + kKeyBytes)[kl];
  }
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Scores of the tiles i = first, first + step, ... < nt of one query row through
// the wave's NB buffers of LdsTile<Op, kScaled>::kBytes at wbuf.  Tile j of the
// wave's sequence goes to buffer j % NB; the DMA into a buffer is issued after
// the MFMAs of the tile it held, so its reads are done.  Past the last tile the
// last tile is fetched again (every iteration issues the same loads, so the wait
// count is fixed), and everything is drained before return.  put(i, score)
// receives each tile's scores, key scale applied (lanes l and l^32 both hold
// key l%32).
template <class Op, int MT, bool kScaled, int NB, class Put>
__device__ __forceinline__ void stream_tiles_lds(const QueryRow<Op, MT>& qr,
                                                 const uint8_t* __restrict__ k,
                                                 const float* __restrict__ k_scale, int base,
                                                 int b, int first, int step, int nt, int lane,
                                                 uint8_t* wbuf, Put put) {
  typedef LdsTile<Op, kScaled> T;
  if (first >= nt) return;
  auto key0 = [&](int i) { return base + (i < nt ? i : nt - 1) * kKeyTile; };
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) T::issue(wbuf + j * T::kBytes, k, k_scale, key0(first + j * step), b, lane);
  int cur = 0;  // buffer of the tile computed next
  for (int i = first; i < nt; i += step) {
    const int nxt = cur == 0 ? NB - 1 : cur - 1;  // (cur + NB - 1) % NB: free since last iteration
    T::issue(wbuf + nxt * T::kBytes, k, k_scale, key0(i + (NB - 1) * step), b, lane);
    wait_vmcnt<(NB - 1) * T::kLoads>();
    typename Op::frag_t kb[Op::kSteps];
    typename Op::kscale_t ks = Op::kscale_one();
    T::read(wbuf + cur * T::kBytes, lane, kb, ks);
    put(i, qr.score(kb, ks));
    cur = cur + 1 == NB ? 0 : cur + 1;
  }
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Key chunks shared by the waves of a workgroup (prefill: several query rows
// read the same keys).  A chunk of CK keys is staged in LDS by LDS-DMA, every
// wave issuing its share of the 1 KB loads, one chunk ahead of the chunk the
// waves compute on; one workgroup barrier per chunk.  LDS rows are unpadded;
// 16-byte pieces are XOR-swizzled by the key (kswz) so that the fragment reads
// are conflict-free.
// ---------------------------------------------------------------------------

// Chunk DMA.  Wave w issues the 1 KB loads j = w, w + NW, ...; load j covers
// the kKeysPerLoad keys from j * kKeysPerLoad, and lane l moves piece
// l % kPieces of key l / kPieces into LDS slot j * 64 + l.  The piece's source
// position in the key row (the swizzle) depends on the key only through
// key & 15 (bf16) or (key >> 1) & 7 (fp8), which for every load of a wave is
// the same per lane, so the lane part of the source address is one fixed offset
// and each load only moves a wave-uniform base (global_load_lds with an SGPR
// base).
template <class Op, int NW, int CK>
struct ChunkDma {
  static constexpr int kPieces = Op::kRowBytes / 16;      // per key
  static constexpr int kKeysPerLoad = kWave / kPieces;    // keys per 1 KB wave load
  static constexpr int kLoads = CK / kKeysPerLoad;        // wave loads per chunk
  static_assert(kLoads % NW == 0, "every wave issues the same loads");
  static_assert((kKeysPerLoad * NW) % 16 == 0, "a wave's loads share the swizzle per lane");
  int lane_off;  // byte offset of this lane's piece from the load's first key row

  __device__ __forceinline__ ChunkDma(int wave, int lane) {
    const int kl = wave * kKeysPerLoad + lane / kPieces;  // local key of load j = wave
    lane_off = (lane / kPieces) * Op::kRowBytes + kswz<Op>(kl, lane % kPieces) * 16;
  }

  __device__ __forceinline__ void issue(uint8_t* buf, const uint8_t* __restrict__ k, int key0,
                                        int n_k, int wave, int lane) const {
    if (key0 + CK <= n_k) {
#pragma unroll
      for (int u = 0; u < kLoads / NW; ++u) {
        const int j = wave + NW * u;
        const uint8_t* base = k + (int64_t(key0) + j * kKeysPerLoad) * Op::kRowBytes;
        // asm: a compiler-issued LDS-DMA would turn every later LDS wait into a
        // full drain; the chunk's only wait is the explicit one of the caller
        asm volatile("global_load_lds_dwordx4 %0, %1 offset:0"
                     :
                     : "v"(lane_off), "s"(base), "{m0}"(lds_addr(buf + j * kWave * 16))
                     : "memory");
      }
      return;
    }
    // the last chunk runs past the keys: lanes past the end read the last key
    // (lane laundered so that none of this is hoisted out of the chunk loop)
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int u = 0; u < kLoads / NW; ++u) {
      const int j = wave + NW * u;
      const int kl = j * kKeysPerLoad + lane / kPieces;
      int key = key0 + kl;
      key = key < n_k ? key : n_k - 1;
      const uint8_t* src = k + int64_t(key) * Op::kRowBytes + kswz<Op>(kl, lane % kPieces) * 16;
      asm volatile("global_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "{m0}"(lds_addr(buf + j * kWave * 16))
                   : "memory");
    }
  }
};

// K fragments of one 32-key tile (local keys kt*32 .. +32) from a chunk buffer.
template <class Op>
__device__ __forceinline__ void load_kfrags(const uint8_t* buf, int kt, int lane,
                                            typename Op::frag_t (&kb)[Op::kSteps]) {
  const int kl = kt * kKeyTile + (lane & 31);
  const uint8_t* row = buf + kl * Op::kRowBytes;
  constexpr int kFragPieces = Op::kFragBytes / 16;
#pragma unroll
  for (int st = 0; st < Op::kSteps; ++st) {
    const int cc = (2 * st + (lane >> 5)) * kFragPieces;
    if constexpr (kFragPieces == 1) {
      kb[st] = *reinterpret_cast<const typename Op::frag_t*>(row + kswz<Op>(kl, cc) * 16);
    } else {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(row + kswz<Op>(kl, cc) * 16);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(row + kswz<Op>(kl, cc + 1) * 16);
      kb[st] = __builtin_bit_cast(typename Op::frag_t,
                                  __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
}

// A wave's tiles go through its matrix core in pairs (A, B), with one tile
// pending across pairs: the MFMAs of A run beside the ReLU / weight epilogue of
// the pending tile, the MFMAs of B beside that of A, and B is left pending.  So
// one wave keeps both the matrix core and the VALU busy instead of leaving the
// overlap to the other wave of its SIMD.  The pending logits always sit in the
// same registers between pairs.
template <class Op, int MT>
struct PendingTile {
  f32x16_t acc[MT];
  int s0 = 0;                                        // first key of the tile
  typename Op::kscale_t ksc = Op::kscale_one();      // the lane's key scale
  bool live = false;
};

// Order of one pair half: each MFMA followed by kV VALU operations of the other
// tile's epilogue.  With kDsStep > 0, the kDsStep fragment reads of step st of
// the second tile follow the last MFMA that uses step st of the first (MFMA i
// is step i / MT), so the second tile's fragments can take the first's
// registers.
template <int kMf, int kV, int MT, int kDsStep, int I = 0>
__device__ __forceinline__ void sched_mfma_valu() {
  if constexpr (I < kMf) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);  // kV VALU
    if constexpr (kDsStep > 0 && I % MT == MT - 1)
      __builtin_amdgcn_sched_group_barrier(0x100, kDsStep, 0);  // DS reads
    sched_mfma_valu<kMf, kV, MT, kDsStep, I + 1>();
  }
}

// Per-lane key scales of the CK/32 tiles of a chunk (1 without scales), read
// before the chunk's barrier so that waiting for them never waits for the DMA
// issued after it.
template <class Op, int CK>
__device__ __forceinline__ void chunk_key_scales(const float* __restrict__ k_scale, int key0,
                                                 int hi, int lane,
                                                 typename Op::kscale_t (&ksc)[CK / kKeyTile]) {
#pragma unroll
  for (int kt = 0; kt < CK / kKeyTile; ++kt) {
    const int s = key0 + kt * kKeyTile + (lane & 31);
    ksc[kt] = (Op::kKeyScale && k_scale != nullptr && s < hi) ? Op::load_kscale(k_scale, s)
                                                                : Op::kscale_one();
  }
}

// Scores of one wave's row over the chunk in `buf` (keys key0 .. key0+CK-1),
// tile pairs skipped outside the window [a, b).  put(s0, score) gets each
// finished tile, key scale applied (lanes l and l^32 both hold key s0 + l%32);
// the chunk's last tile is left pending in pd.
template <class Op, int MT, int CK, class Put>
__device__ __forceinline__ void chunk_tile_pairs(const uint8_t* buf, int key0, int a, int b,
                                                 const QueryRow<Op, MT>& qr, int lane,
                                                 const typename Op::kscale_t (&ksc)[CK / kKeyTile],
                                                 PendingTile<Op, MT>& pd, Put put) {
  constexpr int kTiles = CK / kKeyTile;
  constexpr int kMf = Op::kSteps * MT;                     // MFMAs per tile
  constexpr int kDs = Op::kSteps * (Op::kFragBytes / 16);  // fragment reads per tile
  constexpr int kV = (32 * MT + kMf - 1) / kMf;            // epilogue VALU per MFMA
#pragma unroll
  for (int pr = 0; pr < kTiles / 2; ++pr) {
    const int sA = key0 + 2 * pr * kKeyTile;
    if (sA >= b || sA + 2 * kKeyTile <= a) continue;
    typename Op::frag_t kA[Op::kSteps], kB[Op::kSteps];
    load_kfrags<Op>(buf, 2 * pr, lane, kA);
    load_kfrags<Op>(buf, 2 * pr + 1, lane, kB);
    f32x16_t acc1[MT];
    qr.mma(kA, ksc[2 * pr], acc1);
    const float pP = qr.epilogue(pd.acc);
    __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);  // tile A's fragments
    __builtin_amdgcn_sched_group_barrier(0x002, 2 * kV, 0);
    sched_mfma_valu<kMf, kV, MT, kDs / Op::kSteps>();
    if (pd.live) put(pd.s0, pP * Op::post(pd.ksc));
    qr.mma(kB, ksc[2 * pr + 1], pd.acc);
    const float pA = qr.epilogue(acc1);
    sched_mfma_valu<kMf, kV, MT, 0>();
    put(sA, pA * Op::post(ksc[2 * pr]));
    pd.s0 = sA + kKeyTile;
    pd.ksc = ksc[2 * pr + 1];
    pd.live = true;
  }
}

}  // namespace ixcore
}  // namespace dsa
