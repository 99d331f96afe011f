// Sparse MLA attention over the top-k selected latent rows (gfx950).
//
// Absorbed MLA (vLLM API page "vllm.models.kimi_k3.nvidia.dsa",
// KimiK3DSAAttention: sparse FlashMLA over the indexer's top-k): every head of a
// query reads the same latent row per selected key (512 latent dims followed by
// 64 rope dims, 1152 bytes in bf16); the value is the latent part.  For each
// query t and head h:
//   out[t,h,:] = softmax_j(sm_scale * q[t,h,:] . kv[J_j,:]) @ kv[J, :512]
//   lse[t,h]   = log sum_j exp(sm_scale * q[t,h,:] . kv[J_j,:])
// over J = the entries of topk_idx[t] that are not -1.
//
// bf16 kernel: one workgroup = one query x 128 heads, 4 waves (one per SIMD)
// of 32 heads each; or a slice of the query's selected keys when the key list
// is split (few queries: decode).  A wave keeps its Q^T [576 x 32 heads] in 144
// VGPRs and its O^T [512 x 32 heads] in the 256 accumulation registers for the
// whole query, so no partial result crosses waves.  Per tile of 32 selected
// keys:
//   gather    LDS-DMA (global_load_lds, 16 bytes per lane) of the 32 latent rows
//             into an LDS tile: the 512 latent dims of each key in a 1040-byte
//             slot (slots permuted so that fragment and transposed reads are
//             free of bank conflicts), the 64 rope dims of all keys piece-major
//             after them; four tile buffers, the gather of tile i+2 is issued
//             while tile i is computed;
//   S^T=K.Q^T v_mfma_f32_32x32x16_bf16 with keys on M and the wave's 32 heads on
//             N, 36 K-steps; lane l then holds 16 keys of head l%32;
//   softmax   fp32 in base-2 units (sm_scale * log2 e folded into one multiply)
//             against a fixed per-head reference: the max of the head's first
//             tile with a finite logit.  P = 2^(S - m_ref) <= 2^32 unless a later
//             tile exceeds m_ref + 32, in which case the workgroup runs the
//             query a second time with m_ref = the true max (known by then), so
//             O is never rescaled inside the loop;
//   O += P.V  computed as O^T += V^T . P^T, so that each lane accumulates one
//             head: the probabilities, rounded to bf16 in the order the S^T
//             accumulator holds them (8 keys of one head per lane), are the B
//             operand, and the V fragments (8 keys of one value column per
//             lane, from the same row-major tile through ds_read_b64_tr_b16, a
//             transposing LDS read) are the A operand.
// The P.V of tile i-1 runs while the softmax of tile i is computed (its VALU
// work sits between those MFMAs), and the gather of tile i+2 is issued between
// the MFMAs of S(i).  The row sum adds the bf16-rounded probabilities, so the
// output is an exact convex combination of value rows up to fp32 accumulation.
//
// Split mode writes per-split partials to the workspace -- the normalised output
// in bf16, the lse in fp32 -- and a combine kernel merges them with the
// log-sum-exp weights.
//
// fp8 kernel (the same body over 656-byte fp8 latent rows): each wave gathers
// its 8 rows of a tile into its own staging rows and converts them to the bf16
// tile layout one step ahead of use (three tile buffers).
// The fp32 kernel (small head dims) is plain VALU code.
#include <cfloat>
#include <cmath>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kKT = 32;                         // selected keys per tile
constexpr int kRowBytes = kDqk * 2;             // 1152 bytes = 72 chunks of 16
// LDS tile of 32 latent rows.  Region A holds each key's 512 latent dims (1024
// bytes: the value and the first 512 dims of the key) in 32 slots 1040 bytes
// apart; key j of the tile sits in slot kslot(j), which swaps the two 2-bit
// digits of j % 16.  Slot starts fall 16 bytes apart modulo 256, so
//   * a 16-byte K-fragment read of 16 consecutive keys touches 16 different
//     16-byte bank groups, and
//   * a transposed V read (keys 4g .. 4g+3, 64 bytes of each) touches four
//     disjoint 64-byte bank windows;
// both are free of bank conflicts.  Region B holds the 64 rope dims (128 bytes)
// of every key piece-major: 16-byte piece p of key j at p * 512 + j * 16, so a
// rope fragment read of 16 consecutive keys is 256 contiguous bytes.
constexpr int kRowA = 1040;                     // region A slot stride
__host__ __device__ constexpr int kslot(int j) { return 4 * (j & 3) + ((j >> 2) & 3) + (j & 16); }
constexpr int kRegionA = kKT * kRowA;           // 33280
constexpr bool kslot_is_permutation() {
  uint32_t seen = 0;
  for (int j = 0; j < kKT; ++j) seen |= 1u << kslot(j);
  return seen == 0xFFFFFFFFu;
}
static_assert(kslot_is_permutation(), "slots are a permutation of 0 .. 31");
constexpr int kRegionB = kKT * 128;             // 4096
constexpr int kEpRow = 2 * kDv + 16;            // epilogue staging: bytes per head row
constexpr int kTileBytes = kRegionA + kRegionB;  // 37376
constexpr int kQSteps = kDqk / 16;              // 36 K-steps of 16 dims
constexpr int kVTiles = kDv / 32;               // 16 value tiles of 32 columns
static_assert(32 * kEpRow <= kTileBytes, "a wave's 32 staged output rows fit its tile buffer");
constexpr int kThreads = 256;                   // 4 waves x 32 heads
constexpr int kWaves = kThreads / kWave;
constexpr int kDmaPerWave = kKT / kWaves + 1;  // 8 latent rows + 1 rope load: 9
constexpr int kHeadsPerBlock = kWaves * 32;     // 128
constexpr int kMaxIdx = 2048;                   // selected keys per workgroup (LDS-staged)
constexpr int kMaxTiles = kMaxIdx / kKT;
constexpr float kSpan = 32.0f;                 // base-2 units: P <= 2^32 before a second pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;

// Row (head offset inside the wave's 32) that accumulator register r of a
// 32x32 MFMA output holds in lane half `half`.
__device__ __forceinline__ int acc_row(int r, int half) {
  return 8 * (r >> 2) + 4 * half + (r & 3);
}

struct MlaShared {
  int idx[kMaxIdx];               // this workgroup's slice of the top-k row (-1 -> row 0)
  uint32_t vmask[kMaxTiles + 1];  // per tile: bit j set = selected key j is valid (one
                                  // past the last: read ahead, never used)
  int wlast[kWaves];              // per wave: last valid position of its index loads, or -1
  int redo[2];                    // per pass: some head needs the second pass
};

// Four KV tile buffers, separate LDS objects so that every access names its
// buffer statically: the compiler then knows that reads of one buffer do not
// wait for the LDS-DMA still writing another.  Tile i lives in buffer i % 4;
// while tile i is computed, tile i-1 is still read (P.V) and tiles i+1, i+2
// are in flight.
__shared__ __attribute__((aligned(16))) uint8_t g_kv0[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_kv1[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_kv2[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_kv3[kTileBytes];

template <int B>
__device__ __forceinline__ uint8_t* kvbuf() {
  return B == 0 ? g_kv0 : B == 1 ? g_kv1 : B == 2 ? g_kv2 : g_kv3;
}


// MFMA issued through inline asm, so that each accumulator gets the register
// file it needs: S (16 per lane) in arch VGPRs, O (256 per lane) in the
// accumulation registers.  (With the builtin every MFMA of a kernel takes the
// same form, and S + O do not fit in the 256 accumulation registers.)  The
// compiler does not see into the asm, so the MFMA data hazards it would
// otherwise cover are covered here, with the counts it emits for the builtin on
// gfx950: a VALU write feeding an MFMA operand needs 2 wait states, an MFMA
// result read by a VALU (or accumulation-register move) needs 12, and chained
// accumulation (srcC = previous dst) needs none.
//
// One MFMA per asm statement.  The matrix core runs an MFMA for 32 cycles; the
// wave issues the instructions that follow it meanwhile and waits for the core
// only at the next MFMA, so the LDS reads, gathers and softmax steps are spread
// one small group per MFMA gap (a chained pair in one statement would leave one
// gap per two MFMAs, too short for the work placed there).  Between two asm
// statements the compiler may add a wait state of its own; a chain needs none.
__device__ __forceinline__ void mfma_v0(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// an MFMA whose operands are VALU-written just before (the leading nop)
__device__ __forceinline__ void mfma_v_nop(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// 12 wait states: an MFMA result (arch VGPRs) may be read by the VALU after them
__device__ __forceinline__ void mfma_result_wait(f32x16_t& d) {
  asm volatile("s_nop 7\n\ts_nop 3" : "+v"(d));
}
// accumulation into O.  kNop: the leading wait states cover an operand the
// VALU may have written just before (the first MFMAs of a tile, after P is
// moved into place); the other operands come from LDS reads or from VALU work
// many instructions earlier (a host test scans the compiled code for a VALU
// write closer than two wait states to the MFMA that reads it).
template <bool kNop>
__device__ __forceinline__ void mfma_a(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  if constexpr (kNop)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// before the VALU touches O after MFMAs into it
__device__ __forceinline__ void o_fence(f32x16_t (&o)[kVTiles]) {
  asm volatile("s_nop 7\n\ts_nop 3"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}

// LDS-DMA of local tile lt into buffer B by one wave: the latent rows of keys
// wave, wave+4, ..., wave+28 (one 1 KB load each: the row index is the same for
// the whole wave, so the address is a scalar base plus lane * 16), then rope
// pieces 2*wave and 2*wave+1 of all 32 keys (lane l: key l % 32, piece
// 2*wave + l / 32).  sidx holds the staged rows with -1 replaced by row 0
// (masked later).
//
// The loads are issued through inline asm.  The compiler counts an LDS-DMA it
// issues itself on both the vector-memory and the LDS counters, and with one in
// flight it can only wait for LDS reads with a full drain (lgkmcnt(0)), which
// would empty the fragment rings of both MFMA phases.  The asm loads are
// invisible to its counting: their only wait is the explicit one in wait_tile
// (vector-memory count), and the DMA writes no registers.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_void_ptr)p));
}

// The rows one wave's loads of tile lt need, read from the staged slice ahead
// of the loads: lane l holds the row of key l % 32 (the latent loads take theirs
// with readlane).
struct DmaRows {
  int key;
};
__device__ __forceinline__ DmaRows dma_rows(const int* sidx, int lt, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));  // recomputed here, not held in registers
  return {sidx[lt * kKT + (l & 31)]};
}

template <int B>
__device__ __forceinline__ void dma_latent(const DmaRows& rows, int u,
                                           const uint8_t* __restrict__ kv, int wave, int lane) {
  const int r = wave + kWaves * u;
  const uint32_t row = uint32_t(__builtin_amdgcn_readlane(rows.key, r));
  const uint64_t base = reinterpret_cast<uint64_t>(kv) + uint64_t(row) * kRowBytes;
  const uint32_t vofs = uint32_t(lane) * 16u;
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(vofs), "s"(base), "{m0}"(lds_addr(kvbuf<B>() + kslot(r) * kRowA))
               : "memory");
}

template <int B>
__device__ __forceinline__ void dma_rope(const DmaRows& rows, const uint8_t* __restrict__ kv,
                                         int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));  // recomputed here, not held in registers
  const int piece = 2 * wave + (l >> 5);
  const uint8_t* src = kv + uint64_t(uint32_t(rows.key)) * kRowBytes + 1024 + piece * 16;
  asm volatile("global_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(lds_addr(kvbuf<B>() + kRegionA + wave * 1024))
               : "memory");
}

template <int B>
__device__ __forceinline__ void dma_tile(const int* sidx, int lt, const uint8_t* __restrict__ kv,
                                         int wave, int lane) {
  const DmaRows rows = dma_rows(sidx, lt, lane);
#pragma unroll
  for (int u = 0; u < kKT / kWaves; ++u) dma_latent<B>(rows, u, kv, wave, lane);
  dma_rope<B>(rows, kv, wave, lane);
}

// s_waitcnt lgkmcnt(n), other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// Wait until this wave's LDS-DMA of the current tile has landed.  The next
// tile's 9 loads (issued one tile later, vector-memory counters retire in
// order) may stay in flight.
__device__ __forceinline__ void wait_tile(bool next_in_flight) {
  if (next_in_flight) {
    __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9)
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  static_assert(kDmaPerWave == 9, "vmcnt immediate");
}

// ---------------------------------------------------------------------------
// fp8 latent rows ("fp8_ds_mla", 656 bytes: 512 e4m3 codes, 4 fp32 scales, 64
// bf16 rope values).  Wave w gathers the rows of keys w, w+4, ..., w+28 of a
// tile into its own staging area (8 rows back to back, 41 16-byte pieces each:
// piece p = 64 v + lane of load v is piece p % 41 of row p / 41), and later
// converts the same rows into the bf16 tile layout above.  No other wave
// touches a wave's staging area, so its only synchronisation is the wave's own
// vector-memory count.
constexpr int kRow8 = 656;
constexpr int kPieces8 = kRow8 / 16;                          // 41
constexpr int kRowsPerWave8 = kKT / kWaves;                   // 8
constexpr int kWaveStage8 = kRowsPerWave8 * kRow8;            // 5248
constexpr int kStage8 = kWaves * kWaveStage8;                 // 20992
constexpr int kLoads8 = (kRowsPerWave8 * kPieces8 + kWave - 1) / kWave;  // 6 loads per wave
static_assert(kPieces8 * 16 == kRow8, "rows are whole 16-byte pieces");

__shared__ __attribute__((aligned(16))) uint8_t g_st8a[kStage8];
__shared__ __attribute__((aligned(16))) uint8_t g_st8b[kStage8];

// The rows of this wave's loads of local tile lt, read from the staged slice
// ahead of the loads (and of the fragment reads they are issued between):
// element v is the row of the piece lane l moves in load v.
struct DmaRows8 {
  int row[kLoads8];
};
__device__ __forceinline__ DmaRows8 dma_rows8(const int* sidx, int lt, int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));  // recomputed here, not held in registers
  DmaRows8 d;
#pragma unroll
  for (int v = 0; v < kLoads8; ++v) {
    const int p = min(v * kWave + l, kRowsPerWave8 * kPieces8 - 1);
    d.row[v] = sidx[lt * kKT + wave + kWaves * (p / kPieces8)];
  }
  return d;
}

// load v of this wave's gather into staging buffer `stage` (the last load moves
// the 8 pieces left over: lanes 0..7)
template <int V>
__device__ __forceinline__ void dma_stage8(uint8_t* stage, const DmaRows8& rows,
                                           const uint8_t* __restrict__ kv, int wave, int lane) {
  constexpr int kLast = kRowsPerWave8 * kPieces8 - (kLoads8 - 1) * kWave;  // 8
  int l = lane;
  asm volatile("" : "+v"(l));
  if (V + 1 < kLoads8 || l < kLast) {
    const int p = V * kWave + l;
    const int part = p - (p / kPieces8) * kPieces8;
    const uint8_t* src = kv + uint64_t(uint32_t(rows.row[V])) * kRow8 + part * 16;
    asm volatile("global_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "{m0}"(lds_addr(stage + wave * kWaveStage8 + V * 1024))
                 : "memory");
  }
}

template <int V = 0>
__device__ __forceinline__ void dma_stage8_at(int v, uint8_t* stage, const DmaRows8& rows,
                                              const uint8_t* __restrict__ kv, int wave, int lane) {
  if constexpr (V < kLoads8) {
    if (v == V) dma_stage8<V>(stage, rows, kv, wave, lane);
    else dma_stage8_at<V + 1>(v, stage, rows, kv, wave, lane);
  }
}

__device__ __forceinline__ void dma_tile8(uint8_t* stage, const int* sidx, int lt,
                                          const uint8_t* __restrict__ kv, int wave, int lane) {
  const DmaRows8 rows = dma_rows8(sidx, lt, wave, lane);
#pragma unroll
  for (int v = 0; v < kLoads8; ++v) dma_stage8_at(v, stage, rows, kv, wave, lane);
}

// Wait until this wave's gather of the tile before the last one issued has
// landed (the last one's kLoads8 loads may stay in flight).
__device__ __forceinline__ void wait_stage8(bool next_in_flight) {
  if (next_in_flight) {
    __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  static_assert(kLoads8 == 6, "vmcnt immediate");
}

// This wave's 8 staged rows into tile buffer B.  Latent: row k of the wave
// (key wave + 4 k) is one pass in which lane l converts codes 8 l .. 8 l + 7
// (scale l / 16) into the 16-byte chunk l of the row's bf16 slot, so every read
// and write of the pass covers consecutive bytes.  Rope: one pass, lane
// l = 8 c + k moving rope dims 8 c .. 8 c + 7 of row k.  code * scale is exact
// in bf16 for the power-of-two scales of the cache
// (v_cvt_scalef32_pk_bf16_fp8).
template <int B>
__device__ __forceinline__ void dequant_stage8(const uint8_t* stage, int wave, int lane_in) {
  int lane = lane_in;
  asm volatile("" : "+v"(lane));  // addresses rebuilt here, not held in registers
  const uint8_t* rows = stage + wave * kWaveStage8;
  constexpr int kHalf = kRowsPerWave8 / 2;  // rows read together (register budget)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint2 w[kHalf];
    float sc[kHalf];
#pragma unroll
    for (int j = 0; j < kHalf; ++j) {
      const uint8_t* row = rows + (kHalf * h + j) * kRow8;
      w[j] = *reinterpret_cast<const uint2*>(row + 8 * lane);
      sc[j] = *reinterpret_cast<const float*>(row + 512 + 4 * (lane >> 4));
    }
#pragma unroll
    for (int j = 0; j < kHalf; ++j) {
      const int k = kHalf * h + j;
      const uint32_t y0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j].x, sc[j], false));
      const uint32_t y1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j].x, sc[j], true));
      const uint32_t y2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j].y, sc[j], false));
      const uint32_t y3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j].y, sc[j], true));
      *reinterpret_cast<uint4*>(kvbuf<B>() + kslot(wave + kWaves * k) * kRowA + 16 * lane) =
          make_uint4(y0, y1, y2, y3);
    }
    __builtin_amdgcn_sched_barrier(0);  // one half's registers at a time
  }
  const int rk = lane & 7, rc = lane >> 3;
  const uint4 rope = *reinterpret_cast<const uint4*>(rows + rk * kRow8 + 528 + 16 * rc);
  *reinterpret_cast<uint4*>(kvbuf<B>() + kRegionA + rc * 512 + (wave + kWaves * rk) * 16) = rope;
}

// V fragment m = 2n + ks (value tile n, key step ks) of the tile in buffer B (or
// `buf` when B < 0): the A operand of the V^T . P^T MFMA (8 keys x 1 value column
// per lane), read from the row-major tile with ds_read_b64_tr_b16: in each group of
// 16 lanes, lane 4m'+q reads 4 value columns of key row k0+m' and the transpose
// hands lane i the 4 keys k0..k0+3 of column n0+i.  Lane half h needs keys
// {4h..4h+3} (first read) and {8+4h..8+4h+3} (second read) of each 16-key step:
// the order in which P sits in the S^T accumulator.  Key (li >> 2) + 4 * half
// (+ 8, + 16 per read and step) is in slot 4 * (li >> 2) + half (+ 2, + 16).
template <int B>
__device__ __forceinline__ bf16x8_t vfrag(const uint8_t* buf, int m, int lane) {
  const int half = lane >> 5;
  const int li = lane & 15;
  const int n0 = 16 * ((lane >> 4) & 1);  // value column offset of the group inside a 32-wide tile
  const uint8_t* base = (B >= 0 ? kvbuf<(B < 0 ? 0 : B)>() : buf) +
                        (4 * (li >> 2) + half) * kRowA + (n0 + 4 * (li & 3)) * 2 +
                        16 * (m & 1) * kRowA + (m >> 1) * 64;
  const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base));
  const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + 2 * kRowA));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T = K . Q^T for the tile in buffer B: keys on M, the wave's 32 heads on N,
// 36 K-steps of 16 dims.  Lane l reads key l%32, dims 16*st + 8*(l/32) .. +8;
// the fragment reads run two steps ahead of their MFMA.  With kDma, the
// LDS-DMA loads of a later tile (into buffer BD) are issued between the MFMAs
// (the wave can issue them while the matrix core works).
template <int B, int BD, bool kDma, int BV, bool kF8 = false>
__device__ __forceinline__ f32x16_t qk_tile(bf16x8_t (&fr)[4], const bf16x8_t (&qf)[kQSteps],
                                            uint32_t vmask, int lane, const int* sidx, int lt_dma,
                                            const uint8_t* __restrict__ kv, int wave,
                                            uint8_t* stage = nullptr) {
  const int kk = lane & 31;
  const int h = lane >> 5;
  const uint8_t* ka = kvbuf<B>() + kslot(kk) * kRowA + h * 16;  // latent K-steps 0..31
  int l = lane;
  asm volatile("" : "+v"(l));  // the rope base is rebuilt per tile, not held in registers
  const uint8_t* kr = kvbuf<B>() + kRegionA + (l >> 5) * 512 + (l & 31) * 16;  // K-steps 32..35
  auto frag = [&](int st) {
    return *reinterpret_cast<const bf16x8_t*>(st < 32 ? ka + st * 32 : kr + (st - 32) * 1024);
  };
  DmaRows rows{};
  if constexpr (kDma && !kF8) rows = dma_rows(sidx, lt_dma, lane);  // ahead of the ring reads
  DmaRows8 rows8{};
  if constexpr (kDma && kF8) rows8 = dma_rows8(sidx, lt_dma, wave, lane);
  // fragment reads four steps ahead: one explicit wait per MFMA.  With BV >= 0
  // the last four steps read V fragments 0..3 of buffer BV into the ring for
  // the P.V that follows (two LDS reads each), so that it starts without a wait.
  constexpr int kV = BV >= 0 ? 2 : 0;
#pragma unroll
  for (int st = 0; st < 4; ++st) fr[st] = frag(st);
  f32x16_t s;
#pragma unroll
  for (int st = 0; st < kQSteps; ++st) {
    // the reads of ring fragments st+1 .. st+3 may stay in flight
    if (st + 3 < kQSteps) wait_lgkm<3>();
    else if (st + 2 < kQSteps) wait_lgkm<2 + kV>();
    else if (st + 1 < kQSteps) wait_lgkm<1 + 2 * kV>();
    else wait_lgkm<3 * kV>();
    if (st == 0) mfma_v0(s, fr[0], qf[0]);
    else mfma_v(s, fr[st % 4], qf[st]);
    if (st + 4 < kQSteps) fr[st % 4] = frag(st + 4);
    else if constexpr (BV >= 0) fr[st % 4] = vfrag<BV>(nullptr, st + 4 - kQSteps, lane);
    if constexpr (kDma && kF8) {
      // the gather of a later tile into the wave's staging rows
      if (st % 4 == 1 && st / 4 < kLoads8) dma_stage8_at(st / 4, stage, rows8, kv, wave, lane);
    } else if constexpr (kDma) {
      // the gather of a later tile, spread between the MFMAs
      if (st % 4 == 1 && st / 4 < kKT / kWaves) dma_latent<BD>(rows, st / 4, kv, wave, lane);
      if (st == 33) dma_rope<BD>(rows, kv, wave, lane);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep this order
  }
  // The key mask as one more K-step: dim 0 of the step is -inf for a masked key
  // (lanes 0..31 of the K side) against 1 on the Q side, every other product is
  // 0 * 0, so S = -inf exactly for masked keys and unchanged for the others.
  // Lanes 32..63 carry dims 8..15 of the step: zero on both sides.  Tiles whose
  // 32 keys are all valid (all but the last of a row in practice) skip it.
  if (__builtin_amdgcn_readfirstlane(int(vmask)) != -1) {
    // operands are rebuilt for every tile, not held in registers across the loop
    int l = lane;
    asm volatile("" : "+v"(l));
    int ninf = 0xFF80;
    asm volatile("" : "+v"(ninf));
    const uint64_t keep =
        uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(vmask)))) | 0xFFFFFFFF00000000ull;
    i32x4_t ka = {0, 0, 0, 0};
    // the nop: the lane mask may have just been written by the VALU (readfirstlane)
    asm("s_nop 3\n\tv_cndmask_b32_e64 %0, %1, 0, %2" : "=v"(ka[0]) : "v"(ninf), "s"(keep));
    const i32x4_t qa = {l < 32 ? 0x3F80 : 0, 0, 0, 0};
    mfma_v_nop(s, __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qa));
  }
  // S is complete: the compiler, which does not see the MFMAs, may reuse
  // registers or read S right after this point
  mfma_result_wait(s);
  return s;
}

// Softmax of one tile against a fixed per-head reference m_ref (base-2 units,
// same in both lane halves): P = 2^(S * scale2 - m_ref).  Masked keys already
// hold S = -inf (the bias step of the QK chain), so P = 0 for them.  m_ref is
// the max of the first tile that has a finite logit for the head, so
// P <= 2^kSpan unless a later tile's max exceeds m_ref + kSpan; that sets
// `over` and the query is computed again with m_ref = the true max (m_max
// tracks it).  O is never rescaled inside the loop.
//
// The work is cut into kSmPieces pieces of at most about four VALU operations
// (a transcendental counts as several): the wave runs that much beside an MFMA
// at no cost, and the P.V of the previous tile issues one piece after each of
// its MFMAs from the third on:
//   0 .. 3   max over 4 of the lane's 16 keys each
//   4        max over the lane pair that shares the head, scaled
//   5, 6     reference and running max; overflow flag
//   7 .. 22  P of key register r = piece - 7
//   23 .. 26 bf16 rounding and row sum of key registers 2j, 2j+1, 2j+8, 2j+9
struct Softmax {
  f32x16_t s;      // S^T of the tile: lane = head l%32, 16 keys
  float mt;
  float ps;
  i32x4_t p0w, p1w;  // P of keys 0..7 / 8..15 of the lane half, as packed bf16 pairs
  __device__ __forceinline__ bf16x8_t p0() const { return __builtin_bit_cast(bf16x8_t, p0w); }
  __device__ __forceinline__ bf16x8_t p1() const { return __builtin_bit_cast(bf16x8_t, p1w); }

  // A piece's inputs pass through an empty volatile asm first: the pieces are
  // pure arithmetic, which the instruction selector would otherwise place
  // anywhere (in practice all of it ahead of the P.V MFMAs it is meant to hide
  // behind).
  template <int K>
  __device__ __forceinline__ void piece(float scale2, float& m_ref, float& m_max, bool& over,
                                        float& l_run) {
    if constexpr (K < 4) {
      constexpr int r0 = 4 * K;
      asm volatile("" : "+v"(s[r0]), "+v"(s[r0 + 1]), "+v"(s[r0 + 2]), "+v"(s[r0 + 3]));
      const float m = fmaxf(fmaxf(s[r0], s[r0 + 1]), fmaxf(s[r0 + 2], s[r0 + 3]));
      mt = K == 0 ? m : fmaxf(mt, m);
    } else if constexpr (K == 4) {
      asm volatile("" : "+v"(mt));
      // lanes l and l^32 hold the two key halves of head l%32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale2;
    } else if constexpr (K == 5) {
      asm volatile("" : "+v"(mt));
      // -FLT_MAX = no finite logit yet (an all-masked tile keeps it)
      m_ref = m_ref == -FLT_MAX ? fmaxf(mt, -FLT_MAX) : m_ref;
      m_max = fmaxf(m_max, mt);
    } else if constexpr (K == 6) {
      asm volatile("" : "+v"(mt));
      over = over || mt > m_ref + kSpan;
    } else if constexpr (K < 23) {
      constexpr int r = K - 7;
      asm volatile("" : "+v"(s[r]));
      s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale2, -m_ref));
    } else {
      // P rounded to bf16 (v_cvt_pk_bf16_f32, round to nearest even); the row
      // sum adds the rounded values (v_dot2 with ones), so the output is an
      // exact convex combination of value rows up to fp32 accumulation
      constexpr int r = 2 * (K - 23);
      asm volatile("" : "+v"(s[r]), "+v"(s[r + 1]), "+v"(s[r + 8]), "+v"(s[r + 9]));
      const bf16x2_t ones = {__bf16(1.0f), __bf16(1.0f)};
      const bf16x2_t a = {__bf16(s[r]), __bf16(s[r + 1])};
      const bf16x2_t b = {__bf16(s[r + 8]), __bf16(s[r + 9])};
      float x = K == 23 ? 0.0f : ps;
      x = __builtin_amdgcn_fdot2_f32_bf16(a, ones, x, false);
      x = __builtin_amdgcn_fdot2_f32_bf16(b, ones, x, false);
      p0w[r / 2] = __builtin_bit_cast(int, a);
      p1w[r / 2] = __builtin_bit_cast(int, b);
      if constexpr (K == 26) l_run += x;
      else ps = x;
    }
  }
};
constexpr int kSmPieces = 27;
constexpr int kSmFirstGap = 2;  // the first P.V gaps carry only the reads that start the ring
static_assert(kSmFirstGap + kSmPieces <= 2 * kVTiles, "the softmax pieces fit the P.V gaps");

// piece k of the softmax (k is a constant after unrolling)
template <int K = 0>
__device__ __forceinline__ void sm_piece(int k, Softmax& sm, float scale2, float& m_ref,
                                         float& m_max, bool& over, float& l_run) {
  if constexpr (K < kSmPieces) {
    if (k == K) sm.template piece<K>(scale2, m_ref, m_max, over, l_run);
    else sm_piece<K + 1>(k, sm, scale2, m_ref, m_max, over, l_run);
  }
}

__device__ __forceinline__ void softmax_all(Softmax& sm, float scale2, float& m_ref,
                                            float& m_max, bool& over, float& l_run) {
#pragma unroll
  for (int k = 0; k < kSmPieces; ++k) sm_piece(k, sm, scale2, m_ref, m_max, over, l_run);
}

// O^T += V^T . P^T for the tile in buffer B (B < 0: the buffer `buf` chosen at
// run time).  The V operand comes from vfrag; on entry the ring holds V fragments
// 0..3 (kFill: read them first).  With kSm, one softmax piece of the current
// tile follows each MFMA from gap kSmFirstGap on.
template <int B, bool kSm, bool kFill>
__device__ __forceinline__ void pv_tile(bf16x8_t (&fr)[4], const uint8_t* buf, bf16x8_t p0,
                                        bf16x8_t p1, f32x16_t (&o)[kVTiles], int lane,
                                        Softmax& sm, float scale2, float& m_ref, float& m_max,
                                        bool& over, float& l_run) {
  if constexpr (kFill) {
#pragma unroll
    for (int m = 0; m < 4; ++m) fr[m] = vfrag<B>(buf, m, lane);
  }
#pragma unroll
  for (int m = 0; m < 2 * kVTiles; ++m) {
    // reads of steps m+1 .. m+3 may stay in flight (two per fragment)
    if (m + 3 < 2 * kVTiles) wait_lgkm<6>();
    else if (m + 2 < 2 * kVTiles) wait_lgkm<4>();
    else if (m + 1 < 2 * kVTiles) wait_lgkm<2>();
    else wait_lgkm<0>();
    // O^T += V^T . P^T: the V fragment is the A operand (value column = row)
    // and the P fragment the B operand (head = column), so lane l accumulates
    // head l % 32
    if (m < 2)
      mfma_a<true>(o[m >> 1], fr[m % 4], (m & 1) ? p1 : p0);
    else
      mfma_a<false>(o[m >> 1], fr[m % 4], (m & 1) ? p1 : p0);
    if (m + 4 < 2 * kVTiles) fr[m % 4] = vfrag<B>(buf, m + 4, lane);
    if constexpr (kSm) {
      if (m >= kSmFirstGap && m - kSmFirstGap < kSmPieces)
        sm_piece(m - kSmFirstGap, sm, scale2, m_ref, m_max, over, l_run);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep this order
  }
}

// One tile step i (buffer B = i % 4): wait for tile i, S(i) = K(i).Q^T with
// the gather of tile i+2 issued between its MFMAs, then O += P(i-1).V(i-1) with
// the softmax of S(i) issued between those MFMAs.
template <int B>
__device__ __forceinline__ void tile_step(MlaShared& sh, int i, int nt, const uint8_t* kvb,
                                          const bf16x8_t (&qf)[kQSteps], f32x16_t (&o)[kVTiles],
                                          bf16x8_t& p0, bf16x8_t& p1, uint32_t& vm,
                                          float& m_ref, float& m_max, bool& over, float& l_run,
                                          float scale2, int wave, int lane) {
  wait_tile(i + 1 < nt);
  __builtin_amdgcn_s_barrier();
  Softmax sm;
  bf16x8_t fr[4];  // the fragment ring, shared by the QK and the P.V that follows
  if (i + 2 < nt) {
    sm.s = qk_tile<B, (B + 2) & 3, true, (B + 3) & 3>(fr, qf, vm, lane, sh.idx, i + 2, kvb, wave);
  } else {
    sm.s = qk_tile<B, 0, false, (B + 3) & 3>(fr, qf, vm, lane, sh.idx, 0, kvb, wave);
  }
  pv_tile<(B + 3) & 3, true, false>(fr, nullptr, p0, p1, o, lane, sm, scale2, m_ref, m_max, over,
                                    l_run);
  p0 = sm.p0();
  p1 = sm.p1();
  vm = sh.vmask[i + 1];  // the next tile's mask, read well before it is needed
}

// One tile step i over fp8 rows (tile buffer B = i % 3, staging buffer i % 2):
// S(i) = K(i).Q^T with the gather of tile i+2 into the staging buffer tile i
// left, O += P(i-1).V(i-1) with the softmax of S(i), then the wave's rows of
// tile i+1 (staged one step earlier) into tile buffer (i+1) % 3, free since
// every wave passed this step's barrier after its P.V of tile i-2.
template <int B>
__device__ __forceinline__ void tile_step8(MlaShared& sh, int i, int nt, const uint8_t* kvb,
                                           const bf16x8_t (&qf)[kQSteps], f32x16_t (&o)[kVTiles],
                                           bf16x8_t& p0, bf16x8_t& p1, uint32_t& vm,
                                           float& m_ref, float& m_max, bool& over, float& l_run,
                                           float scale2, int wave, int lane) {
  wait_lgkm<0>();  // this wave's conversion writes have landed
  __builtin_amdgcn_s_barrier();  // tile i converted by every wave
  Softmax sm;
  bf16x8_t fr[4];
  if (i + 2 < nt) {
    sm.s = qk_tile<B, 0, true, (B + 2) % 3, true>(fr, qf, vm, lane, sh.idx, i + 2, kvb, wave,
                                                  (i & 1) ? g_st8b : g_st8a);
  } else {
    sm.s = qk_tile<B, 0, false, (B + 2) % 3>(fr, qf, vm, lane, sh.idx, 0, kvb, wave);
  }
  pv_tile<(B + 2) % 3, true, false>(fr, nullptr, p0, p1, o, lane, sm, scale2, m_ref, m_max, over,
                                    l_run);
  p0 = sm.p0();
  p1 = sm.p1();
  if (i + 1 < nt) {
    wait_stage8(i + 2 < nt);
    dequant_stage8<(B + 1) % 3>((i & 1) ? g_st8a : g_st8b, wave, lane);
  }
  vm = sh.vmask[i + 1];
}

// One workgroup: one query x 128 heads (wave w: heads 32w .. 32w+31 of the
// block's head range), or one key slice of it in split mode.  The query's Q^T
// stays in registers (144 per lane), O [32 heads x 512] in 256 accumulation
// registers per lane.  kF8: kv holds fp8 rows (656 bytes), gathered into
// per-wave staging rows and converted to bf16 tiles one step ahead of use (three
// tile buffers); otherwise bf16 rows are gathered straight into four tile buffers.
template <bool kF8>
__device__ __forceinline__ void mla_body(
    const __bf16* __restrict__ q, const void* __restrict__ kv,
    const int32_t* __restrict__ idx, int n_kv, int H, int K, float sm_scale,
    __bf16* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_lse, int nsplit) {
  __shared__ __attribute__((aligned(16))) MlaShared sh;

  // longest rows first: in causal prefill the last queries select the most keys
  const int64_t t = int64_t(gridDim.x) - 1 - blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane >> 5;
  const int h0 = int(blockIdx.y) * kHeadsPerBlock + wave * 32;
  const int head = h0 + (lane & 31);
  const bool hvalid = head < H;
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  const float scale2 = sm_scale * kLog2e;

  const int ntiles = (K + kKT - 1) / kKT;
  const int i0 = int(int64_t(ntiles) * blockIdx.z / nsplit);
  int i1 = int(int64_t(ntiles) * (blockIdx.z + 1) / nsplit);
  const int32_t* irow = idx + t * K;

  // The index slice and the query's Q^T are loaded together: the index loads
  // first (vector-memory loads complete in order, so staging the indices waits
  // only for them), then Q, which stays in flight until the first tile.
  const int jbase = i0 * kKT;
  const int nx = (i1 - i0) * kKT;
  constexpr int kPer = kMaxIdx / kThreads;
  int rv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int x = tid + u * kThreads;
    const int j = jbase + x;
    rv[u] = (x < nx && j < K) ? irow[j] : -1;
  }
  // Q^T fragments: lane holds q[t, head, 16*st + 8*half .. +8].  A head past H
  // (the last head block of a head count that is not a multiple of 128) reads
  // head H-1 instead: finite values whose results are never written.
  bf16x8_t qf[kQSteps];
  {
    const __bf16* qr = q + (t * H + (hvalid ? head : H - 1)) * int64_t(kDqk) + 8 * half;
#pragma unroll
    for (int st = 0; st < kQSteps; ++st) qf[st] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * st);
  }

  // Stage the index slice in LDS (padded with -1 to whole tiles, -1 stored as
  // row 0) with per-tile validity masks, and drop trailing tiles that hold only
  // -1 padding (top-k rows are -1 padded at the end); padding elsewhere is
  // masked per key.  An entry outside [0, n_kv) is treated as -1, so no gather
  // reads outside kv.
  {
    int wl = -1;  // last valid position among this wave's loads (wave-uniform)
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int x = tid + u * kThreads;
      const bool ok = unsigned(rv[u]) < unsigned(n_kv);
      if (x < nx) sh.idx[x] = ok ? rv[u] : 0;
      // x advances by whole waves: 2 tiles per ballot (the wave is uniform in x < nx)
      const uint64_t b = __ballot(x < nx && ok);
      if (x < nx && lane == 0) sh.vmask[x / kKT] = uint32_t(b);
      if (x < nx && lane == 32) sh.vmask[x / kKT] = uint32_t(b >> 32);
      if (b != 0ull) wl = u * kThreads + wave * kWave + 63 - __builtin_clzll(b);
    }
    if (lane == 0) sh.wlast[wave] = wl;
    __syncthreads();
    int last = sh.wlast[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) last = max(last, sh.wlast[w]);
    i1 = last < 0 ? i0 : i0 + last / kKT + 1;
  }
  // tiles 1 .. nt-1 run in groups of four (fp8: three: the tile buffers of each
  // step are static); steps past the last tile are skipped, no tile is padded
  const int nt = i1 - i0;
  if (tid < 2) sh.redo[tid] = 0;
  __syncthreads();
  // Q^T has landed before the first gather is issued.  (The gathers are inline
  // asm that the compiler does not count; waiting for Q at its first use would
  // make it wait for gathers issued after Q as well.)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  f32x16_t o[kVTiles];
  float m_ref = -FLT_MAX;  // per head (lane column, base-2 units), same in both lane halves
  float m_max = -FLT_MAX;
  float l_run = 0.0f;      // per head, partial over this lane half's keys
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int n = 0; n < kVTiles; ++n) o[n] = f32x16_t{};
    l_run = 0.0f;
    bool over = false;
    bf16x8_t p0 = bf16x8_t{}, p1 = bf16x8_t{};
    if constexpr (kF8) {
      if (nt > 0) dma_tile8(g_st8a, sh.idx, 0, kvb, wave, lane);
      if (nt > 1) dma_tile8(g_st8b, sh.idx, 1, kvb, wave, lane);
      if (nt > 0) {
        // tile 0: converted, then S and softmax only
        wait_stage8(nt > 1);
        dequant_stage8<0>(g_st8a, wave, lane);
        wait_lgkm<0>();
        __builtin_amdgcn_s_barrier();
        {
          Softmax sm;
          bf16x8_t fr[4];
          if (nt > 2)
            sm.s = qk_tile<0, 0, true, -1, true>(fr, qf, sh.vmask[0], lane, sh.idx, 2, kvb, wave,
                                                 g_st8a);
          else
            sm.s = qk_tile<0, 0, false, -1>(fr, qf, sh.vmask[0], lane, sh.idx, 0, kvb, wave);
          softmax_all(sm, scale2, m_ref, m_max, over, l_run);
          p0 = sm.p0();
          p1 = sm.p1();
        }
        if (nt > 1) {
          wait_stage8(nt > 2);
          dequant_stage8<1>(g_st8b, wave, lane);
        }
        uint32_t vm = sh.vmask[1];
        for (int i = 1; i < nt; i += 3) {
          tile_step8<1>(sh, i, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run, scale2,
                        wave, lane);
          if (i + 1 < nt)
            tile_step8<2>(sh, i + 1, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run,
                          scale2, wave, lane);
          if (i + 2 < nt)
            tile_step8<0>(sh, i + 2, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run,
                          scale2, wave, lane);
        }
        const int lb = (nt - 1) % 3;
        const uint8_t* buf = lb == 0 ? g_kv0 : lb == 1 ? g_kv1 : g_kv2;
        Softmax none;
        bf16x8_t fr[4];
        pv_tile<-1, false, true>(fr, buf, p0, p1, o, lane, none, scale2, m_ref, m_max, over, l_run);
      }
    } else {
      if (nt > 0) dma_tile<0>(sh.idx, 0, kvb, wave, lane);
      if (nt > 1) dma_tile<1>(sh.idx, 1, kvb, wave, lane);
      if (nt > 0) {
        // tile 0: no P.V yet
        wait_tile(nt > 1);
        __builtin_amdgcn_s_barrier();
        if (nt > 2) dma_tile<2>(sh.idx, 2, kvb, wave, lane);
        {
          Softmax sm;
          bf16x8_t fr[4];
          sm.s = qk_tile<0, 0, false, -1>(fr, qf, sh.vmask[0], lane, sh.idx, 0, kvb, wave);
          softmax_all(sm, scale2, m_ref, m_max, over, l_run);
          p0 = sm.p0();
          p1 = sm.p1();
        }
        uint32_t vm = sh.vmask[1];
        // tiles 1 .. nt-1 in groups of four, the steps past nt skipped (one exit:
        // a loop left in the middle makes the register allocator copy O out of
        // the accumulation registers)
        for (int i = 1; i < nt; i += 4) {
          tile_step<1>(sh, i, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run, scale2, wave, lane);
          if (i + 1 < nt)
            tile_step<2>(sh, i + 1, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run, scale2,
                         wave, lane);
          if (i + 2 < nt)
            tile_step<3>(sh, i + 2, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run, scale2,
                         wave, lane);
          if (i + 3 < nt)
            tile_step<0>(sh, i + 3, nt, kvb, qf, o, p0, p1, vm, m_ref, m_max, over, l_run, scale2,
                         wave, lane);
        }
        // P.V of the last tile: no gather is in flight any more, so its buffer can
        // be chosen at run time
        const int lb = (nt - 1) & 3;
        const uint8_t* buf = lb == 0 ? g_kv0 : lb == 1 ? g_kv1 : lb == 2 ? g_kv2 : g_kv3;
        Softmax none;
        bf16x8_t fr[4];
        pv_tile<-1, false, true>(fr, buf, p0, p1, o, lane, none, scale2, m_ref, m_max, over, l_run);
      }
    }
    o_fence(o);  // the last MFMAs into O finish before O is read or cleared
    // the whole workgroup agrees on a second pass (its waves share barriers)
    if (__ballot(over) != 0ull && lane == 0) sh.redo[pass] = 1;
    __syncthreads();
    if (sh.redo[pass] == 0) break;
    m_ref = fmaxf(m_max, -FLT_MAX);
  }

  // epilogue (the head index is rebuilt here rather than kept live across the loop)
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int head_e = h0 + (lane_e & 31);
  const int half_e = lane_e >> 5;
  const bool hvalid_e = head_e < H;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_h = l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  // Output rows (or split partials) of the wave's 32 heads, 1 KB each in bf16.
  // O^T puts head h0 + l % 32 in lane l, value columns 32 n + acc_row(r, half)
  // in its registers, so the lane scales by its own head's 1 / l.  The tile
  // buffers are free now (the barrier above follows every wave's last read):
  // each wave stages its block in its own buffer row-major per head (kEpRow
  // bytes per head: 16 bytes of padding move successive heads 4 banks apart),
  // four consecutive columns per 8-byte write, then reads back whole head rows
  // (lane j: columns 8 j .. 8 j + 7) and writes each with one 1 KB store.
  // (fp8: three tile buffers, so wave 3 stages its block after the others, in buffer 0)
  if constexpr (kF8) {
    if (wave == 3) __syncthreads();
  }
  uint8_t* eb = wave == 0 ? g_kv0 : wave == 1 ? g_kv1 : wave == 2 ? g_kv2 : kF8 ? g_kv0 : g_kv3;
  {
    uint8_t* wb = eb + (lane_e & 31) * kEpRow + 8 * half_e;
#pragma unroll
    for (int n = 0; n < kVTiles; ++n) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2_t lo = {__bf16(o[n][4 * g] * inv), __bf16(o[n][4 * g + 1] * inv)};
        const bf16x2_t hi = {__bf16(o[n][4 * g + 2] * inv), __bf16(o[n][4 * g + 3] * inv)};
        const uint2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<uint2*>(wb + (32 * n + 8 * g) * 2) = v;
      }
    }
  }
  uint16_t* obase = nsplit == 1 ? reinterpret_cast<uint16_t*>(out) + t * H * int64_t(kDv)
                                : part_o + (t * nsplit + blockIdx.z) * H * int64_t(kDv);
  // every row is read before the first store (the registers that held Q^T are
  // free), so the LDS latency is paid once
  v8i16_t ov[32];
#pragma unroll
  for (int h = 0; h < 32; ++h)
    ov[h] = *reinterpret_cast<const v8i16_t*>(eb + h * kEpRow + 16 * lane_e);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 32; ++h)
    if (h0 + h < H) *reinterpret_cast<v8i16_t*>(obase + (h0 + h) * int64_t(kDv) + 8 * lane_e) = ov[h];
  if (half_e == 0 && hvalid_e) {
    if (nsplit == 1) {
      if (lse) lse[t * H + head_e] = lse_h;
    } else {
      part_lse[(t * nsplit + blockIdx.z) * H + head_e] = lse_h;
    }
  }
  if constexpr (kF8) {
    if (wave < 3) __syncthreads();  // buffer 0 is free for wave 3
  }
}

__global__ __launch_bounds__(kThreads, 1) void mla_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ idx, int n_kv, int H, int K, float sm_scale,
    __bf16* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_lse, int nsplit) {
  mla_body<false>(q, kv, idx, n_kv, H, K, sm_scale, out, lse, part_o, part_lse, nsplit);
}

// The same over the fp8 latent cache (656-byte rows).
__global__ __launch_bounds__(kThreads, 1) void mla_fp8_kernel(
    const __bf16* __restrict__ q, const uint8_t* __restrict__ kv,
    const int32_t* __restrict__ idx, int n_kv, int H, int K, float sm_scale,
    __bf16* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_lse, int nsplit) {
  mla_body<true>(q, kv, idx, n_kv, H, K, sm_scale, out, lse, part_o, part_lse, nsplit);
}

// Merge split partials (bf16, normalised per split): out = sum_s e^{lse_s - L} o_s
// with L = logsumexp_s lse_s.  One wave per (query, head), four heads per
// workgroup; lane l takes value columns 8l .. 8l+7 (16-byte loads and stores).
constexpr int kCombineHeads = 4;
__global__ __launch_bounds__(kCombineHeads * kWave) void mla_combine_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse, int H, int nsplit,
    __bf16* __restrict__ out, float* __restrict__ lse) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int h = int(blockIdx.y) * kCombineHeads + int(threadIdx.x) / kWave;
  if (h >= H) return;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part_lse[(t * nsplit + s) * H + h]);
  float wsum = 0.0f;
  float acc[8] = {};
  for (int s = 0; s < nsplit; ++s) {
    const float ls = part_lse[(t * nsplit + s) * H + h];
    const float ws = ls == -INFINITY ? 0.0f : __expf(ls - mx);
    wsum += ws;
    const uint4 v = *reinterpret_cast<const uint4*>(part_o + ((t * nsplit + s) * H + h) *
                                                                 int64_t(kDv) + 8 * lane);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = fmaf(ws, bf16_bits_to_f32(uint16_t(w4[j] & 0xFFFFu)), acc[2 * j]);
      acc[2 * j + 1] = fmaf(ws, bf16_bits_to_f32(uint16_t(w4[j] >> 16)), acc[2 * j + 1]);
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  uint4 r;
  uint32_t* r4 = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r4[j] = uint32_t(f32_to_bf16_bits(acc[2 * j] * inv)) |
            (uint32_t(f32_to_bf16_bits(acc[2 * j + 1] * inv)) << 16);
  *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + (t * H + h) * int64_t(kDv) +
                            8 * lane) = r;
  if (lse && lane == 0) lse[t * H + h] = wsum > 0.0f ? mx + __logf(wsum) : -INFINITY;
}

// fp32 inputs: one workgroup per (query, head).
__global__ __launch_bounds__(128) void mla_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ kv,
                                                      const int32_t* __restrict__ idx, int n_kv,
                                                      int H, int K, int dqk, int dv,
                                                      float sm_scale,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse) {
  extern __shared__ float sm[];  // q row [dqk], logits [K], reduction [4]
  float* sq = sm;
  float* sl = sm + dqk;
  float* red = sl + K;
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const float* qr = q + (t * H + h) * int64_t(dqk);
  for (int d = tid; d < dqk; d += 128) sq[d] = qr[d];
  __syncthreads();
  const int32_t* irow = idx + t * K;
  float mx = -INFINITY;
  for (int j = tid; j < K; j += 128) {
    const int r = irow[j];
    float l = -INFINITY;
    if (unsigned(r) < unsigned(n_kv)) {  // -1 and out-of-range entries are skipped
      const float* kr = kv + int64_t(r) * dqk;
      float dot = 0.0f;
      for (int d = 0; d < dqk; ++d) dot = fmaf(sq[d], kr[d], dot);
      l = dot * sm_scale;
    }
    sl[j] = l;
    mx = fmaxf(mx, l);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float den = 0.0f;
  for (int j = tid; j < K; j += 128) {
    const float p = sl[j] == -INFINITY ? 0.0f : __expf(sl[j] - mx);
    sl[j] = p;
    den += p;
  }
  den = wave_sum(den);
  if ((tid & 63) == 0) red[2 + (tid >> 6)] = den;
  __syncthreads();
  den = red[2] + red[3];
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  for (int d = tid; d < dv; d += 128) {
    float acc = 0.0f;
    for (int j = 0; j < K; ++j) {
      const int r = irow[j];
      if (unsigned(r) < unsigned(n_kv)) acc = fmaf(sl[j], kv[int64_t(r) * dqk + d], acc);
    }
    out[(t * H + h) * int64_t(dv) + d] = acc * inv;
  }
  if (lse && tid == 0) lse[t * H + h] = den > 0.0f ? mx + __logf(den) : -INFINITY;
}

// Number of key splits per query for the bf16 kernel (shared by the launcher
// and the workspace query).
int mla_splits(int64_t n_q, int32_t n_heads, int32_t K) {
  const int64_t blocks = n_q * ((n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
  const int ntiles = (K + kKT - 1) / kKT;
  const int min_s = (ntiles + kMaxIdx / kKT - 1) / (kMaxIdx / kKT);  // <= kMaxIdx keys each
  int s = 1;
  if (blocks < 192) {
    s = int((256 + blocks - 1) / blocks);
    if (s > ntiles) s = ntiles;
    if (s > 16) s = 16;
  }
  return s < min_s ? min_s : (s < 1 ? 1 : s);
}

}  // namespace

size_t mla_workspace_bytes(int64_t n_q, int32_t n_heads, int32_t d_qk, int32_t d_v,
                           int32_t K, int32_t dtype) {
  (void)d_qk;
  if (dtype != 1 && dtype != 2) return 0;
  const int s = mla_splits(n_q, n_heads, K);
  if (s == 1) return 0;
  // bf16 partial outputs, then fp32 partial LSEs
  return size_t(n_q) * s * n_heads * (size_t(d_v) * sizeof(uint16_t) + sizeof(float));
}

hipError_t launch_sparse_mla(const void* q, const void* kv, const int32_t* idx, int64_t n_q,
                             int64_t n_kv, int32_t n_heads, int32_t d_qk, int32_t d_v,
                             int32_t K, float sm_scale, int32_t dtype, void* out, float* lse,
                             void* workspace, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  if (dtype == 0) {
    const size_t smem = (size_t(d_qk) + K + 4) * sizeof(float);
    hipLaunchKernelGGL(mla_f32_kernel, dim3(unsigned(n_q), n_heads), dim3(128), smem, stream,
                       static_cast<const float*>(q), static_cast<const float*>(kv), idx,
                       int(n_kv), n_heads, K, d_qk, d_v, sm_scale, static_cast<float*>(out), lse);
    return hipGetLastError();
  }
  const int s = mla_splits(n_q, n_heads, K);
  const unsigned hb = unsigned((n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
  uint16_t* part_o = static_cast<uint16_t*>(workspace);
  float* part_lse =
      s > 1 ? reinterpret_cast<float*>(part_o + size_t(n_q) * s * n_heads * d_v) : nullptr;
  if (dtype == 2)
    hipLaunchKernelGGL(mla_fp8_kernel, dim3(unsigned(n_q), hb, s), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const uint8_t*>(kv), idx,
                       int(n_kv), n_heads, K, sm_scale, static_cast<__bf16*>(out), lse, part_o,
                       part_lse, s);
  else
    hipLaunchKernelGGL(mla_bf16_kernel, dim3(unsigned(n_q), hb, s), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(kv), idx,
                       int(n_kv), n_heads, K, sm_scale, static_cast<__bf16*>(out), lse, part_o,
                       part_lse, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  static_assert(kDv == 8 * kWave, "one wave per head row in the combine");
  hipLaunchKernelGGL(mla_combine_kernel, dim3(unsigned(n_q), (n_heads + kCombineHeads - 1) / kCombineHeads),
                     dim3(kCombineHeads * kWave), 0, stream, part_o, part_lse, n_heads, s,
                     static_cast<__bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace dsa
