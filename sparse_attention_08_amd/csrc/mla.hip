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
// bf16 kernel: one workgroup = one query x 128 heads, 8 waves = 4 head groups of
// 32 heads x 2 halves; or a slice of the query's selected keys when the key list
// is split (few queries: decode).  Per tile of 32 selected keys:
//   gather    LDS-DMA (global_load_lds, 16 bytes per lane) of the 32 latent rows
//             into a row-major LDS tile whose rows are padded to 1168 bytes
//             (conflict-free 16-byte fragment reads); the next tile's gather is
//             in flight while this one is computed (two LDS buffers);
//   S^T=K.Q^T v_mfma_f32_32x32x16_bf16 with keys on M and the wave's 32 heads on
//             N; half h of a head group contracts dims [288h, 288h+288) with its
//             Q^T half held in registers for the whole query, and the two fp32
//             partials are added through LDS (both waves then hold the same S);
//   softmax   fp32 in base-2 units (sm_scale * log2 e folded into one multiply);
//             lane l holds 16 keys of head l%32, so the max over keys is in-lane
//             plus one exchange with lane l^32; the running max only moves (and
//             the output is rescaled) when a tile's max exceeds it by more than
//             8, so the probabilities stay <= 2^8 and the rescale is rare;
//   O += P.V  the probabilities, rounded to bf16, are the A operand of the next
//             MFMA (heads on M, keys on K) in the order the S^T accumulator holds
//             them; the B operand (keys x value columns) comes from the same
//             row-major tile through ds_read_b64_tr_b16 (transposing LDS read);
//             half h accumulates value columns [256h, 256h+256) of its 32 heads
//             in 128 registers per lane.
// The row sum adds the bf16-rounded probabilities, so the output is an exact
// convex combination of value rows up to fp32 accumulation.
//
// Split mode writes per-split (normalised output, lse) in fp32 to the workspace;
// a combine kernel merges them with the log-sum-exp weights.
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
constexpr int kRowChunks = kRowBytes / 16 + 1;  // 73: one pad chunk per LDS row
constexpr int kKvStride = kRowChunks * 16;      // 1168: padded LDS row
constexpr int kTileChunks = kKT * kRowChunks;   // 2336
constexpr int kDmaPerTile = (kTileChunks + kWave - 1) / kWave;  // 37 wave loads of 1 KB
constexpr int kQSteps = kDqk / 16 / 2;          // 18 K-steps per wave (half of d_qk)
constexpr int kVTiles = kDv / 32 / 2;           // 8 value tiles per wave (half of d_v)
constexpr int kThreads = 512;                   // 8 waves: 4 head groups x 2 halves
constexpr int kWaves = kThreads / kWave;
constexpr int kDmaPerWave = (kDmaPerTile + kWaves - 1) / kWaves;  // 5
constexpr int kHeadsPerBlock = 128;
constexpr int kMaxIdx = 2048;                   // selected keys per workgroup (LDS-staged)
constexpr float kRescaleSlack = 8.0f;             // base-2 units: P <= 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;

// Row (head offset inside the wave's 32) that accumulator register r of a
// 32x32 MFMA output holds in lane half `half`.
__device__ __forceinline__ int acc_row(int r, int half) {
  return 8 * (r >> 2) + 4 * half + (r & 3);
}

struct MlaShared {
  float sx[kWaves][16][kWave];    // partial S^T exchange between the two d_qk halves
  int idx[kMaxIdx];               // this workgroup's slice of the top-k row (-1 -> row 0)
  uint32_t vmask[kMaxIdx / kKT];  // per tile: bit j set = selected key j is valid
  int last;
};

// Per-lane part of the LDS-DMA of a tile: wave-load j = wave + 8u copies LDS
// chunks [64j, 64j+64) of the padded tile; chunk c is (key c/73, 16-byte piece
// c%73 of that key's latent row; piece 72 is the row pad and repeats piece 71).
static_assert(kTileChunks <= 2400, "the c / 73 multiply-shift holds for c < 2400");

struct DmaLane {
  // (byte offset of the chunk in the latent row) << 16 | 4 * (key of the chunk)
  int pk[kDmaPerWave];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
      const int c = (wave + kWaves * u) * kWave + lane;
      const int k = (c * 1796) >> 17;  // c / 73 for c < 2400
      const int cc = c - k * kRowChunks;
      pk[u] = ((cc < kRowChunks - 1 ? cc : kRowChunks - 2) * 16) << 16 | (k < kKT ? k : 0) * 4;
    }
  }
};

// Issue the LDS-DMA loads of local tile lt (rows staged in sidx, -1 already
// replaced by row 0, whose scores are masked).
__device__ __forceinline__ void dma_tile(uint8_t* buf, const int* sidx, int lt,
                                         const uint8_t* __restrict__ kv, int wave, int lane) {
  // the per-lane pieces are recomputed here: held across the tile loop they
  // would be spilled, and the scratch reloads would wait on the DMA counter
  asm volatile("" : "+v"(lane));
  DmaLane d2;
  d2.init(wave, lane);
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int j = wave + kWaves * u;
    const bool last = j == kDmaPerTile - 1;   // the last wave-load covers 32 chunks
    if (j < kDmaPerTile && (!last || lane < kTileChunks - (kDmaPerTile - 1) * kWave)) {
      const int* ps = reinterpret_cast<const int*>(
          reinterpret_cast<const uint8_t*>(sidx + lt * kKT) + (d2.pk[u] & 0xFFFF));
      const uint32_t r = uint32_t(*ps);
      const uint8_t* src = kv + (uint64_t(r) * kRowBytes + (uint32_t(d2.pk[u]) >> 16));
      __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(buf + j * kWave * 16), 16, 0, 0);
    }
  }
}

// One workgroup: one query, 128 heads.  Wave w: head group g = w & 3 (32 heads),
// half h = w >> 2.  Half h computes the partial S^T over dims [288h, 288h+288),
// the two partials are added through LDS (both waves then hold the same S and run
// the same softmax), and half h accumulates output columns [256h, 256h+256).
// Everything lives in VGPRs (Q^T half: 72, O half: 128 per lane).
__shared__ __attribute__((aligned(16))) uint8_t g_kv0[kKT * kKvStride];
__shared__ __attribute__((aligned(16))) uint8_t g_kv1[kKT * kKvStride];

template <int kBuf>
__device__ __forceinline__ void mla_tile(MlaShared& sh, const bf16x8_t (&qf)[kQSteps],
                                         f32x16_t (&o)[kVTiles], float& m_run, float& l_run,
                                         uint32_t vmask, float scale2, int wave, int lane) {
  const uint8_t* buf = kBuf == 0 ? g_kv0 : g_kv1;
  const int half = lane >> 5;
  const int hs = wave >> 2;

  // partial S^T = K . Q^T over this wave's half of d_qk (keys on M, heads on N)
  f32x16_t s = f32x16_t{};
  const uint8_t* ka = buf + (lane & 31) * kKvStride + hs * kDqk + half * 16;
#pragma unroll
  for (int st = 0; st < kQSteps; ++st)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(ka + st * 32),
                                                qf[st], s, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) sh.sx[wave][r][lane] = s[r];
  // LDS-only exchange: wait for this wave's LDS writes, then a plain barrier (a
  // full __syncthreads would also wait for the in-flight LDS-DMA of the next tile)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  // full S (both halves add the same two partials: IEEE addition commutes, so
  // the two waves hold identical bits), in base-2 logit units
  const float* other = &sh.sx[wave ^ 4][0][lane];
  // key validity as per-register lane masks built on the scalar unit: register
  // r holds key 8*(r/4) + r%4 in lanes 0..31 and that key + 4 in lanes 32..63
  const float neg_inf = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = 8 * (r >> 2) + (r & 3);
    const uint64_t lm = (((vmask >> kr) & 1u) ? 0x00000000FFFFFFFFull : 0ull) |
                        (((vmask >> (kr + 4)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
    const float x = (s[r] + other[r * kWave]) * scale2;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(s[r]) : "v"(neg_inf), "v"(x), "s"(lm));
  }
  float mt = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  // m_run starts at -FLT_MAX (finite), so exp2(s - m_run) is 0 for masked keys
  // and the first tile with a finite logit always moves it (alpha = 0, O = 0)
  const bool grow = mt > m_run + kRescaleSlack;
  if (__ballot(grow) != 0ull) {
    const float m_new = grow ? mt : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float ar = __shfl(alpha, acc_row(r, half));
#pragma unroll
      for (int n = 0; n < kVTiles; ++n) o[n][r] *= ar;
    }
  }
  // P = 2^(S - m) rounded to bf16 (v_cvt_pk_bf16_f32, round to nearest even); the
  // row sum adds the rounded values (v_dot2 with ones), so the output is an exact
  // convex combination of value rows up to fp32 accumulation
  bf16x8_t p0, p1;
  float ps = 0.0f;
  const bf16x2_t ones = {__bf16(1.0f), __bf16(1.0f)};
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(s[r] - m_run);
#pragma unroll
  for (int r = 0; r < 8; r += 2) {
    const bf16x2_t a = {__bf16(s[r]), __bf16(s[r + 1])};
    const bf16x2_t b = {__bf16(s[r + 8]), __bf16(s[r + 9])};
    ps = __builtin_amdgcn_fdot2_f32_bf16(a, ones, ps, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(b, ones, ps, false);
    p0[r] = a[0];
    p0[r + 1] = a[1];
    p1[r] = b[0];
    p1[r + 1] = b[1];
  }
  l_run += ps;

  // O[:, 256*hs .. +256] += P . V.  The B operand (8 keys x 1 value column per
  // lane) is read from the row-major tile with ds_read_b64_tr_b16: in each group
  // of 16 lanes, lane 4m+q reads 4 value columns of key row k0+m and the
  // transpose hands lane i the 4 keys k0..k0+3 of column n0+i.  Lane half h
  // needs keys {4h..4h+3} (first read) and {8+4h..8+4h+3} (second read) of each
  // 16-key step, the order in which P sits in the S^T accumulator.
  const int grp = lane >> 4;      // 16-lane group
  const int li = lane & 15;
  const int n0 = 16 * (grp & 1);  // value column offset of the group inside a 32-wide tile
  const uint8_t* vb = buf + (li >> 2) * kKvStride + (hs * kVTiles * 32 + n0 + 4 * (li & 3)) * 2;
#pragma unroll
  for (int n = 0; n < kVTiles; ++n) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* base = vb + (16 * ks + 4 * half) * kKvStride + n * 64;
      const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base));
      const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + 8 * kKvStride));
      const bf16x8_t v = __builtin_bit_cast(
          bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
      o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ks == 0 ? p0 : p1, v, o[n], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void mla_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ idx, int H, int K, float sm_scale,
    __bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_lse, int nsplit) {
  __shared__ __attribute__((aligned(16))) MlaShared sh;

  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int half = lane >> 5;
  const int grp = wave & 3;
  const int hs = wave >> 2;  // which half of d_qk (Q.K) and of d_v (P.V)
  const int h0 = int(blockIdx.y) * kHeadsPerBlock + grp * 32;
  const int head = h0 + (lane & 31);
  const bool hvalid = head < H;
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);

  const float scale2 = sm_scale * kLog2e;
  const int ntiles = (K + kKT - 1) / kKT;
  const int i0 = int(int64_t(ntiles) * blockIdx.z / nsplit);
  int i1 = int(int64_t(ntiles) * (blockIdx.z + 1) / nsplit);
  const int32_t* irow = idx + t * K;

  // Stage this workgroup's index slice in LDS (padded with -1 to whole tiles) and
  // drop trailing tiles that hold only -1 padding (top-k rows are -1 padded at
  // the end); padding elsewhere is masked per key.
  {
    if (tid == 0) sh.last = -1;
    __syncthreads();
    int last = -1;
    const int jbase = i0 * kKT;
    for (int x = tid; x < (i1 - i0) * kKT; x += kThreads) {
      const int j = jbase + x;
      const int r = j < K ? irow[j] : -1;
      sh.idx[x] = r < 0 ? 0 : r;
      const uint64_t b = __ballot(r >= 0);   // x advances by whole waves: 2 tiles per ballot
      if (lane == 0) sh.vmask[x / kKT] = uint32_t(b);
      if (lane == 32) sh.vmask[x / kKT] = uint32_t(b >> 32);
      if (r >= 0) last = x;
    }
    if (last >= 0) atomicMax(&sh.last, last);
    __syncthreads();
    last = sh.last;
    i1 = last < 0 ? i0 : i0 + last / kKT + 1;
  }
  const int nt = i1 - i0;
  if (nt > 0) dma_tile(g_kv0, sh.idx, 0, kvb, wave, lane);

  // Q^T fragments: lane holds q[t, head, 288*hs + 16*st + 8*half .. +8]
  bf16x8_t qf[kQSteps];
  {
    const __bf16* qr =
        q + (t * H + (hvalid ? head : 0)) * int64_t(kDqk) + (kDqk / 2) * hs + 8 * half;
#pragma unroll
    for (int st = 0; st < kQSteps; ++st) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qr + 16 * st);
      qf[st] = hvalid ? v : bf16x8_t{};
    }
  }

  f32x16_t o[kVTiles];
#pragma unroll
  for (int n = 0; n < kVTiles; ++n) o[n] = f32x16_t{};
  float m_run = -FLT_MAX;   // per head (lane column, base-2 units), same in both lane halves
  float l_run = 0.0f;       // per head, partial over this lane half's keys

  for (int lt = 0; lt < nt; lt += 2) {
    // tile lt (buffer 0); the DMA of tile lt+1 into buffer 1 overlaps it
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (lt + 1 < nt) dma_tile(g_kv1, sh.idx, lt + 1, kvb, wave, lane);
    mla_tile<0>(sh, qf, o, m_run, l_run, sh.vmask[lt],
                scale2, wave, lane);
    if (lt + 1 >= nt) break;
    // tile lt+1 (buffer 1)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (lt + 2 < nt) dma_tile(g_kv0, sh.idx, lt + 2, kvb, wave, lane);
    mla_tile<1>(sh, qf, o, m_run, l_run,
                sh.vmask[lt + 1], scale2, wave, lane);
  }

  // epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_h = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  const int col0 = hs * kVTiles * 32 + (lane & 31);
  if (nsplit == 1) {
    if (lse && half == 0 && hs == 0 && hvalid) lse[t * H + head] = lse_h;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = h0 + acc_row(r, half);
      const float ir = __shfl(inv, acc_row(r, half));
      if (hr < H) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(out) + (t * H + hr) * int64_t(kDv) + col0;
#pragma unroll
        for (int n = 0; n < kVTiles; ++n) orow[n * 32] = f32_to_bf16_bits(o[n][r] * ir);
      }
    }
  } else {
    const int64_t slot = t * nsplit + blockIdx.z;
    if (half == 0 && hs == 0 && hvalid) part_lse[slot * H + head] = lse_h;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = h0 + acc_row(r, half);
      const float ir = __shfl(inv, acc_row(r, half));
      if (hr < H) {
        float* orow = part_o + (slot * H + hr) * int64_t(kDv) + col0;
#pragma unroll
        for (int n = 0; n < kVTiles; ++n) orow[n * 32] = o[n][r] * ir;
      }
    }
  }
}

// Merge split partials: out = sum_s e^{lse_s - L} o_s with L = logsumexp_s lse_s.
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          int H, int nsplit,
                                                          __bf16* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part_lse[(t * nsplit + s) * H + h]);
  float wsum = 0.0f;
  float acc[kDv / 128] = {};
  for (int s = 0; s < nsplit; ++s) {
    const float ls = part_lse[(t * nsplit + s) * H + h];
    const float ws = ls == -INFINITY ? 0.0f : __expf(ls - mx);
    wsum += ws;
    const float* po = part_o + ((t * nsplit + s) * H + h) * int64_t(kDv);
#pragma unroll
    for (int x = 0; x < kDv / 128; ++x) acc[x] = fmaf(ws, po[threadIdx.x + 128 * x], acc[x]);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  uint16_t* orow = reinterpret_cast<uint16_t*>(out) + (t * H + h) * int64_t(kDv);
#pragma unroll
  for (int x = 0; x < kDv / 128; ++x) orow[threadIdx.x + 128 * x] = f32_to_bf16_bits(acc[x] * inv);
  if (lse && threadIdx.x == 0) lse[t * H + h] = wsum > 0.0f ? mx + __logf(wsum) : -INFINITY;
}

// fp32 inputs: one workgroup per (query, head).
__global__ __launch_bounds__(128) void mla_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ kv,
                                                      const int32_t* __restrict__ idx, int H,
                                                      int K, int dqk, int dv, float sm_scale,
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
    if (r >= 0) {
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
      if (r >= 0) acc = fmaf(sl[j], kv[int64_t(r) * dqk + d], acc);
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
  if (dtype != 1) return 0;
  const int s = mla_splits(n_q, n_heads, K);
  if (s == 1) return 0;
  return size_t(n_q) * s * n_heads * (size_t(d_v) + 1) * sizeof(float);
}

hipError_t launch_sparse_mla(const void* q, const void* kv, const int32_t* idx, int64_t n_q,
                             int64_t n_kv, int32_t n_heads, int32_t d_qk, int32_t d_v,
                             int32_t K, float sm_scale, int32_t dtype, void* out, float* lse,
                             void* workspace, hipStream_t stream) {
  (void)n_kv;
  if (n_q == 0) return hipSuccess;
  if (dtype == 0) {
    const size_t smem = (size_t(d_qk) + K + 4) * sizeof(float);
    hipLaunchKernelGGL(mla_f32_kernel, dim3(unsigned(n_q), n_heads), dim3(128), smem, stream,
                       static_cast<const float*>(q), static_cast<const float*>(kv), idx,
                       n_heads, K, d_qk, d_v, sm_scale, static_cast<float*>(out), lse);
    return hipGetLastError();
  }
  const int s = mla_splits(n_q, n_heads, K);
  const unsigned hb = unsigned((n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = s > 1 ? part_o + size_t(n_q) * s * n_heads * d_v : nullptr;
  hipLaunchKernelGGL(mla_bf16_kernel, dim3(unsigned(n_q), hb, s), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(kv), idx, n_heads,
                     K, sm_scale, static_cast<__bf16*>(out), lse, part_o, part_lse, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(unsigned(n_q), n_heads), dim3(128), 0, stream,
                     part_o, part_lse, n_heads, s, static_cast<__bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace dsa
