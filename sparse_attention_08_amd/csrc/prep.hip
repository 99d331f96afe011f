// Indexer operand preparation (gfx950), run once per input set.
//
// From the vLLM API page "vllm.models.kimi_k3.nvidia.dsa":
//   KimiK3DSAIndexerKNorm             LayerNorm of the shared key (weight 1, bias 0),
//                                     computed in fp32;
//   KimiK3DSAIndexer._apply_index_rope RoPE on the leading rope_dim dims, half-split
//                                     pairing, after the norm; leading rope_dim/2
//                                     frequencies of the main rotary cache;
//   KimiK3DSAIndexer (scale format, score)
//                                     power-of-two scale per head_dim block, query
//                                     scale folded into the head weights.
// One wave per row; a row is either one (token, head) query vector or one key.
// The rotation angle pos * inv_freq and its sine/cosine are evaluated in double
// so that large positions do not lose the angle; the rest is fp32.
#include <cmath>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kMaxD = 256;
constexpr int kRowsPerBlock = 4;

// OCP e4m3fn encoding of |x| <= 448 with round-to-nearest-even.
__device__ __forceinline__ uint8_t encode_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0.015625f) {  // below 2^-6: subnormal step 2^-9 (8 rounds up to 2^-6)
    const uint32_t qv = uint32_t(rintf(a * 512.0f));
    return uint8_t(sign | qv);
  }
  int e = int((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // floor(log2 a)
  const float m = ldexpf(a, -e);                        // [1, 2)
  uint32_t qv = uint32_t(rintf(m * 8.0f));              // [8, 16]
  if (qv == 16u) {
    qv = 8u;
    ++e;
  }
  return uint8_t(sign | (uint32_t(e + 7) << 3) | (qv - 8u));
}

// OCP FP4 E2M1 code of x (round to nearest even on the grid 0, .5, 1, 1.5, 2,
// 3, 4, 6; beyond 6 saturates): sign in bit 3.
__device__ __forceinline__ uint32_t encode_e2m1(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fabsf(x);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f  ? 4u : a < 3.5f  ? 5u : a <= 5.0f  ? 6u : 7u;
  return sign | c;
}

// MXFP4 block scale exponent: floor(log2 amax) - 2 (0 for amax == 0), within
// the E8M0 range.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = ilogbf(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Smallest power of two s with amax <= 448 * s (1 for amax == 0).
__device__ __forceinline__ float pow2_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  const int ea = int((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
  float s = ldexpf(1.0f, ea - 8);
  while (amax > 448.0f * s) s *= 2.0f;
  while (amax <= 448.0f * s * 0.5f) s *= 0.5f;
  return s;
}

// LayerNorm of one row held by one wave (x[j] = element lane + 64 j, zero past
// D): fp32, biased variance.
__device__ __forceinline__ void wave_layer_norm(float (&x)[kMaxD / kWave], int D, float eps,
                                                int lane) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxD / kWave; ++j) s += x[j];
  const float mean = wave_sum(s) / float(D);
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxD / kWave; ++j) {
    const int e = lane + kWave * j;
    const float d = e < D ? x[j] - mean : 0.0f;
    v = fmaf(d, d, v);
  }
  const float var = wave_sum(v) / float(D);
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < kMaxD / kWave; ++j) {
    const int e = lane + kWave * j;
    x[j] = e < D ? (x[j] - mean) * rstd : 0.0f;
  }
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void prep_kernel(
    const float* __restrict__ q_raw, const float* __restrict__ k_raw,
    const float* __restrict__ w, const int32_t* __restrict__ pos_q,
    const int32_t* __restrict__ pos_k, int64_t n_q, int64_t n_k, int H, int D, int rope_dim,
    int rope_main, float theta, float eps, int dtype, void* __restrict__ q_out,
    void* __restrict__ k_out, float* __restrict__ w_out, float* __restrict__ k_scale_out) {
  __shared__ float buf[kRowsPerBlock][kMaxD];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t nqr = n_q * H;
  const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + wave;
  const bool live = row < nqr + n_k;
  const bool is_key = row >= nqr;
  const int64_t r = is_key ? row - nqr : row;  // key index, or (token*H + head)
  const float* src = live ? (is_key ? k_raw + r * D : q_raw + r * D) : k_raw;

  float x[kMaxD / kWave];
#pragma unroll
  for (int j = 0; j < kMaxD / kWave; ++j) {
    const int e = lane + kWave * j;
    x[j] = (live && e < D) ? src[e] : 0.0f;
  }
  if (is_key) wave_layer_norm(x, D, eps, lane);  // LayerNorm, fp32, biased variance
  if (rope_dim > 0) {
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j) buf[wave][lane + kWave * j] = x[j];
    __syncthreads();
    const int halfr = rope_dim / 2;
    const int64_t pos = live ? (is_key ? pos_k[r] : pos_q[r / H]) : 0;
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j) {
      const int e = lane + kWave * j;
      if (e < rope_dim) {
        const int i = e < halfr ? e : e - halfr;
        const double inv_freq = pow(double(theta), -2.0 * double(i) / double(rope_main));
        double sn, cs;
        sincos(double(pos) * inv_freq, &sn, &cs);
        const float c = float(cs), s = float(sn);
        x[j] = e < halfr ? x[j] * c - buf[wave][e + halfr] * s
                         : x[j] * c + buf[wave][e - halfr] * s;
      }
    }
  }
  if (!live) return;

  if (dtype == 3) {
    // MXFP4: element e = lane + 64 j sits in block e / 32, i.e. the lane half
    // of slot j; the block max reduces over those 32 lanes
    const int half = lane >> 5;
    uint8_t* codes;
    uint8_t* scales;
    if (is_key) {
      codes = static_cast<uint8_t*>(k_out) + r * (D / 2);
      scales = reinterpret_cast<uint8_t*>(k_scale_out) + r * (D / 32);
    } else {
      const int64_t t = r / H, h = r % H;
      uint8_t* tok = static_cast<uint8_t*>(q_out) + t * H * int64_t(D / 2 + D / 32);
      codes = tok + h * (D / 2);
      scales = tok + int64_t(H) * (D / 2) + h * (D / 32);
      if (lane == 0) w_out[r] = w[r];
    }
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j) {
      if (kWave * j >= D) break;
      float amax = fabsf(x[j]);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const int ex = mx_exponent(amax);
      const uint32_t c = encode_e2m1(ldexpf(x[j], -ex));
      const uint32_t nb = uint32_t(__shfl_down(int(c), 1));  // the next element's code
      if ((lane & 1) == 0) codes[(lane + kWave * j) / 2] = uint8_t(c | (nb << 4));
      if ((lane & 31) == 0) scales[2 * j + half] = uint8_t(ex + 127);
    }
    return;
  }
  if (dtype == 0) {
    float* dst = (is_key ? static_cast<float*>(k_out) : static_cast<float*>(q_out)) + r * D;
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j)
      if (lane + kWave * j < D) dst[lane + kWave * j] = x[j];
  } else if (dtype == 1) {
    uint16_t* dst =
        (is_key ? static_cast<uint16_t*>(k_out) : static_cast<uint16_t*>(q_out)) + r * D;
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j)
      if (lane + kWave * j < D) dst[lane + kWave * j] = f32_to_bf16_bits(x[j]);
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax = wave_max(amax);
    const float s = pow2_scale(amax);
    uint8_t* dst = (is_key ? static_cast<uint8_t*>(k_out) : static_cast<uint8_t*>(q_out)) + r * D;
#pragma unroll
    for (int j = 0; j < kMaxD / kWave; ++j)
      if (lane + kWave * j < D) dst[lane + kWave * j] = encode_e4m3(x[j] / s);
    if (lane == 0) {
      if (is_key) k_scale_out[r] = s;
      else w_out[r] = w[r] * s;
    }
    return;
  }
  if (!is_key && lane == 0 && w_out) w_out[r] = w[r];
}

// The fused insert into the fp8 index-key cache (KimiK3DSAIndexer._fused_k_insert
// on the vLLM API page "vllm.models.kimi_k3.nvidia.dsa"): one wave per new key
// row -- LayerNorm with the norm's weight and bias, one power-of-two scale for
// the row, e4m3 codes -- written to its cache slot.  A negative slot (padding)
// or one past the cache writes nothing.  Lane l holds the kPer consecutive
// elements kPer*l .. (the row is read and written with one vector access per
// lane; the norm's sums and the max do not depend on the order), and a wave
// issues the loads of kInsRows rows before it works on any of them.
constexpr int kInsRows = 4;  // rows per wave, their loads issued together

template <bool kBf16In, int kPer>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_insert_kernel(
    const void* __restrict__ k_raw, const float* __restrict__ weight,
    const float* __restrict__ bias, float eps, const int64_t* __restrict__ slots,
    int64_t n_tok, int64_t n_slots, int D, uint8_t* __restrict__ cache,
    float* __restrict__ cache_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave) * kInsRows;
  const int e0 = kPer * lane;
  const bool on = e0 < D;  // D is a multiple of kPer
  float wg[kPer], bs[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    wg[j] = (on && weight) ? weight[e0 + j] : 1.0f;
    bs[j] = (on && bias) ? bias[e0 + j] : 0.0f;
  }
  float x[kInsRows][kPer];
  int64_t slot[kInsRows];
#pragma unroll
  for (int r = 0; r < kInsRows; ++r) {
    const int64_t row = row0 + r;
    const bool live = row < n_tok;
    slot[r] = live ? slots[row] : -1;
    const int64_t rr = live ? row : 0;
    if constexpr (kBf16In) {
      const uint16_t* src = static_cast<const uint16_t*>(k_raw) + rr * D + e0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) x[r][j] = on ? bf16_bits_to_f32(src[j]) : 0.0f;
    } else {
      const float* src = static_cast<const float*>(k_raw) + rr * D + e0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) x[r][j] = on ? src[j] : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < kInsRows; ++r) {
    if (slot[r] < 0 || slot[r] >= n_slots) continue;  // padding or past the cache (wave-uniform)
    // LayerNorm, fp32, biased variance, then the norm's weight and bias
    float sm = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) sm += x[r][j];
    const float mean = wave_sum(sm) / float(D);
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float d = on ? x[r][j] - mean : 0.0f;
      v = fmaf(d, d, v);
    }
    const float rstd = 1.0f / sqrtf(wave_sum(v) / float(D) + eps);
    float y[kPer];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      y[j] = fmaf((x[r][j] - mean) * rstd, wg[j], bs[j]);
      amax = on ? fmaxf(amax, fabsf(y[j])) : amax;
    }
    amax = wave_max(amax);
    const float s = pow2_scale(amax);
    if (on) {
      uint8_t c[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) c[j] = encode_e4m3(y[j] / s);
      uint8_t* dst = cache + slot[r] * D + e0;
      if constexpr (kPer == 2) {
        *reinterpret_cast<uint16_t*>(dst) = uint16_t(c[0] | (c[1] << 8));
      } else {
        *reinterpret_cast<uint32_t*>(dst) =
            uint32_t(c[0]) | (uint32_t(c[1]) << 8) | (uint32_t(c[2]) << 16) | (uint32_t(c[3]) << 24);
      }
    }
    if (lane == 0) cache_scale[slot[r]] = s;
  }
}

// head_dim 128: 16 lanes per row, four rows per wave, eight consecutive
// elements per lane (one 16- or 32-byte load, one 8-byte store of codes); the
// row sums and max reduce over the 16 lanes of the row.
template <int O>
__device__ __forceinline__ float xor16_sum(float v) {
  if constexpr (O > 0) return xor16_sum<O / 2>(v + __shfl_xor(v, O));
  return v;
}
template <int O>
__device__ __forceinline__ float xor16_max(float v) {
  if constexpr (O > 0) return xor16_max<O / 2>(fmaxf(v, __shfl_xor(v, O)));
  return v;
}

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_insert128_kernel(
    const void* __restrict__ k_raw, const float* __restrict__ weight,
    const float* __restrict__ bias, float eps, const int64_t* __restrict__ slots,
    int64_t n_tok, int64_t n_slots, uint8_t* __restrict__ cache,
    float* __restrict__ cache_scale) {
  constexpr int D = 128;
  const int sub = threadIdx.x & 15;
  const int64_t row = (int64_t(blockIdx.x) * 256 + threadIdx.x) / 16;
  const int e0 = 8 * sub;
  float x[8], wg[8], bs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    wg[j] = weight ? weight[e0 + j] : 1.0f;
    bs[j] = bias ? bias[e0 + j] : 0.0f;
  }
  const int64_t rr = row < n_tok ? row : n_tok - 1;
  const int64_t slot = slots[rr];
  if constexpr (kBf16In) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k_raw) + rr * D + e0);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_bits_to_f32(uint16_t(w4[j] & 0xFFFFu));
      x[2 * j + 1] = bf16_bits_to_f32(uint16_t(w4[j] >> 16));
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(k_raw) + rr * D + e0);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(k_raw) + rr * D + e0 + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  float sm = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sm += x[j];
  const float mean = xor16_sum<8>(sm) / float(D);
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = x[j] - mean;
    v = fmaf(d, d, v);
  }
  const float rstd = 1.0f / sqrtf(xor16_sum<8>(v) / float(D) + eps);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = fmaf((x[j] - mean) * rstd, wg[j], bs[j]);
    amax = fmaxf(amax, fabsf(x[j]));
  }
  const float s = pow2_scale(xor16_max<8>(amax));
  if (row >= n_tok || slot < 0 || slot >= n_slots) return;
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= uint32_t(encode_e4m3(x[j] / s)) << (8 * j);
    hi |= uint32_t(encode_e4m3(x[4 + j] / s)) << (8 * j);
  }
  *reinterpret_cast<uint2*>(cache + slot * D + e0) = make_uint2(lo, hi);
  if (sub == 0) cache_scale[slot] = s;
}

// One latent row into the fp8 MLA cache: a wave per token, lane l holding
// latent dims 8l .. 8l+7 (the 128-dim scale block of 16 lanes reduces its amax
// with xor 1, 2, 4, 8), lanes 0..15 also four rope dims each.  Output row of
// 656 bytes: 512 e4m3 codes, 4 fp32 power-of-two scales, 64 bf16 rope values.
constexpr int kMlaLatent = 512, kMlaRope = 64, kMlaRow8 = 656;
template <bool kBf16In>
__global__ __launch_bounds__(256) void mla_kv_insert_kernel(const void* __restrict__ kv,
                                                           const int64_t* __restrict__ slots,
                                                           int64_t n_tok, int64_t n_slots,
                                                           uint8_t* __restrict__ cache) {
  constexpr int D = kMlaLatent + kMlaRope;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = int64_t(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  if (row >= n_tok) return;  // whole waves: the xor reductions stay inside one row
  const int64_t slot = slots[row];  // checked after the row's loads are issued: no serial round trip
  float x[8], r[4];
  if constexpr (kBf16In) {
    const uint16_t* src = static_cast<const uint16_t*>(kv) + row * D;
    const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * lane);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_bits_to_f32(uint16_t(w4[j] & 0xFFFFu));
      x[2 * j + 1] = bf16_bits_to_f32(uint16_t(w4[j] >> 16));
    }
    uint2 rp = make_uint2(0u, 0u);
    if (lane < 16) rp = *reinterpret_cast<const uint2*>(src + kMlaLatent + 4 * lane);
    if (slot < 0 || slot >= n_slots) return;
    // bf16 rope values are copied as they are
    if (lane < 16) *reinterpret_cast<uint2*>(cache + slot * kMlaRow8 + kMlaLatent + 16 + 8 * lane) = rp;
  } else {
    const float* src = static_cast<const float*>(kv) + row * D;
    const float4 a = *reinterpret_cast<const float4*>(src + 8 * lane);
    const float4 b = *reinterpret_cast<const float4*>(src + 8 * lane + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < 16) c = *reinterpret_cast<const float4*>(src + kMlaLatent + 4 * lane);
    if (slot < 0 || slot >= n_slots) return;
    if (lane < 16) {
      r[0] = c.x; r[1] = c.y; r[2] = c.z; r[3] = c.w;
      const uint32_t lo = uint32_t(f32_to_bf16_bits(r[0])) | (uint32_t(f32_to_bf16_bits(r[1])) << 16);
      const uint32_t hi = uint32_t(f32_to_bf16_bits(r[2])) | (uint32_t(f32_to_bf16_bits(r[3])) << 16);
      *reinterpret_cast<uint2*>(cache + slot * kMlaRow8 + kMlaLatent + 16 + 8 * lane) =
          make_uint2(lo, hi);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  const float s = pow2_scale(xor16_max<8>(amax));
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= uint32_t(encode_e4m3(x[j] / s)) << (8 * j);
    hi |= uint32_t(encode_e4m3(x[4 + j] / s)) << (8 * j);
  }
  uint8_t* dst = cache + slot * kMlaRow8;
  *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(lo, hi);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(dst + kMlaLatent + 4 * (lane >> 4)) = s;
}

__global__ __launch_bounds__(256) void row_windows_kernel(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ cu_k,
                                                          int n_seqs, int64_t n_rows, int causal,
                                                          int32_t* __restrict__ rs,
                                                          int32_t* __restrict__ re) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_rows) return;
  // last b with cu_q[b] <= t
  int lo = 0, hi = n_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int q0 = cu_q[b], q_len = cu_q[b + 1] - q0;
  const int k0 = cu_k[b], k_len = cu_k[b + 1] - k0;
  const int p = int(t) - q0;
  int e = k0 + k_len;
  if (causal) {
    e = k0 + k_len - q_len + p + 1;
    e = e < k0 ? k0 : (e > k0 + k_len ? k0 + k_len : e);
  }
  rs[t] = k0;
  re[t] = e;
}

}  // namespace

hipError_t launch_indexer_prep(const float* q_raw, const float* k_raw, const float* w,
                               const int32_t* pos_q, const int32_t* pos_k, int64_t n_q,
                               int64_t n_k, int32_t n_heads, int32_t head_dim, int32_t rope_dim,
                               int32_t rope_main_dim, float theta, float eps, int32_t dtype,
                               void* q_out, void* k_out, float* w_out, float* k_scale_out,
                               hipStream_t stream) {
  const int64_t rows = n_q * n_heads + n_k;
  if (rows == 0) return hipSuccess;
  const unsigned grid = unsigned((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(kRowsPerBlock * kWave), 0, stream, q_raw,
                     k_raw, w, pos_q, pos_k, n_q, n_k, n_heads, head_dim, rope_dim,
                     rope_main_dim, theta, eps, dtype, q_out, k_out, w_out, k_scale_out);
  return hipGetLastError();
}

hipError_t launch_indexer_k_insert(const void* k_raw, int32_t k_dtype, const float* weight,
                                   const float* bias, float eps, const int64_t* slot_mapping,
                                   int64_t n_tokens, int32_t head_dim, uint8_t* k_cache,
                                   float* k_scale_cache, int64_t n_slots, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  if (head_dim == 128) {
    const unsigned g128 = unsigned((n_tokens + 15) / 16);
    if (k_dtype == 1)
      hipLaunchKernelGGL(k_insert128_kernel<true>, dim3(g128), dim3(256), 0, stream, k_raw,
                         weight, bias, eps, slot_mapping, n_tokens, n_slots, k_cache,
                         k_scale_cache);
    else
      hipLaunchKernelGGL(k_insert128_kernel<false>, dim3(g128), dim3(256), 0, stream, k_raw,
                         weight, bias, eps, slot_mapping, n_tokens, n_slots, k_cache,
                         k_scale_cache);
    return hipGetLastError();
  }
  const int64_t per_block = int64_t(kRowsPerBlock) * kInsRows;
  const unsigned grid = unsigned((n_tokens + per_block - 1) / per_block);
  const dim3 blk(kRowsPerBlock * kWave);
  // two elements per lane up to 128 dims, four up to 256 (the C ABI admits
  // only those head dims)
  if (head_dim <= 128 && head_dim % 2 == 0) {
    if (k_dtype == 1)
      hipLaunchKernelGGL((k_insert_kernel<true, 2>), dim3(grid), blk, 0, stream, k_raw, weight,
                         bias, eps, slot_mapping, n_tokens, n_slots, head_dim, k_cache,
                         k_scale_cache);
    else
      hipLaunchKernelGGL((k_insert_kernel<false, 2>), dim3(grid), blk, 0, stream, k_raw, weight,
                         bias, eps, slot_mapping, n_tokens, n_slots, head_dim, k_cache,
                         k_scale_cache);
  } else if (head_dim % 4 == 0) {
    if (k_dtype == 1)
      hipLaunchKernelGGL((k_insert_kernel<true, 4>), dim3(grid), blk, 0, stream, k_raw, weight,
                         bias, eps, slot_mapping, n_tokens, n_slots, head_dim, k_cache,
                         k_scale_cache);
    else
      hipLaunchKernelGGL((k_insert_kernel<false, 4>), dim3(grid), blk, 0, stream, k_raw, weight,
                         bias, eps, slot_mapping, n_tokens, n_slots, head_dim, k_cache,
                         k_scale_cache);
  } else {
    return hipErrorInvalidValue;  // rejected by the C ABI before this point
  }
  return hipGetLastError();
}

hipError_t launch_mla_kv_insert(const void* kv, int32_t kv_dtype, const int64_t* slot_mapping,
                                int64_t n_tokens, uint8_t* kv_cache, int64_t n_slots,
                                hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const unsigned grid = unsigned((n_tokens + 3) / 4);
  if (kv_dtype == 1)
    hipLaunchKernelGGL(mla_kv_insert_kernel<true>, dim3(grid), dim3(256), 0, stream, kv,
                       slot_mapping, n_tokens, n_slots, kv_cache);
  else
    hipLaunchKernelGGL(mla_kv_insert_kernel<false>, dim3(grid), dim3(256), 0, stream, kv,
                       slot_mapping, n_tokens, n_slots, kv_cache);
  return hipGetLastError();
}

hipError_t launch_row_windows(const int32_t* cu_q, const int32_t* cu_k, int32_t n_seqs,
                              int64_t n_rows, int32_t causal, int32_t* row_starts,
                              int32_t* row_ends, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const unsigned grid = unsigned((n_rows + 255) / 256);
  hipLaunchKernelGGL(row_windows_kernel, dim3(grid), dim3(256), 0, stream, cu_q, cu_k, n_seqs,
                     n_rows, causal, row_starts, row_ends);
  return hipGetLastError();
}

}  // namespace dsa
