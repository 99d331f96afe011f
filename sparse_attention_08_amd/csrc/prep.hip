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

// Smallest power of two s with amax <= 448 * s (1 for amax == 0).
__device__ __forceinline__ float pow2_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  const int ea = int((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
  float s = ldexpf(1.0f, ea - 8);
  while (amax > 448.0f * s) s *= 2.0f;
  while (amax <= 448.0f * s * 0.5f) s *= 0.5f;
  return s;
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
  if (is_key) {  // LayerNorm, fp32, biased variance
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
