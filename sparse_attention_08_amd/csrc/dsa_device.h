// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Order-preserving 32-bit key of an fp32 score: a > b  <=>  key(a) > key(b) for
// non-NaN values.  -0.0 is folded onto +0.0 first so that they tie.  -inf (and
// anything that sorts below it) maps to 0, which marks "never selectable".
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return k > 0x007FFFFFu ? k : 0u;
}

// ---------------------------------------------------------------------------
// bf16 <-> f32 (round to nearest even; inputs here are finite)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(r >> 16);
}

// ---------------------------------------------------------------------------
// wave64 / block reductions and scans
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// within each row of 16 lanes by shifts of 1, 2, 4 and 8 (lanes shifted in
// from outside the row add 0), then lane 15 of rows 0 and 2 into rows 1 and 3,
// then lane 31 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  int x = int(v);
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return uint32_t(x);
}

// Exclusive prefix sum over the threads of a block of NT threads (NT/64 waves).
// `tmp` needs NT/64 entries of shared memory.  Returns the prefix; `total` gets
// the block total.  Contains two __syncthreads().
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* tmp,
                                                       uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t x = wave_inclusive_sum(v);
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = tmp[w];
    off += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* tmp) {
  uint32_t total;
  block_exclusive_sum<NT>(v, tmp, total);
  return total;
}

}  // namespace dsa
