// Shared device helpers of the CSA2 HIP library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxHeads = CSA2_IDX_HEADS;  // 32
constexpr int kIdxDim = CSA2_IDX_DIM;      // 128
constexpr int kHeads = CSA2_HEADS;         // 64
constexpr int kDim = CSA2_DIM;             // 512
constexpr int kTopK = CSA2_TOPK;           // 512

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Order-preserving maps: larger float <-> larger unsigned key.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t f64_key(double d) {
  if (d == 0.0) d = 0.0;  // one key for +0 and -0
  uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Bin of x among 256 equal-width bins starting at a (scale = 255.99 / width);
// monotone non-decreasing in x.
__device__ __forceinline__ uint32_t value_bin(float x, float a, float scale) {
  const float f = (x - a) * scale;
  return f >= 255.f ? 255u : (f > 0.f ? (uint32_t)f : 0u);
}

// Number of compressed entries visible to query t (see csa2.h).
__device__ __forceinline__ int64_t n_visible(const int32_t* q_pos, int t, int ratio, int64_t N) {
  if (q_pos == nullptr) return N;
  int64_t p = (int64_t)q_pos[t];
  if (p < 0) return 0;
  int64_t n = (p + 1) / ratio;
  return n < N ? n : N;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace csa2
