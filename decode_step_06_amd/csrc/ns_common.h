// Shared device/host definitions of the gfx950 decode-step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef NS_BLOCK
#define NS_BLOCK 16  // KV slots per cache block
#endif

namespace ns {

typedef uint16_t bf16_t;  // raw bf16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// float -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Low / high bf16 of a packed pair as float.
__device__ __forceinline__ float lo_bf16(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element storage type helpers: T is float or bf16_t.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int per16 = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ float load(const float* p, long i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, long i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int per16 = 8;
  __device__ static __forceinline__ float load(const bf16_t* p, long i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(bf16_t* p, long i, float v) { p[i] = f32_to_bf16(v); }
};

// Wavefront (64-lane) reductions.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace ns
