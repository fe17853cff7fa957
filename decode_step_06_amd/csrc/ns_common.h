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

// Rotate-half RoPE of one pair (x1 = element j, x2 = element j + d/2) by the
// angle with cosine cs and sine sn.  Contraction is off, so every kernel that
// rotates produces the same bits.
__device__ __forceinline__ void rope_pair(float x1, float x2, float cs, float sn, float& y1, float& y2) {
#pragma clang fp contract(off)
  y1 = x1 * cs - x2 * sn;
  y2 = x2 * cs + x1 * sn;
}

// Low / high bf16 of a packed pair as float.
__device__ __forceinline__ float lo_bf16(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element storage type helpers: T is float or bf16_t.
// Element (row, col) of a bf16 activation matrix: row-major with row stride
// ld when slab_rows == 0; otherwise K-slab-major, the layout of the
// projection weights: each 32-wide column slab is a contiguous [slab_rows][32]
// block, so that a GEMM's load of 16 rows of one slab reads 1 KB contiguous.
__device__ __forceinline__ long act_idx(int row, int col, int ld, int slab_rows) {
  return slab_rows ? ((long)(col >> 5) * slab_rows + row) * 32 + (col & 31) : (long)row * ld + col;
}

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

// 16-byte chunks: E = Elem<T>::per16 values of a row as float, and back.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  __device__ static __forceinline__ void load(const float* p, float* v) {
    const f32x4_t a = *(const f32x4_t*)p;
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  }
  __device__ static __forceinline__ void store(float* p, const float* v) {
    *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]};
  }
};
template <> struct Chunk<bf16_t> {
  __device__ static __forceinline__ void load(const bf16_t* p, float* v) {
    const u32x4_t a = *(const u32x4_t*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = a[i];
      v[2 * i] = lo_bf16(w);
      v[2 * i + 1] = hi_bf16(w);
    }
  }
  __device__ static __forceinline__ void store(bf16_t* p, const float* v) {
    *(u32x4_t*)p = u32x4_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                           pack_bf16(v[6], v[7])};
  }
};

constexpr int kMaxSplits = 8;  // split-K slices a consumer sums

// Sum of S fp32 slices (slice_stride floats apart) at one 16-byte position,
// in slice order, every load issued before the first add.
template <int S>
__device__ __forceinline__ f32x4_t slice_sum4_n(const float* p, long slice_stride) {
  f32x4_t v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) v[s] = __builtin_nontemporal_load((const f32x4_t*)(p + s * slice_stride));
  f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < S; ++s) a += v[s];
  return a;
}

// The same for a runtime count 1..8 (a uniform branch to straight-line code;
// predicated loads would wait for each load in turn).
__device__ __forceinline__ f32x4_t slice_sum4(const float* p, long slice_stride, int splits) {
  switch (splits) {
    case 1: return slice_sum4_n<1>(p, slice_stride);
    case 2: return slice_sum4_n<2>(p, slice_stride);
    case 3: return slice_sum4_n<3>(p, slice_stride);
    case 4: return slice_sum4_n<4>(p, slice_stride);
    case 5: return slice_sum4_n<5>(p, slice_stride);
    case 6: return slice_sum4_n<6>(p, slice_stride);
    case 7: return slice_sum4_n<7>(p, slice_stride);
    default: return slice_sum4_n<kMaxSplits>(p, slice_stride);
  }
}

// Step rows t0 .. t0+31 form a prefill tile: one sequence (row_seq >= 0) at
// consecutive positions.  Lanes i and i + 32 both check row t0 + i; the
// result is uniform over the wavefront.  The caller ensures the 32 rows exist.
__device__ __forceinline__ bool prefill_tile(const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
                                             int t0, int lane) {
  const int i = lane & 31;
  const int s0 = row_seq[t0], p0 = row_pos[t0];
  const bool ok = s0 >= 0 && row_seq[t0 + i] == s0 && row_pos[t0 + i] == p0 + i;
  return __all(ok);
}

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
