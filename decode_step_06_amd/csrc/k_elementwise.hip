// Row-wise kernels of the decode step: embedding gather, RoPE table (once per
// step), RMSNorm, RoPE + paged KV-cache write, and KV scatter/gather helpers.
//
// These are the "negligible" class of the NanoFlow review's operator table
// (section "Four resource classes, one serialized queue"): each moves a few
// bytes per row, so the design goal is one launch per use and coalesced
// row access, not arithmetic throughput.
#include <climits>

#include "ns_kernels.h"

namespace ns {

// ---------------------------------------------------------------- embedding
// x[t][:] = E[token[t]][:] widened to fp32 (the residual stream is fp32).
template <typename T>
__global__ void __launch_bounds__(256) embed_kernel(const T* __restrict__ E, const int32_t* __restrict__ tok,
                                                    float* __restrict__ x, int H, int V) {
  const int t = blockIdx.x;
  int id = tok[t];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const T* src = E + (long)id * H;
  float* dst = x + (long)t * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) dst[i] = Elem<T>::load(src, i);
}

__global__ void __launch_bounds__(256) copy_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                        long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// ---------------------------------------------------------------- RoPE table
// cos/sin[t][j] of angle pos[t] * base^(-2j/d), built once per step and read
// by every layer (nanoserve notes, changes table: "RoPE cos/sin computed once
// per step").  Angles and sin/cos in fp64, stored fp32.
__global__ void __launch_bounds__(256) rope_table_kernel(const int32_t* __restrict__ pos, float* __restrict__ cosb,
                                                         float* __restrict__ sinb, int n_rows, int half,
                                                         double log2_base) {
  const long n = (long)n_rows * half;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int t = (int)(i / half), j = (int)(i % half);
    const double inv_freq = exp2(-2.0 * j / (2.0 * half) * log2_base);
    const double a = (double)pos[t] * inv_freq;
    double s, c;
    sincos(a, &s, &c);
    cosb[i] = (float)c;
    sinb[i] = (float)s;
  }
}

// ---------------------------------------------------------------- RMSNorm
// h[t] = x[t] / sqrt(mean(x[t]^2) + eps) * g, one workgroup per row; the
// residual add that precedes it in the layer is fused into the producing
// projection's epilogue, so x already holds the updated residual stream.
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ x, const T* __restrict__ g,
                                                      T* __restrict__ h, int H, float eps, int hs) {
  const int t = blockIdx.x;
  const float* xr = x + (long)t * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) {
    const float v = xr[i];
    ss += v * v;
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256) Elem<T>::store(h, act_idx(t, i, H, hs), xr[i] * r * Elem<T>::load(g, i));
}

// The split-K residual add fused in front of the norm: x[t] += the slices
// of the previous projection (slice order), written back, then the norm.
// 16-byte chunks, CH per thread held in registers between the two passes.
// Every load of the row -- all S slices of all CH chunks, x and the norm
// weights -- is issued before the first add, so the row costs one memory
// round trip before the reduction (a chunk at a time, or the weights loaded
// after the reduction, would each add one).  NT threads per row: 256 up to
// 2048 elements, 1024 above.
template <typename T> struct Gain4;
template <> struct Gain4<float> {
  __device__ static __forceinline__ f32x4_t load(const float* p) { return *(const f32x4_t*)p; }
};
template <> struct Gain4<bf16_t> {
  __device__ static __forceinline__ f32x4_t load(const bf16_t* p) {
    const uint2 w = *(const uint2*)p;
    return f32x4_t{lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y)};
  }
};

// Four consecutive outputs in one store (8 bytes of bf16, 16 of fp32); p is
// aligned to four elements.
template <typename T> struct Store4;
template <> struct Store4<float> {
  __device__ static __forceinline__ void store(float* p, f32x4_t v) { *(f32x4_t*)p = v; }
};
template <> struct Store4<bf16_t> {
  __device__ static __forceinline__ void store(bf16_t* p, f32x4_t v) {
    *(uint2*)p = uint2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
};

template <typename T, int CH, int NT, int S>
__device__ __forceinline__ void rmsnorm_reduce_row(float* __restrict__ xr, const float* __restrict__ pr,
                                                   long slice_stride, const T* __restrict__ g, T* __restrict__ h,
                                                   int t, int hs, int H, float eps) {
  const int H4 = H >> 2;
  f32x4_t p[CH][S], v[CH], gv[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < H4) {
#pragma unroll
      for (int s = 0; s < S; ++s)
        p[c][s] = __builtin_nontemporal_load((const f32x4_t*)(pr + 4 * i4 + s * slice_stride));
      v[c] = *(const f32x4_t*)(xr + 4 * i4);
      gv[c] = Gain4<T>::load(g + 4 * i4);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < H4) {
      f32x4_t add = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; ++s) add += p[c][s];
      v[c] += add;
      *(f32x4_t*)(xr + 4 * i4) = v[c];
      ss += v[c][0] * v[c][0] + v[c][1] * v[c][1] + v[c][2] * v[c][2] + v[c][3] * v[c][3];
    }
  }
  constexpr int NW = NT / 64;
  __shared__ float red[NW];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < H4) {
      // 4 consecutive columns from a multiple of 4: consecutive (and aligned
      // to 4) in either layout
      f32x4_t y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = v[c][e] * r * gv[c][e];
      Store4<T>::store(h + act_idx(t, 4 * i4, H, hs), y);
    }
  }
}

template <typename T, int CH, int NT>
__global__ void __launch_bounds__(NT) rmsnorm_reduce_kernel(float* __restrict__ x, const float* __restrict__ P,
                                                            long slice_stride, int splits, const T* __restrict__ g,
                                                            T* __restrict__ h, int H, float eps, int hs) {
  const int t = blockIdx.x;
  const long o = (long)t * H;
  switch (splits) {  // uniform: straight-line code for each slice count
    case 1: return rmsnorm_reduce_row<T, CH, NT, 1>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    case 2: return rmsnorm_reduce_row<T, CH, NT, 2>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    case 3: return rmsnorm_reduce_row<T, CH, NT, 3>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    case 4: return rmsnorm_reduce_row<T, CH, NT, 4>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    case 5: return rmsnorm_reduce_row<T, CH, NT, 5>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    case 6: return rmsnorm_reduce_row<T, CH, NT, 6>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    case 7: return rmsnorm_reduce_row<T, CH, NT, 7>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
    default: return rmsnorm_reduce_row<T, CH, NT, kMaxSplits>(x + o, P + o, slice_stride, g, h, t, hs, H, eps);
  }
}

// Rows of more than 8192 elements: a chunk's slices at a time (all of a
// row's would not fit the registers of 1024 threads).
template <typename T, int CH, int NT>
__global__ void __launch_bounds__(NT) rmsnorm_reduce_wide_kernel(float* __restrict__ x, const float* __restrict__ P,
                                                                 long slice_stride, int splits,
                                                                 const T* __restrict__ g, T* __restrict__ h, int H,
                                                                 float eps, int hs) {
  const int t = blockIdx.x, H4 = H >> 2;
  float* xr = x + (long)t * H;
  const float* pr = P + (long)t * H;
  f32x4_t v[CH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < H4) {
      const f32x4_t add = slice_sum4(pr + 4 * i4, slice_stride, splits);
      f32x4_t xv = *(const f32x4_t*)(xr + 4 * i4);
      xv += add;
      *(f32x4_t*)(xr + 4 * i4) = xv;
      v[c] = xv;
      ss += xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3];
    }
  }
  constexpr int NW = NT / 64;
  __shared__ float red[NW];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < H4) {
      const long o = act_idx(t, 4 * i4, H, hs);
#pragma unroll
      for (int e = 0; e < 4; ++e) Elem<T>::store(h, o + e, v[c][e] * r * Elem<T>::load(g, 4 * i4 + e));
    }
  }
}

// Any H: one element at a time.
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_reduce_any_kernel(float* __restrict__ x, const float* __restrict__ P,
                                                                 long slice_stride, int splits,
                                                                 const T* __restrict__ g, T* __restrict__ h, int H,
                                                                 float eps, int hs) {
  const int t = blockIdx.x;
  float* xr = x + (long)t * H;
  const float* pr = P + (long)t * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) {
    float v = xr[i];
    float add = 0.f;
    for (int sp = 0; sp < splits; ++sp) add += pr[sp * slice_stride + i];
    v += add;
    xr[i] = v;
    ss += v * v;
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256) Elem<T>::store(h, act_idx(t, i, H, hs), xr[i] * r * Elem<T>::load(g, i));
}

__global__ void __launch_bounds__(256) reduce_rows_kernel(const float* __restrict__ x, const float* __restrict__ P,
                                                          long slice_stride, int splits, float* __restrict__ out,
                                                          int H) {
  const int t = blockIdx.x;
  if ((H & 3) == 0) {
    for (int i4 = threadIdx.x; i4 < (H >> 2); i4 += 256) {
      const long o = (long)t * H + 4 * i4;
      *(f32x4_t*)(out + o) = *(const f32x4_t*)(x + o) + slice_sum4(P + o, slice_stride, splits);
    }
    return;
  }
  for (int i = threadIdx.x; i < H; i += 256) {
    float add = 0.f;
    for (int sp = 0; sp < splits; ++sp) add += P[sp * slice_stride + (long)t * H + i];
    out[(long)t * H + i] = x[(long)t * H + i] + add;
  }
}

// ---------------------------------------------------------------- step prologue
// One workgroup per row does everything the step needs before layer 0's
// projections: the embedding gather (models with a vocabulary; otherwise x
// already holds the hidden input), this row's RoPE cos/sin (the table every
// layer reads, built once per step) and layer 0's RMSNorm.  Three launches
// become one.  A token id outside [0, V) (possible only for ids fed from
// device memory) gathers the nearest valid row and adds 1 to *bad_tok.
template <typename T>
__global__ void __launch_bounds__(256) step_prologue_kernel(const T* __restrict__ E, const int32_t* __restrict__ tok,
                                                            float* __restrict__ x, const int32_t* __restrict__ pos,
                                                            float* __restrict__ cosb, float* __restrict__ sinb,
                                                            const T* __restrict__ g0, T* __restrict__ h, int H, int V,
                                                            int half, double log2_base, float eps,
                                                            int32_t* __restrict__ bad_tok, int hs) {
  const int t = blockIdx.x;
  float* xr = x + (long)t * H;
  float ss = 0.f;
  if (E) {
    int id = tok[t];
    if (id < 0 || id >= V) {
      if (threadIdx.x == 0 && bad_tok) atomicAdd(bad_tok, 1);
      id = id < 0 ? 0 : V - 1;
    }
    const T* src = E + (long)id * H;
    for (int i = threadIdx.x; i < H; i += 256) {
      const float v = Elem<T>::load(src, i);
      xr[i] = v;
      ss += v * v;
    }
  } else {
    for (int i = threadIdx.x; i < H; i += 256) {
      const float v = xr[i];
      ss += v * v;
    }
  }
  const double p = (double)pos[t];
  for (int j = threadIdx.x; j < half; j += 256) {
    const double a = p * exp2(-2.0 * j / (2.0 * half) * log2_base);
    double sn, cs;
    sincos(a, &sn, &cs);
    cosb[(long)t * half + j] = (float)cs;
    sinb[(long)t * half + j] = (float)sn;
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256) Elem<T>::store(h, act_idx(t, i, H, hs), xr[i] * r * Elem<T>::load(g0, i));
}

// ---------------------------------------------------------------- greedy sampling
// Row argmax (lowest index among equal maxima; NaN never wins).  One
// workgroup of 1024 threads per row; each thread keeps its best (value,
// index) over a strided share of the row -- eight 16-byte loads at a time
// when the row is made of aligned 16-byte chunks, else four 4-byte loads --
// then the pairs meet in wavefront shuffles and LDS.
__device__ __forceinline__ bool argmax_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ void __launch_bounds__(1024) argmax_rows_kernel(const float* __restrict__ logits, int V,
                                                           int32_t* __restrict__ out) {
  const float* row = logits + (long)blockIdx.x * V;
  float bv = -INFINITY;
  int bi = INT_MAX;
  int i = threadIdx.x;
  // The winner is the greatest (value, lower index) pair under
  // argmax_better, whatever order the entries are visited in.  Rows of whole
  // 16-byte chunks: eight 16-byte loads in flight per thread.
  if ((V & 3) == 0 && (((uintptr_t)row) & 15) == 0) {
    const f32x4_t* row4 = (const f32x4_t*)row;
    const int V4 = V >> 2;
    int j = threadIdx.x;
    for (; j + 7 * 1024 < V4; j += 8 * 1024) {
      f32x4_t c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = row4[j + k * 1024];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * (j + k * 1024) + e;
          if (argmax_better(c[k][e], idx, bv, bi)) bv = c[k][e], bi = idx;
        }
    }
    for (; j < V4; j += 1024) {
      const f32x4_t c = row4[j];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (argmax_better(c[e], 4 * j + e, bv, bi)) bv = c[e], bi = 4 * j + e;
    }
    i = V;  // nothing left for the scalar loops
  }
  for (; i + 3 * 1024 < V; i += 4 * 1024) {
    const float v0 = row[i], v1 = row[i + 1024], v2 = row[i + 2048], v3 = row[i + 3072];
    if (argmax_better(v0, i, bv, bi)) bv = v0, bi = i;
    if (argmax_better(v1, i + 1024, bv, bi)) bv = v1, bi = i + 1024;
    if (argmax_better(v2, i + 2048, bv, bi)) bv = v2, bi = i + 2048;
    if (argmax_better(v3, i + 3072, bv, bi)) bv = v3, bi = i + 3072;
  }
  for (; i < V; i += 1024)
    if (argmax_better(row[i], i, bv, bi)) bv = row[i], bi = i;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (argmax_better(ov, oi, bv, bi)) bv = ov, bi = oi;
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 16; ++k)
      if (argmax_better(sv[k], si[k], bv, bi)) bv = sv[k], bi = si[k];
    out[blockIdx.x] = bi == INT_MAX ? 0 : bi;
  }
}

void launch_argmax_rows(const float* logits, int n_rows, int V, int32_t* out, hipStream_t st) {
  if (n_rows <= 0) return;
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(n_rows), dim3(1024), 0, st, logits, V, out);
}

// ---------------------------------------------------------------- RoPE + KV write
// Element j of head g's V at slot tok of block blk: fp32 caches keep token
// rows ([blk][nkv][16][d]); bf16 caches store each block transposed
// ([blk][nkv][d][16]) for the matrix-core attention kernel.
template <typename T>
__device__ __forceinline__ long v_index(long blk, int g, int tok, int j, int nkv, int d) {
  if constexpr (sizeof(T) == 2) return ((blk * nkv + g) * d + j) * (long)NS_BLOCK + tok;
  return ((blk * nkv + g) * NS_BLOCK + tok) * (long)d + j;
}

// From the QKV projection (fp32 [T, (nq + 2 nkv) d]) for one row per
// workgroup: rotate-half RoPE on q and k with the step's table, store q in
// the attention layout [T][nkv][d/E][G][E] (the G query heads of one KV head
// chunk by chunk, so attention reads them as one uniform block), and write
// the rotated k and the v into the paged cache at the row's slot (padding
// rows, slot < 0, write no K/V).
//
// The row is first staged in LDS -- summed in slice order when the projection
// arrives as split-K slices -- together with its cos/sin, in one round of
// loads: a thread's CPT chunks of every slice are all in flight before the
// first add (CPT = 0: rows too wide for that, a chunk's slices at a time).
// Then each thread produces whole 16-byte chunks: E consecutive elements j of
// one head and, for q and k, their rotation partners j + d/2.
template <int S, int CPT, int NT>
__device__ __forceinline__ void stage_slices(const float* __restrict__ row, long slice_stride, float* rowbuf,
                                             int n4) {
  f32x4_t p[CPT][S];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < n4) {
#pragma unroll
      for (int s = 0; s < S; ++s)
        p[c][s] = __builtin_nontemporal_load((const f32x4_t*)(row + 4 * i4 + s * slice_stride));
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i4 = threadIdx.x + c * NT;
    if (i4 < n4) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; ++s) a += p[c][s];
      *(f32x4_t*)(rowbuf + 4 * i4) = a;
    }
  }
}

template <int CPT, int NT>
__device__ __forceinline__ void stage_row(const float* __restrict__ row, long slice_stride, int splits, float* rowbuf,
                                          int n4) {
  if constexpr (CPT == 0) {
    for (int i4 = threadIdx.x; i4 < n4; i4 += NT)
      *(f32x4_t*)(rowbuf + 4 * i4) = slice_sum4(row + 4 * i4, slice_stride, splits);
  } else {
    switch (splits) {  // uniform
      case 1: return stage_slices<1, CPT, NT>(row, slice_stride, rowbuf, n4);
      case 2: return stage_slices<2, CPT, NT>(row, slice_stride, rowbuf, n4);
      case 3: return stage_slices<3, CPT, NT>(row, slice_stride, rowbuf, n4);
      case 4: return stage_slices<4, CPT, NT>(row, slice_stride, rowbuf, n4);
      case 5: return stage_slices<5, CPT, NT>(row, slice_stride, rowbuf, n4);
      case 6: return stage_slices<6, CPT, NT>(row, slice_stride, rowbuf, n4);
      case 7: return stage_slices<7, CPT, NT>(row, slice_stride, rowbuf, n4);
      default: return stage_slices<kMaxSplits, CPT, NT>(row, slice_stride, rowbuf, n4);
    }
  }
}

template <typename T, int NT, int CPT>
__global__ void __launch_bounds__(NT) rope_kv_kernel(const float* __restrict__ qkv, long slice_stride, int splits,
                                                      const float* __restrict__ cosb,
                                                      const float* __restrict__ sinb, const int32_t* __restrict__ slot,
                                                      T* __restrict__ q_att, T* __restrict__ kc, T* __restrict__ vc,
                                                      int nq, int nkv, int d) {
  constexpr int E = Elem<T>::per16;
  extern __shared__ __attribute__((aligned(16))) float rowbuf[];
  const int t = blockIdx.x;
  const int half = d >> 1, G = nq / nkv, nch = d / E, hch = half / E;
  const int width = (nq + 2 * nkv) * d;
  const float* row = qkv + (long)t * width;
  const int s = slot[t];
  // the row's cos/sin after the row in LDS (half / 4 chunks each)
  float* cr = rowbuf + width;
  float* sr = cr + half;
  f32x4_t cv, sv;
  const bool trig = (int)threadIdx.x < (half >> 2);
  if (trig) {
    cv = *(const f32x4_t*)(cosb + (long)t * half + 4 * threadIdx.x);
    sv = *(const f32x4_t*)(sinb + (long)t * half + 4 * threadIdx.x);
  }
  stage_row<CPT, NT>(row, slice_stride, splits, rowbuf, width >> 2);
  if (trig) {
    *(f32x4_t*)(cr + 4 * threadIdx.x) = cv;
    *(f32x4_t*)(sr + 4 * threadIdx.x) = sv;
  }
  __syncthreads();
  const long blk = s >= 0 ? (long)(s / NS_BLOCK) : 0;
  const int tok = s >= 0 ? s % NS_BLOCK : 0;
  const int n_q = nq * hch, n_k = s >= 0 ? nkv * hch : 0, n_v = s >= 0 ? nkv * nch : 0;
  for (int it = threadIdx.x; it < n_q + n_k + n_v; it += NT) {
    if (it < n_q + n_k) {
      // rotate chunk c (elements j0..j0+E) of head hd with its partners
      const bool is_q = it < n_q;
      const int w = is_q ? it : it - n_q;
      const int hd = w / hch, c = w % hch, j0 = c * E;
      const float* src = rowbuf + (is_q ? 0 : nq * d) + hd * d;
      float y1[E], y2[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        rope_pair(src[j0 + e], src[j0 + half + e], cr[j0 + e], sr[j0 + e], y1[e], y2[e]);
      }
      if (is_q) {
        const int g = hd / G, hh = hd % G;
        T* base = q_att + ((long)t * nkv + g) * nch * G * E + (long)hh * E;
        Chunk<T>::store(base + (long)c * G * E, y1);
        Chunk<T>::store(base + (long)(c + hch) * G * E, y2);
      } else {
        T* base = kc + (blk * nkv + hd) * (long)nch * NS_BLOCK * E + (long)tok * E;
        Chunk<T>::store(base + (long)c * NS_BLOCK * E, y1);
        Chunk<T>::store(base + (long)(c + hch) * NS_BLOCK * E, y2);
      }
    } else {
      // v chunk c of KV head g into its token row
      const int w = it - n_q - n_k;
      const int g = w / nch, c = w % nch;
      float y[E];
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = rowbuf[(nq + nkv) * d + g * d + c * E + e];
      if constexpr (sizeof(T) == 2) {  // bf16: V^T within the block, one element per head-dim row
#pragma unroll
        for (int e = 0; e < E; ++e) Elem<T>::store(vc, v_index<T>(blk, g, tok, c * E + e, nkv, d), y[e]);
      } else {
        Chunk<T>::store(vc + v_index<T>(blk, g, tok, c * E, nkv, d), y);
      }
    }
  }
}

// ---------------------------------------------------------------- KV scatter / gather
// Logical [n, nkv, d] <-> physical cache layout (setting up or reading back
// cached context).
template <typename T>
__global__ void __launch_bounds__(256) kv_scatter_kernel(const int32_t* __restrict__ slots, const T* __restrict__ k,
                                                         const T* __restrict__ v, T* __restrict__ kc,
                                                         T* __restrict__ vc, int nkv, int d) {
  constexpr int E = Elem<T>::per16;
  const int i = blockIdx.x;
  const int s = slots[i];
  if (s < 0) return;
  const long blk = s / NS_BLOCK;
  const int tok = s % NS_BLOCK, nch = d / E;
  for (int e = threadIdx.x; e < nkv * d; e += 256) {
    const int g = e / d, j = e % d;
    kc[((blk * nkv + g) * nch + j / E) * (long)NS_BLOCK * E + (long)tok * E + j % E] = k[(long)i * nkv * d + e];
    vc[v_index<T>(blk, g, tok, j, nkv, d)] = v[(long)i * nkv * d + e];
  }
}

template <typename T>
__global__ void __launch_bounds__(256) kv_gather_kernel(const int32_t* __restrict__ slots, T* __restrict__ k,
                                                        T* __restrict__ v, const T* __restrict__ kc,
                                                        const T* __restrict__ vc, int nkv, int d) {
  constexpr int E = Elem<T>::per16;
  const int i = blockIdx.x;
  const int s = slots[i];
  const int nch = d / E;
  for (int e = threadIdx.x; e < nkv * d; e += 256) {
    if (s < 0) {
      k[(long)i * nkv * d + e] = T(0);
      v[(long)i * nkv * d + e] = T(0);
      continue;
    }
    const long blk = s / NS_BLOCK;
    const int tok = s % NS_BLOCK;
    const int g = e / d, j = e % d;
    k[(long)i * nkv * d + e] = kc[((blk * nkv + g) * nch + j / E) * (long)NS_BLOCK * E + (long)tok * E + j % E];
    v[(long)i * nkv * d + e] = vc[v_index<T>(blk, g, tok, j, nkv, d)];
  }
}

// ---------------------------------------------------------------- read ceiling
// Streams a buffer once: each lane reads 16-byte chunks (non-temporal) in a
// grid-stride loop and XORs them; each workgroup stores the XOR of its
// lanes.  Its rate is the HBM read rate a kernel can reach on this chip, the
// ceiling the attention's bytes per second are compared against.  One load
// in flight per lane over 2048 workgroups of 256 was the fastest of the
// shapes measured on MI355X (7.0 TB/s; 4 or 8 loads per round at 4096-16384
// workgroups 6.5-6.9 TB/s).
__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4_t* __restrict__ p, long n16,
                                                          uint32_t* __restrict__ sink) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const long stride = (long)gridDim.x * 256;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) r ^= __shfl_xor(r, o, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// ---------------------------------------------------------------- launchers
static inline int nblocks(long n, int per) {
  long b = (n + per - 1) / per;
  return (int)(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

void launch_embed(int dtype, const void* E, const int32_t* tok, float* x, int T, int H, int V, hipStream_t st) {
  if (dtype == NS_DT_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(T), dim3(256), 0, st, (const bf16_t*)E, tok, x, H, V);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)E, tok, x, H, V);
}

void launch_copy_rows(const float* src, float* dst, long n, hipStream_t st) {
  hipLaunchKernelGGL(copy_rows_kernel, dim3(nblocks(n, 1024)), dim3(256), 0, st, src, dst, n);
}

void launch_rope_table(const int32_t* pos, float* cosb, float* sinb, int T, int d, float base, hipStream_t st) {
  const int half = d / 2;
  hipLaunchKernelGGL(rope_table_kernel, dim3(nblocks((long)T * half, 256)), dim3(256), 0, st, pos, cosb, sinb, T,
                     half, log2((double)base));
}

void launch_step_prologue(int dtype, const void* E, const int32_t* tok, float* x, const int32_t* pos, float* cosb,
                          float* sinb, const void* g0, void* h, int T, int H, int V, int d, float base, float eps,
                          int32_t* bad_tok, hipStream_t st, int h_slab_rows) {
  if (T <= 0) return;
  const double lb = log2((double)base);
  if (dtype == NS_DT_BF16)
    hipLaunchKernelGGL(step_prologue_kernel<bf16_t>, dim3(T), dim3(256), 0, st, (const bf16_t*)E, tok, x, pos, cosb,
                       sinb, (const bf16_t*)g0, (bf16_t*)h, H, V, d / 2, lb, eps, bad_tok, h_slab_rows);
  else
    hipLaunchKernelGGL(step_prologue_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)E, tok, x, pos, cosb,
                       sinb, (const float*)g0, (float*)h, H, V, d / 2, lb, eps, bad_tok, 0);
}

void launch_rmsnorm(int dtype, const float* x, const void* g, void* h, int T, int H, float eps, hipStream_t st,
                    int h_slab_rows) {
  if (T <= 0) return;
  if (dtype == NS_DT_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(T), dim3(256), 0, st, x, (const bf16_t*)g, (bf16_t*)h, H, eps,
                       h_slab_rows);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(T), dim3(256), 0, st, x, (const float*)g, (float*)h, H, eps, 0);
}

void launch_read_stream(const void* src, long n16, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(kReadStreamGrid), dim3(256), 0, st, (const u32x4_t*)src, n16, sink);
}

void launch_rope_kv(int dtype, const float* qkv, long slice_stride, int splits, const float* cosb,
                    const float* sinb, const int32_t* slot, void* q_att, void* kc, void* vc, int T, int nq, int nkv,
                    int d, hipStream_t st) {
  if (T <= 0) return;
  // rows wider than 2048 floats take 1024 threads; a thread's chunks of
  // every slice are loaded in one round where they fit its registers
  const int width = (nq + 2 * nkv) * d;
  const size_t lds = (size_t)(width + d) * sizeof(float);  // the row, then its cos and sin
  const int nt = width > 2048 ? 1024 : 256;
  const int cpt = (width / 4 + nt - 1) / nt;
#define NS_ROPE_KV(TT, NT, CPT)                                                                                  \
  hipLaunchKernelGGL((rope_kv_kernel<TT, NT, CPT>), dim3(T), dim3(NT), lds, st, qkv, slice_stride, splits, cosb, \
                     sinb, slot, (TT*)q_att, (TT*)kc, (TT*)vc, nq, nkv, d)
  if (dtype == NS_DT_BF16) {
    if (nt == 1024) {
      if (cpt == 1) NS_ROPE_KV(bf16_t, 1024, 1);
      else if (cpt == 2) NS_ROPE_KV(bf16_t, 1024, 2);
      else if (cpt == 3) NS_ROPE_KV(bf16_t, 1024, 3);
      else NS_ROPE_KV(bf16_t, 1024, 0);
    } else {
      if (cpt == 1) NS_ROPE_KV(bf16_t, 256, 1);
      else NS_ROPE_KV(bf16_t, 256, 2);
    }
  } else {
    if (cpt == 1) NS_ROPE_KV(float, 256, 1);
    else NS_ROPE_KV(float, 256, 2);
  }
#undef NS_ROPE_KV
}

template <typename T>
static void run_rmsnorm_reduce(float* x, const float* P, long slice_stride, int splits, const T* g, T* h, int T_,
                               int H, float eps, hipStream_t st, int hs) {
  const int ch = (H / 4 + 255) / 256;
  // the one-round kernel reads the gains 4 at a time and holds a row's
  // slices in registers: rows of up to 8192 elements
  const bool aligned = ((uintptr_t)g % (4 * sizeof(T))) == 0;
  if (H % 4 != 0 || ch > 32)
    hipLaunchKernelGGL(rmsnorm_reduce_any_kernel<T>, dim3(T_), dim3(256), 0, st, x, P, slice_stride, splits, g, h,
                       H, eps, hs);
  else if (ch > 8 || !aligned)
    hipLaunchKernelGGL((rmsnorm_reduce_wide_kernel<T, 8, 1024>), dim3(T_), dim3(1024), 0, st, x, P, slice_stride,
                       splits, g, h, H, eps, hs);
  else if (ch == 1)
    hipLaunchKernelGGL((rmsnorm_reduce_kernel<T, 1, 256>), dim3(T_), dim3(256), 0, st, x, P, slice_stride, splits, g,
                       h, H, eps, hs);
  else if (ch == 2)
    hipLaunchKernelGGL((rmsnorm_reduce_kernel<T, 2, 256>), dim3(T_), dim3(256), 0, st, x, P, slice_stride, splits, g,
                       h, H, eps, hs);
  else if (ch <= 4)
    hipLaunchKernelGGL((rmsnorm_reduce_kernel<T, 1, 1024>), dim3(T_), dim3(1024), 0, st, x, P, slice_stride, splits,
                       g, h, H, eps, hs);
  else
    hipLaunchKernelGGL((rmsnorm_reduce_kernel<T, 2, 1024>), dim3(T_), dim3(1024), 0, st, x, P, slice_stride, splits,
                       g, h, H, eps, hs);
}

void launch_rmsnorm_reduce(int dtype, float* x, const float* P, long slice_stride, int splits, const void* g,
                           void* h, int T, int H, float eps, hipStream_t st, int h_slab_rows) {
  if (T <= 0) return;
  if (dtype == NS_DT_BF16)
    run_rmsnorm_reduce<bf16_t>(x, P, slice_stride, splits, (const bf16_t*)g, (bf16_t*)h, T, H, eps, st, h_slab_rows);
  else
    run_rmsnorm_reduce<float>(x, P, slice_stride, splits, (const float*)g, (float*)h, T, H, eps, st, 0);
}

void launch_reduce_rows(const float* x, const float* P, long slice_stride, int splits, float* out, int T, int H,
                        hipStream_t st) {
  if (T <= 0) return;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3(T), dim3(256), 0, st, x, P, slice_stride, splits, out, H);
}

void launch_kv_scatter(int dtype, const int32_t* slots, const void* k, const void* v, void* kc, void* vc, int n,
                       int nkv, int d, hipStream_t st) {
  if (n <= 0) return;
  if (dtype == NS_DT_BF16)
    hipLaunchKernelGGL(kv_scatter_kernel<bf16_t>, dim3(n), dim3(256), 0, st, slots, (const bf16_t*)k,
                       (const bf16_t*)v, (bf16_t*)kc, (bf16_t*)vc, nkv, d);
  else
    hipLaunchKernelGGL(kv_scatter_kernel<float>, dim3(n), dim3(256), 0, st, slots, (const float*)k, (const float*)v,
                       (float*)kc, (float*)vc, nkv, d);
}

void launch_kv_gather(int dtype, const int32_t* slots, void* k, void* v, const void* kc, const void* vc, int n,
                      int nkv, int d, hipStream_t st) {
  if (n <= 0) return;
  if (dtype == NS_DT_BF16)
    hipLaunchKernelGGL(kv_gather_kernel<bf16_t>, dim3(n), dim3(256), 0, st, slots, (bf16_t*)k, (bf16_t*)v,
                       (const bf16_t*)kc, (const bf16_t*)vc, nkv, d);
  else
    hipLaunchKernelGGL(kv_gather_kernel<float>, dim3(n), dim3(256), 0, st, slots, (float*)k, (float*)v,
                       (const float*)kc, (const float*)vc, nkv, d);
}

}  // namespace ns
