// Paged grouped-query decode attention for gfx950 (vector ALU; HBM-bound).
//
// What it computes (nanoserve notes, changes table: GQA with no expanded K/V
// copy, paged cache through block tables; NanoFlow review, operator table:
// decode attention is the memory-bound class): for each row (a query at
// position pos of a sequence), each query head h attends with scale 1/sqrt(d)
// over keys 0..pos of its sequence, reading KV head h / G.
//
// Design (MI355X-first):
//  * one workgroup of 1 or 4 wavefronts per work item (row, KV head,
//    partition of the context): 4 when there are few items (small batches),
//    1 when items alone fill the chip; the wavefronts take interleaved
//    64-token passes and each
//    K/V block of the KV head is streamed exactly once for all G query heads
//    of the group, so the HBM traffic is the cache bytes themselves;
//  * QK: lane = token (64 tokens = 4 blocks per pass).  The K cache stores
//    each block as 16-byte chunks interleaved over its 16 tokens, so for every
//    chunk the 16 lanes of a block read 256 contiguous bytes.  The q values
//    are wavefront-uniform (all lanes need the same q), loaded through the
//    scalar cache, and each K pair feeds v_dot2_f32_bf16 for every head of
//    the group;
//  * online softmax in the log2 domain with wavefront max/sum reductions;
//  * PV: lane = (token lane j, 16-byte chunk c of the head dim): each lane
//    accumulates G x E outputs of its chunk over the tokens j, j+TL, ...;
//    V rows are read 16 bytes per lane, a whole block row per 64/TL lanes;
//  * all K and V loads of a pass are issued before any arithmetic, so each
//    wavefront keeps 2 x 64 tokens of KV in flight;
//  * the wavefronts of a workgroup merge their (max, sum, accumulator)
//    triples in LDS; split context partitions (a multiple of 64 tokens, for
//    long contexts with few rows) write partials that a combine kernel merges
//    the same way.  A row that fits one partition writes its output directly.
#include "ns_kernels.h"

namespace ns {

namespace {

template <typename T, int D, int G>
struct AttnTraits {
  static constexpr int E = Elem<T>::per16;  // elements per 16-byte chunk
  static constexpr int NCH = D / E;         // chunks per head row
  static constexpr int TL = 64 / NCH;       // token lanes in the PV layout
  static_assert(64 % NCH == 0, "head row must split into a power-of-two number of chunks <= 64");
  static_assert(TL <= 16, "PV token lanes must stay inside one block per iteration");
};

__device__ __forceinline__ float dot2(uint32_t q, uint32_t k, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q), __builtin_bit_cast(bf16x2_t, k), acc,
                                         false);
}
// The vector elements are copied to scalars before the bit casts: with this
// compiler, bit-casting q.y etc. of a vector read through a reference
// silently yields q.x.
__device__ __forceinline__ float dot_chunk(const u32x4_t& q, const u32x4_t& k, float acc, bf16_t) {
  const uint32_t q0 = q.x, q1 = q.y, q2 = q.z, q3 = q.w;
  const uint32_t k0 = k.x, k1 = k.y, k2 = k.z, k3 = k.w;
  acc = dot2(q0, k0, acc);
  acc = dot2(q1, k1, acc);
  acc = dot2(q2, k2, acc);
  acc = dot2(q3, k3, acc);
  return acc;
}
__device__ __forceinline__ float dot_chunk(const u32x4_t& q, const u32x4_t& k, float acc, float) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Unpack one 16-byte chunk into floats.
__device__ __forceinline__ void unpack_chunk(const u32x4_t& v, float* f, bf16_t) {
  f[0] = lo_bf16(v.x); f[1] = hi_bf16(v.x);
  f[2] = lo_bf16(v.y); f[3] = hi_bf16(v.y);
  f[4] = lo_bf16(v.z); f[5] = hi_bf16(v.z);
  f[6] = lo_bf16(v.w); f[7] = hi_bf16(v.w);
}
__device__ __forceinline__ void unpack_chunk(const u32x4_t& v, float* f, float) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

}  // namespace

// Pointers are separate __restrict__ parameters (not struct members) so the
// compiler can prove the wavefront-uniform q and block-table reads are never
// clobbered and serve them from the scalar cache.
//
// A workgroup of NWAVE wavefronts owns one work item (row, KV head, context
// partition); wavefront w takes the 64-token passes w, w + NWAVE, ... of the
// partition with its own running max, sums and accumulators, and the
// wavefronts' results are merged in LDS in wavefront order (deterministic).
template <typename T, int D, int G, int NWAVE>
__global__ void __launch_bounds__(64 * NWAVE) attn_decode_kernel(
    const T* __restrict__ qatt, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ row_bseq, const int32_t* __restrict__ row_pos, const int32_t* __restrict__ btab,
    T* __restrict__ out, float* __restrict__ part_acc, float* __restrict__ part_ml, int maxb, int row0, int n_rows,
    int nq, int nkv, int P, int n_parts, float scale_log2, const int32_t* __restrict__ skip_seq) {
  using Tr = AttnTraits<T, D, G>;
  constexpr int E = Tr::E, NCH = Tr::NCH, TL = Tr::TL;
  constexpr long HEAD_BLK = 16L * D;  // elements of one (block, KV head)
  // A pass rescales only when some score exceeds the running max by more
  // than this (log2 units): exp2 of at most 2^8 cannot overflow, and the
  // final division by the summed weights cancels the common factor.
  constexpr float kSlack = 8.0f;
  __shared__ float plds[NWAVE][64][8];  // a wavefront's probabilities, token x head
  __shared__ float macc[NWAVE][G][D];   // per-wavefront accumulators for the merge
  __shared__ float mml[NWAVE][G][2];    // per-wavefront shift and sum

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pj = lane / NCH, pc = lane % NCH;  // PV layout
  const int total = n_rows * nkv * n_parts;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int part = w % n_parts;
    const int rest = w / n_parts;
    const int g = rest % nkv;
    const int t = row0 + rest / nkv;
    if (skip_seq) {  // rows of prefill tiles belong to the prefill kernel
      const int t0 = row0 + ((t - row0) & ~31);
      if (t0 + 32 <= row0 + n_rows && prefill_tile(skip_seq, row_pos, t0, lane)) continue;
    }
    // The row's block-table row: btab[row_bseq[t]], or row t itself when
    // the table is laid out per row (row_bseq null) -- one dependent load
    // fewer before the K/V loads.  Padding rows have no blocks.
    const int32_t* __restrict__ bt;
    bool pad;
    if (row_bseq) {
      const int bs = row_bseq[t];
      pad = bs < 0;
      bt = btab + (long)(pad ? 0 : bs) * maxb;
    } else {
      bt = btab + (long)t * maxb;
      pad = bt[0] < 0;
    }
    T* outp = out + (long)t * nq * D + (long)g * G * D;
    if (pad) {  // padding row: zero output
      if (part == 0)
        for (int i = threadIdx.x; i < G * D; i += 64 * NWAVE) outp[i] = T(0);
      continue;
    }
    const int ctx = row_pos[t] + 1;
    const int start = part * P;
    if (start >= ctx) continue;
    const int end = min(start + P, ctx);
    const int nparts_row = (ctx + P - 1) / P;
    const u32x4_t* __restrict__ q4 = (const u32x4_t*)(qatt + ((long)t * nkv + g) * NCH * G * E);

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -1e30f;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }

    for (int c0 = start + 64 * wave; c0 < end; c0 += 64 * NWAVE) {
      // Block ids of this pass's 4 blocks (wavefront-uniform).
      int blk[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) blk[b] = (c0 + 16 * b < end) ? bt[(c0 >> 4) + b] : bt[c0 >> 4];
      // Issue every K and V load of the pass.  Lanes past the context end
      // read the pass's first token instead (a written slot) and are masked.
      const int tq = c0 + lane;
      const bool valid = tq < end;
      const int tqs = valid ? lane : 0;
      const int kb = blk[tqs >> 4];
      const T* kp = kc + ((long)kb * nkv + g) * HEAD_BLK + (long)(tqs & 15) * E;
      u32x4_t kr[NCH];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) kr[ch] = *(const u32x4_t*)(kp + (long)ch * 16 * E);
      u32x4_t vr[NCH];
#pragma unroll
      for (int it = 0; it < NCH; ++it) {
        const int tl = it * TL + pj;  // token of this lane in iteration it
        const int tls = (c0 + tl < end) ? tl : 0;
        const int vb = blk[(it * TL) >> 4];
        vr[it] = *(const u32x4_t*)(vc + ((long)vb * nkv + g) * HEAD_BLK + (long)(tls & 15) * D + pc * E);
      }

      // QK: lane = token.  q (G x d values, up to 2 KB) is re-read from the
      // scalar cache every pass: the opaque zero keeps the compiler from
      // hoisting all of it out of the pass loop into (spilled) SGPRs.
      int zero = 0;
      asm volatile("" : "+s"(zero));
      const u32x4_t* __restrict__ qp = q4 + zero;
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = dot_chunk(qp[ch * G + h], kr[ch], s[h], T());
      }

      // Online softmax (log2 domain) with a wavefront-uniform shift m: the
      // wavefront max is taken (and the running sums rescaled) only when a
      // score exceeds m by more than kSlack.
      float sh[G], pr[G];
      float excess = -INFINITY;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sh[h] = valid ? s[h] * scale_log2 : -INFINITY;
        excess = fmaxf(excess, sh[h] - m[h]);
      }
      if (__ballot(excess > kSlack)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mn = fmaxf(m[h], wave_max(sh[h]));
          const float alpha = exp2f(m[h] - mn);
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
          m[h] = mn;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pr[h] = exp2f(sh[h] - m[h]);
        l[h] += pr[h];
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) plds[wave][lane][h] = h < G ? pr[h] : 0.f;
      // the probabilities cross lanes within the wavefront only
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // PV: lane = (token lane pj, chunk pc).
#pragma unroll
      for (int it = 0; it < NCH; ++it) {
        const int tl = it * TL + pj;
        const f32x4_t p0 = *(const f32x4_t*)&plds[wave][tl][0];
        const f32x4_t p1 = *(const f32x4_t*)&plds[wave][tl][4];
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        float vf[E];
        unpack_chunk(vr[it], vf, T());
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pv[h], vf[e], acc[h][e]);
      }
      // the next pass overwrites this wavefront's probabilities
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // Finish the wavefront: sum the per-lane softmax denominators and the PV
    // partials of the token lanes.
    float lsum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lsum[h] = wave_sum(l[h]);
#pragma unroll
    for (int off = NCH; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);

    // Merge the wavefronts: M = max m_w, L = sum l_w 2^(m_w - M),
    // acc = sum acc_w 2^(m_w - M), in wavefront order.  A wavefront that had
    // no pass contributes m = -1e30, l = 0, acc = 0 (weight 0).
    if (lane < NCH) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) macc[wave][h][pc * E + e] = acc[h][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mml[wave][h][0] = m[h];
        mml[wave][h][1] = lsum[h];
      }
    }
    __syncthreads();
    const long item = ((long)t * nkv + g) * n_parts + part;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * NWAVE) {
      const int h = idx / D, dd = idx % D;
      float M = mml[0][h][0];
#pragma unroll
      for (int v = 1; v < NWAVE; ++v) M = fmaxf(M, mml[v][h][0]);
      float L = 0.f, o = 0.f;
#pragma unroll
      for (int v = 0; v < NWAVE; ++v) {
        const float wgt = exp2f(mml[v][h][0] - M);
        L += mml[v][h][1] * wgt;
        o += macc[v][h][dd] * wgt;
      }
      if (nparts_row == 1) {
        Elem<T>::store(outp, (long)h * D + dd, o / L);
      } else {
        part_acc[item * G * D + idx] = o;
        if (dd == 0) {
          part_ml[(item * G + h) * 2] = M;
          part_ml[(item * G + h) * 2 + 1] = L;
        }
      }
    }
    __syncthreads();  // the LDS is reused by the next work item
  }
}

// Merge the partitions of rows whose context spans more than one.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  const int t = a.row0 + blockIdx.x / a.nkv;
  const int g = blockIdx.x % a.nkv;
  if (a.row_seq) {  // set only when the prefill kernel takes the prefill tiles
    const int t0 = a.row0 + ((t - a.row0) & ~31);
    if (t0 + 32 <= a.row0 + a.n_rows && prefill_tile(a.row_seq, a.row_pos, t0, threadIdx.x & 63)) return;
  }
  if ((a.row_bseq ? a.row_bseq[t] : a.btab[(long)t * a.maxb]) < 0) return;
  const int ctx = a.row_pos[t] + 1;
  const int np = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  const long item0 = ((long)t * a.nkv + g) * a.n_parts;
  T* outp = (T*)a.out + (long)t * a.nq * D + (long)g * G * D;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_ml[(item0 + p) * G * 2 + 2 * h]);
    float L = 0.f, o = 0.f;
    for (int p = 0; p < np; ++p) {
      const float wgt = exp2f(a.part_ml[(item0 + p) * G * 2 + 2 * h] - M);
      L += a.part_ml[(item0 + p) * G * 2 + 2 * h + 1] * wgt;
      o += a.part_acc[(item0 + p) * G * D + idx] * wgt;
    }
    Elem<T>::store(outp, idx, o / L);
  }
}

template <typename T, int D, int G>
static void launch_attn_t(const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  if (!a.row_seq || !prefill_supported(a.dtype, D, G) || a.n_rows < 32) a.row_seq = nullptr;  // no prefill tiles
  const long total = (long)a.n_rows * a.nkv * a.n_parts;
  if (total <= 0) return;
  long grid = total;
  if (a.wg_cap > 0 && grid > a.wg_cap) grid = a.wg_cap;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
#define NS_ATTN_LAUNCH(NW)                                                                                         \
  hipLaunchKernelGGL((attn_decode_kernel<T, D, G, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st,               \
                     (const T*)a.q_att, (const T*)a.kc, (const T*)a.vc, a.row_bseq, a.row_pos, a.btab, (T*)a.out, \
                     a.part_acc, a.part_ml, a.maxb, a.row0, a.n_rows, a.nq, a.nkv, a.part_tokens, a.n_parts,      \
                     scale_log2, a.row_seq)
  if (a.waves == 1) NS_ATTN_LAUNCH(1);
  else NS_ATTN_LAUNCH(4);
#undef NS_ATTN_LAUNCH
  if (a.n_parts > 1)
    hipLaunchKernelGGL((attn_combine_kernel<T, D, G>), dim3((unsigned)(a.n_rows * a.nkv)), dim3(256), 0, st, a);
  if (a.row_seq) launch_attention_prefill(a, st);
}

#define NS_ATTN_CASES(X)                                                                               \
  X(bf16_t, 64, 1) X(bf16_t, 64, 2) X(bf16_t, 64, 4) X(bf16_t, 64, 7) X(bf16_t, 64, 8)                 \
  X(bf16_t, 128, 1) X(bf16_t, 128, 2) X(bf16_t, 128, 4) X(bf16_t, 128, 7) X(bf16_t, 128, 8)            \
  X(bf16_t, 32, 4) X(bf16_t, 32, 8) X(float, 32, 1) X(float, 32, 2) X(float, 32, 4) X(float, 32, 8)    \
  X(float, 64, 4) X(float, 64, 7) X(float, 64, 8) X(float, 128, 4) X(float, 128, 8)

int attention_supported(int dtype, int d, int G) {
#define X(TY, DD, GG) \
  if ((dtype == NS_DT_BF16) == (sizeof(TY) == 2) && d == DD && G == GG) return 1;
  NS_ATTN_CASES(X)
#undef X
  return 0;
}

void launch_attention(const AttnArgs& a, hipStream_t st) {
  const int G = a.nq / a.nkv;
#define X(TY, DD, GG)                                                               \
  if ((a.dtype == NS_DT_BF16) == (sizeof(TY) == 2) && a.d == DD && G == GG) { \
    launch_attn_t<TY, DD, GG>(a, st);                                               \
    return;                                                                         \
  }
  NS_ATTN_CASES(X)
#undef X
}

}  // namespace ns
