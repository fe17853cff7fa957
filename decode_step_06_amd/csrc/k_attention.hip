// Paged grouped-query decode attention for gfx950 (HBM-bound).
//
// What it computes (nanoserve notes, changes table: GQA with no expanded K/V
// copy, paged cache through block tables; NanoFlow review, operator table:
// decode attention is the memory-bound class): for each row (a query at
// position pos of a sequence), each query head h attends with scale 1/sqrt(d)
// over keys 0..pos of its sequence, reading KV head h / G.
//
// Work decomposition (both kernels): a work item is (row, KV head, partition
// of the context); a workgroup of 1 or 4 wavefronts owns one: 4 when there
// are few items (small batches), 1 when items alone fill the chip.  The
// wavefronts take interleaved 64-token passes (4 blocks), each K/V block of
// the KV head is streamed exactly once for all G query heads of the group, so
// the HBM traffic is the cache bytes themselves.  The wavefronts of a
// workgroup merge their (max, sum, accumulator) triples in LDS; split context
// partitions (a multiple of 64 tokens, for long contexts with few rows) write
// partials that a combine kernel merges the same way.  A row that fits one
// partition writes its output directly.
//
// bf16 cache: matrix cores (attn_mfma_kernel).  V is stored transposed within
// each block ([block][nkv][d][16 tokens]), so the 8 consecutive tokens of one
// head-dim element that an MFMA operand needs are one 16-byte load.  Per pass:
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: four tiles of 16 tokens x 16
//    columns (the G query heads, zero-padded), d deep.  Row r of tile (s, u)
//    is token 32 s + 8 (r / 4) + 4 u + r % 4, which leaves lane l (column =
//    head l % 16) holding the scores of tokens 32 s + 8 (l / 16) + 0..7 of its
//    head: exactly its k slots of the PV step s, so P never crosses lanes;
//  * online softmax in the log2 domain, per head: one max and one sum over
//    the four lanes of a head (l, l ^ 16, l ^ 32, l ^ 48) per pass;
//  * O^T += V^T P^T on the same MFMA over 32 tokens per step, with P as a
//    pair of bf16 terms (the value rounded, then its residual: about 16
//    significant bits) and V^T fragments loaded straight from the cache.
//
// fp32 cache: vector ALU (attn_decode_kernel).  QK with lane = token (the K
// cache interleaves 16-byte chunks over a block's 16 tokens, so for every
// chunk the 16 lanes of a block read 256 contiguous bytes; q is wavefront-
// uniform, read through the scalar cache); PV with lane = (token lane j,
// 16-byte chunk c of the head dim) over V token rows; all K and V loads of a
// pass are issued before any arithmetic.
#include <type_traits>

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

__device__ __forceinline__ float dot_chunk(const u32x4_t& q, const u32x4_t& k, float acc, float) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Unpack one 16-byte chunk into floats.
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
    Elem<T>::store((T*)a.out, act_idx(t, g * G * D + idx, a.nq * D, a.out_slab_rows), o / L);
  }
}

// ------------------------------------------------------------------ bf16 on matrix cores
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Inputs of the fused RoPE prologue (see AttnArgs).
struct RopeIn {
  const float* qkv;
  long slice_stride;
  int splits;
  const float* cosb;
  const float* sinb;
  const int32_t* slot;
};

// Registers of one 64-token pass: K fragments of QK tile (s, u) for each
// k-step over d, and V^T fragments of PV step s for each 16-row d tile.
template <int D>
struct MfmaPass {
  bf16x8_t k[2][2][D / 32];
  u32x4_t v[D / 16][2];
};

// A 16-byte load, non-temporal when NT.
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Block ids of the pass's 4 blocks, wave-uniform scalars (never an indexed
// array: a lane-dependent pick between two entries of one made the compiler
// keep the array in LDS, a store and a load between the block ids and every
// K/V address).
struct Blk4 {
  int b[4];
};

// The block ids of the pass at c0 (c0 < end); blocks past the context end
// are read as the pass's first block (written, in range).
__device__ __forceinline__ Blk4 pass_blocks(const int32_t* __restrict__ bt, int c0, int end) {
  Blk4 r;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    r.b[b] = __builtin_amdgcn_readfirstlane(bt[(c0 + 16 * b < end) ? (c0 >> 4) + b : (c0 >> 4)]);
  return r;
}

// Issue every K and V load of the pass (tokens past the context end are
// masked by the math).  NT: non-temporal loads, for launches that stream
// hundreds of MB (each K/V byte is read once per step; measured on MI355X,
// random 4 KB reads stream at 6.8-6.9 TB/s with the hint and 6.1-6.2 TB/s
// without).  Smaller launches, latency-bound, run faster with ordinary loads.
template <int D, bool NT>
__device__ __forceinline__ void mfma_issue(MfmaPass<D>& r, const bf16_t* __restrict__ kc,
                                           const bf16_t* __restrict__ vc, const Blk4& blk, int g, int nkv, int hc,
                                           int grp) {
  constexpr long HEAD_BLK = 16L * D;
  const int b0 = blk.b[0], b1 = blk.b[1], b2 = blk.b[2], b3 = blk.b[3];
  // QK tile (s, u), A row hc: token 32 s + 8 (hc / 4) + 4 u + hc % 4, i.e.
  // block 2 s + hc / 8, slot 8 ((hc / 4) % 2) + 4 u + hc % 4; k-step j reads
  // the 16-byte chunk 4 j + grp of that token's K row.
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int b = (hc >> 3) ? (s ? b3 : b1) : (s ? b2 : b0);
    const bf16_t* kb = kc + ((long)b * nkv + g) * HEAD_BLK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int slot = 8 * ((hc >> 2) & 1) + 4 * u + (hc & 3);
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
        r.k[s][u][j] = ld<NT>((const bf16x8_t*)(kb + ((long)(4 * j + grp) * 16 + slot) * 8));
    }
  }
  // PV step s, d tile dt, A row hc: V^T row 16 dt + hc, tokens
  // 32 s + 8 grp + 0..7 = block 2 s + grp / 2, slots 8 (grp % 2) + 0..7.
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int b = (grp >> 1) ? (s ? b3 : b1) : (s ? b2 : b0);
    const bf16_t* vb = vc + ((long)b * nkv + g) * HEAD_BLK + 8 * (grp & 1);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      r.v[dt][s] = ld<NT>((const u32x4_t*)(vb + (long)(16 * dt + hc) * 16));
  }
}

// The math of the pass at c0: scores, online softmax update of (m, l, acc).
template <int D>
__device__ __forceinline__ void mfma_compute(MfmaPass<D>& r, const bf16x8_t (&qf)[D / 32], f32x4_t (&acc)[D / 16],
                                             float& m, float& l, int c0, int end, int grp, float scale_log2) {
  const bool full = c0 + 64 <= end;
  float sv[2][2][4];
  float bm = -INFINITY;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 32; ++j) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[s][u][j], qf[j], st, 0, 0, 0);
      // element e: token c0 + 32 s + 8 grp + 4 u + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = st[e] * scale_log2;
        if (!full && c0 + 32 * s + 8 * grp + 4 * u + e >= end) x = -INFINITY;  // also drops unwritten slots
        sv[s][u][e] = x;
        bm = fmaxf(bm, x);
      }
    }
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float mn = fmaxf(m, bm);  // finite: token c0 is in range
  const float alpha = exp2f(m - mn);
  m = mn;
  l *= alpha;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
  if (!full) {  // V of tokens past the end (possibly unwritten) must not meet P = 0 as NaN
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int nv = end - (c0 + 32 * s + 8 * grp);  // valid leading tokens of this lane's 8
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t mk = nv >= 2 * w + 2 ? 0xffffffffu : (nv == 2 * w + 1 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) r.v[dt][s][w] &= mk;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // k slots 8 grp + 0..7: tile (s, 0) elements 0..3, then tile (s, 1).  P
    // enters as a bf16 pair hi + lo (lo = the rounding residual, so hi + lo
    // carries about 16 significant bits) against the exact bf16 V.
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = exp2f(sv[s][w >> 1][2 * (w & 1)] - mn), p1 = exp2f(sv[s][w >> 1][2 * (w & 1) + 1] - mn);
      ph[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t));  // RNE
      const f32x2_t r = {p0 - lo_bf16(ph[w]), p1 - hi_bf16(ph[w])};
      pl[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
      l += p0 + p1;
    }
    const bf16x8_t pbh = __builtin_bit_cast(bf16x8_t, (u32x4_t){ph[0], ph[1], ph[2], ph[3]});
    const bf16x8_t pbl = __builtin_bit_cast(bf16x8_t, (u32x4_t){pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const bf16x8_t vt = __builtin_bit_cast(bf16x8_t, r.v[dt][s]);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pbh, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pbl, acc[dt], 0, 0, 0);
    }
  }
}

}  // namespace

// Fused RoPE prologue of a work item (row t, KV head g): stage the G query
// heads of this KV head, its k and its v from the QKV projection (summing
// split-K slices in slice order) in LDS, rotate q and k (rotate-half, the
// step's cos/sin table), round to bf16 into rq / rv.  The workgroup whose
// partition holds the row's last position writes the row's k and v into the
// paged cache at its slot (rows of other sequences never read that slot; this
// row's own passes take the token from LDS).  Same arithmetic as the separate
// RoPE / cache-write kernel, so the results are the same bits.
// The staging of one work item's q heads, k and v: a thread's chunks of
// every slice are all in flight before the first add (slice order kept).
template <int D, int G, int NT, int S>
__device__ __forceinline__ void rope_stage(const float* __restrict__ row, long slice_stride, int g, int nq, int nkv,
                                           float* rbuf) {
  constexpr int N4 = (G + 2) * D / 4, CPT = (N4 + NT - 1) / NT;
  f32x4_t p[CPT][S];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = 4 * (threadIdx.x + c * NT);
    if (e < 4 * N4) {
      const int src = e < G * D ? g * G * D + e
                                : (e < (G + 1) * D ? nq * D + g * D + (e - G * D)
                                                   : (nq + nkv) * D + g * D + (e - (G + 1) * D));
#pragma unroll
      for (int s = 0; s < S; ++s)
        p[c][s] = __builtin_nontemporal_load((const f32x4_t*)(row + src + s * slice_stride));
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = 4 * (threadIdx.x + c * NT);
    if (e < 4 * N4) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; ++s) a += p[c][s];
      *(f32x4_t*)(rbuf + e) = a;
    }
  }
}

template <int D, int G, int NWAVE>
__device__ __forceinline__ void rope_prologue(const RopeIn& ra, int t, int g, int nq, int nkv, int ctx, int start,
                                              int end, bf16_t* kcw, bf16_t* vcw, bf16_t* rq, bf16_t* rv) {
  constexpr int HALF = D / 2, NCH = D / 8, NT = 64 * NWAVE;
  // the item's rows of the projection, then the row's cos and sin
  __shared__ __attribute__((aligned(16))) float rbuf[(G + 2) * D + D];
  float* cr = rbuf + (G + 2) * D;
  float* sr = cr + HALF;
  const int width = (nq + 2 * nkv) * D;
  const float* row = ra.qkv + (long)t * width;
  // the table entries are loaded with the row's slices: one round of loads
  float cv = 0.f, sv = 0.f;
  if ((int)threadIdx.x < HALF) {
    cv = ra.cosb[(long)t * HALF + threadIdx.x];
    sv = ra.sinb[(long)t * HALF + threadIdx.x];
  }
  switch (ra.splits) {  // uniform
    case 1: rope_stage<D, G, NT, 1>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    case 2: rope_stage<D, G, NT, 2>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    case 3: rope_stage<D, G, NT, 3>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    case 4: rope_stage<D, G, NT, 4>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    case 5: rope_stage<D, G, NT, 5>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    case 6: rope_stage<D, G, NT, 6>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    case 7: rope_stage<D, G, NT, 7>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
    default: rope_stage<D, G, NT, kMaxSplits>(row, ra.slice_stride, g, nq, nkv, rbuf); break;
  }
  if ((int)threadIdx.x < HALF) {
    cr[threadIdx.x] = cv;
    sr[threadIdx.x] = sv;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (G + 1) * HALF + D; i += 64 * NWAVE) {
    if (i < (G + 1) * HALF) {
      const int hh = i / HALF, j = i % HALF;
      float y1, y2;
      rope_pair(rbuf[hh * D + j], rbuf[hh * D + j + HALF], cr[j], sr[j], y1, y2);
      rq[hh * D + j] = f32_to_bf16(y1);
      rq[hh * D + j + HALF] = f32_to_bf16(y2);
    } else {
      const int j = i - (G + 1) * HALF;
      rv[j] = f32_to_bf16(rbuf[(G + 1) * D + j]);
    }
  }
  __syncthreads();
  const int own = ctx - 1;
  if (own >= start && own < end) {
    const int s = ra.slot[t];
    if (s >= 0) {
      const long blk = s / NS_BLOCK;
      const int tok = s % NS_BLOCK;
      for (int j = threadIdx.x; j < D; j += 64 * NWAVE) {
        // K rows chunk-major within the block ([blk][nkv][d/8][16][8]), V
        // transposed ([blk][nkv][d][16])
        kcw[(((blk * nkv + g) * NCH + j / 8) * NS_BLOCK + tok) * 8 + (j & 7)] = rq[G * D + j];
        vcw[((blk * nkv + g) * D + j) * NS_BLOCK + tok] = rv[j];
      }
    }
  }
}

// Replace the row's own token (pass offset o) in the pass registers: K
// fragments of lanes with head column 4 (o%32/8) + o%4 (tile (o/32,
// o%8/4), chunk 4 j + grp) and element o%8 of the V^T fragments of lanes
// with grp = o%32/8 (head-dim row 16 dt + hc).
template <int D, int G>
__device__ __forceinline__ void patch_own_token(MfmaPass<D>& r, int o, int hc, int grp, const bf16_t* rq,
                                                const bf16_t* rv) {
  const int ss = o >> 5, rem = o & 31;
  if (hc == 4 * (rem >> 3) + (rem & 3)) {
    const int uu = (rem >> 2) & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (s == ss && u == uu) {
#pragma unroll
          for (int j = 0; j < D / 32; ++j) r.k[s][u][j] = *(const bf16x8_t*)(rq + G * D + (4 * j + grp) * 8);
        }
  }
  if (grp == (rem >> 3)) {
    const int e = o & 7;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s == ss) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const uint32_t val = rv[16 * dt + hc];
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if (w == (e >> 1)) {
              const uint32_t x = r.v[dt][s][w];
              r.v[dt][s][w] = (e & 1) ? ((x & 0x0000ffffu) | (val << 16)) : ((x & 0xffff0000u) | val);
            }
        }
      }
  }
}

// Lane l of a wavefront: head column hc = l % 16 (heads >= G are zero
// padding whose results are dropped), lane group grp = l / 16.  Arguments as
// attn_decode_kernel.
template <int D, int G, int NWAVE, bool ROPE, bool KNT>
__global__ void __launch_bounds__(64 * NWAVE) attn_mfma_kernel(
    const bf16_t* __restrict__ qatt, const bf16_t* kc, const bf16_t* vc,
    const int32_t* __restrict__ row_bseq, const int32_t* __restrict__ row_pos, const int32_t* __restrict__ btab,
    bf16_t* __restrict__ out, float* __restrict__ part_acc, float* __restrict__ part_ml, int maxb, int row0,
    int n_rows, int nq, int nkv, int P, int n_parts, float scale_log2, const int32_t* __restrict__ skip_seq,
    RopeIn ra, const int32_t* __restrict__ row_order, int osr) {
  static_assert(G <= 16 && D % 32 == 0, "heads must fit the 16 MFMA columns, d whole k-steps");
  constexpr int NCH = D / 8;  // 16-byte chunks per head row
  constexpr int KS = D / 32, DT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hc = lane & 15, grp = lane >> 4;
  const int total = n_rows * nkv * n_parts;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int part = w % n_parts;
    const int rest = w / n_parts;
    const int g = rest % nkv;
    // rows in the order given (longest context first: the long items start
    // early and the dispatch tail is short ones), else in index order
    const int t = row_order ? row_order[row0 + rest / nkv] : row0 + rest / nkv;
    if (skip_seq) {  // rows of prefill tiles belong to the prefill kernel
      const int t0 = row0 + ((t - row0) & ~31);
      if (t0 + 32 <= row0 + n_rows && prefill_tile(skip_seq, row_pos, t0, lane)) continue;
    }
    const int32_t* __restrict__ bt;
    bool pad;
    const int pos_t = row_pos[t];  // loaded with the row's sequence: one round
    if (row_bseq) {
      const int bs = row_bseq[t];
      pad = bs < 0;
      bt = btab + (long)(pad ? 0 : bs) * maxb;
    } else {
      bt = btab + (long)t * maxb;
      pad = bt[0] < 0;
    }
    // The first pass's block ids, read before the context length is known
    // (indices clamped into the row) so that they arrive with it; the empty
    // asm keeps the loads ahead of the branches below.
    const int cf = part * P + 64 * wave;
    const int f0 = __builtin_amdgcn_readfirstlane(bt[min((cf >> 4), maxb - 1)]);
    const int f1 = __builtin_amdgcn_readfirstlane(bt[min((cf >> 4) + 1, maxb - 1)]);
    const int f2 = __builtin_amdgcn_readfirstlane(bt[min((cf >> 4) + 2, maxb - 1)]);
    const int f3 = __builtin_amdgcn_readfirstlane(bt[min((cf >> 4) + 3, maxb - 1)]);
    asm volatile("" : : "s"(f0), "s"(f1), "s"(f2), "s"(f3));
    // output column c of this item's heads (row-major or slab-major out)
    auto oix = [&](int c) { return act_idx(t, g * G * D + c, nq * D, osr); };
    if (pad) {  // padding row: zero output
      if (part == 0)
        for (int i = threadIdx.x; i < G * D; i += 64 * NWAVE) out[oix(i)] = 0;
      continue;
    }
    const int ctx = pos_t + 1;
    const int start = part * P;
    if (start >= ctx) continue;
    const int end = min(start + P, ctx);
    const int nparts_row = (ctx + P - 1) / P;

    // Q^T fragments (B operand of QK): head hc, d chunk 4 j + grp
    bf16x8_t qf[KS];
    // fused RoPE: the rotated q heads of this KV head and the rotated k (bf16
    // [G + 1][D]) and v (bf16 [D]) of the row's own token, in LDS
    __shared__ __attribute__((aligned(16))) bf16_t rq[ROPE ? (G + 1) * D : 8];
    __shared__ __attribute__((aligned(16))) bf16_t rv[ROPE ? D : 8];
    if constexpr (ROPE) {
      rope_prologue<D, G, NWAVE>(ra, t, g, nq, nkv, ctx, start, end, const_cast<bf16_t*>(kc), const_cast<bf16_t*>(vc),
                                 rq, rv);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        u32x4_t q = *(const u32x4_t*)(rq + (hc < G ? hc : 0) * D + (4 * j + grp) * 8);
        if (hc >= G) q = (u32x4_t){0u, 0u, 0u, 0u};
        qf[j] = __builtin_bit_cast(bf16x8_t, q);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        u32x4_t q = *(const u32x4_t*)(qatt + ((((long)t * nkv + g) * NCH + 4 * j + grp) * G + (hc < G ? hc : 0)) * 8);
        if (hc >= G) q = (u32x4_t){0u, 0u, 0u, 0u};
        qf[j] = __builtin_bit_cast(bf16x8_t, q);
      }
    }
    float m = -INFINITY, l = 0.f;
    f32x4_t acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // blocks past the context end are read as the pass's first block
    Blk4 cur;
    cur.b[0] = f0;
    cur.b[1] = cf + 16 < end ? f1 : f0;
    cur.b[2] = cf + 32 < end ? f2 : f0;
    cur.b[3] = cf + 48 < end ? f3 : f0;
    for (int c0 = cf; c0 < end; c0 += 64 * NWAVE) {
      MfmaPass<D> pr;
      mfma_issue<D, KNT>(pr, kc, vc, cur, g, nkv, hc, grp);
      // the next pass's block ids load while this pass's K/V are in flight
      const int cn = c0 + 64 * NWAVE;
      if (cn < end) cur = pass_blocks(bt, cn, end);
      if constexpr (ROPE) {
        // the row's own token: its K/V from LDS (the cache copy is written
        // by this workgroup, not necessarily visible to these loads)
        const int o = ctx - 1 - c0;
        if (o >= 0 && o < 64) patch_own_token<D, G>(pr, o, hc, grp, rq, rv);
      }
      mfma_compute<D>(pr, qf, acc, m, l, c0, end, grp, scale_log2);
    }
    // the four lanes of a head hold disjoint tokens: sum their denominators
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // lane (hc, grp) owns O^T rows 16 dt + 4 grp + 0..3 of head hc
    const long item = ((long)t * nkv + g) * n_parts + part;
    if constexpr (NWAVE == 1) {
      if (hc < G) {
        if (nparts_row == 1) {
          const float inv = 1.f / l;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            uint2 o2;
            o2.x = pack_bf16(acc[dt][0] * inv, acc[dt][1] * inv);
            o2.y = pack_bf16(acc[dt][2] * inv, acc[dt][3] * inv);
            // 4 consecutive columns from a multiple of 4: one slab piece
            *(uint2*)(out + oix(hc * D + 16 * dt + 4 * grp)) = o2;
          }
        } else {
          float* pa = part_acc + (item * G + hc) * D + 4 * grp;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(pa + 16 * dt) = acc[dt];
          if (grp == 0) {
            part_ml[(item * G + hc) * 2] = m;
            part_ml[(item * G + hc) * 2 + 1] = l;
          }
        }
      }
    } else {
      // Merge the wavefronts: M = max m_w, L = sum l_w 2^(m_w - M),
      // acc = sum acc_w 2^(m_w - M), in wavefront order.  A wavefront that
      // had no pass contributes m = -inf, l = 0, acc = 0 (weight 0).
      __shared__ float macc[NWAVE][G][D];
      __shared__ float mml[NWAVE][G][2];
      if (hc < G) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)&macc[wave][hc][16 * dt + 4 * grp] = acc[dt];
        if (grp == 0) {
          mml[wave][hc][0] = m;
          mml[wave][hc][1] = l;
        }
      }
      __syncthreads();
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
          out[oix(h * D + dd)] = f32_to_bf16(o / L);
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
}

// The bf16 matrix-core kernel in its launch shape: 8 or 4 wavefronts per
// item with the fused RoPE prologue, else 1, 4 or 8.
template <int D, int G, bool KNT>
static void launch_mfma(const AttnArgs& a, long grid, float scale_log2, hipStream_t st) {
  const RopeIn ra{a.rope_qkv, a.rope_slice_stride, a.rope_splits, a.cosb, a.sinb, a.slot};
#define NS_MFMA_ARGS                                                                                           \
  (const bf16_t*)a.q_att, (const bf16_t*)a.kc, (const bf16_t*)a.vc, a.row_bseq, a.row_pos, a.btab,             \
      (bf16_t*)a.out, a.part_acc, a.part_ml, a.maxb, a.row0, a.n_rows, a.nq, a.nkv, a.part_tokens, a.n_parts,  \
      scale_log2, a.row_seq, ra, a.row_order, a.out_slab_rows
  const dim3 g((unsigned)grid);
  if (a.rope_qkv) {  // the fused prologue runs on 8 or 4 wavefronts per item
    if (a.waves == 8)
      hipLaunchKernelGGL((attn_mfma_kernel<D, G, 8, true, KNT>), g, dim3(512), 0, st, NS_MFMA_ARGS);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, G, 4, true, KNT>), g, dim3(256), 0, st, NS_MFMA_ARGS);
  } else if (a.waves == 1) {
    hipLaunchKernelGGL((attn_mfma_kernel<D, G, 1, false, KNT>), g, dim3(64), 0, st, NS_MFMA_ARGS);
  } else if (a.waves == 8) {
    hipLaunchKernelGGL((attn_mfma_kernel<D, G, 8, false, KNT>), g, dim3(512), 0, st, NS_MFMA_ARGS);
  } else {
    hipLaunchKernelGGL((attn_mfma_kernel<D, G, 4, false, KNT>), g, dim3(256), 0, st, NS_MFMA_ARGS);
  }
#undef NS_MFMA_ARGS
}

template <typename T, int D, int G>
static void launch_attn_t(const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  if (!a.row_seq || !prefill_supported(a.dtype, D, G) || a.n_rows < 32) a.row_seq = nullptr;  // no prefill tiles
  if (a.rope_qkv) a.row_seq = nullptr;  // fused RoPE: rows of distinct sequences, no q_att for prefill tiles
  const long total = (long)a.n_rows * a.nkv * a.n_parts;
  if (total <= 0) return;
  long grid = total;
  if (a.wg_cap > 0 && grid > a.wg_cap) grid = a.wg_cap;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
#define NS_ATTN_ARGS                                                                                             \
  (const T*)a.q_att, (const T*)a.kc, (const T*)a.vc, a.row_bseq, a.row_pos, a.btab, (T*)a.out, a.part_acc,       \
      a.part_ml, a.maxb, a.row0, a.n_rows, a.nq, a.nkv, a.part_tokens, a.n_parts, scale_log2, a.row_seq
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.kv_nt)
      launch_mfma<D, G, true>(a, grid, scale_log2, st);
    else
      launch_mfma<D, G, false>(a, grid, scale_log2, st);
  } else {
    if (a.waves == 1)
      hipLaunchKernelGGL((attn_decode_kernel<T, D, G, 1>), dim3((unsigned)grid), dim3(64), 0, st, NS_ATTN_ARGS);
    else
      hipLaunchKernelGGL((attn_decode_kernel<T, D, G, 4>), dim3((unsigned)grid), dim3(256), 0, st, NS_ATTN_ARGS);
  }
#undef NS_ATTN_ARGS
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
