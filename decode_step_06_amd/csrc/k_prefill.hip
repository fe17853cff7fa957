// Paged grouped-query attention for prefill tiles, on MFMA (gfx950).
//
// A prefill tile is 32 consecutive step rows of one sequence at consecutive
// positions p0 .. p0+31 (a chunk of a prompt; NanoFlow review, "Runtime
// details that keep the pipeline fed": prefill is chunked at token
// granularity to top up the dense batch).  Row i attends keys 0 .. p0+i of
// its sequence, read through the block table, like every decode row; the
// decode kernel skips the rows of such tiles and this kernel computes them
// with matrix cores, since a tile reuses every K/V block for 32 rows.
//
// One workgroup per (tile, KV head), one wavefront per query head of the
// group.  For each block of 32 keys:
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16: keys x queries, d deep), so
//                 lane l owns query l % 32 and 16 of the block's keys: the
//                 softmax max and sum need one exchange between lane halves;
//   online softmax in the log2 domain (fp32), causal mask by position;
//   O^T += V^T P^T (v_mfma_f32_32x32x16_f16): V is staged transposed in LDS
//                 as fp16 (exact for bf16 values in fp16 range) and P goes
//                 to fp16 (11 significant bits); the softmax denominator sums
//                 the same rounded P, so the weights of every row sum to 1.
// K of keys past the tile's last position is read at that position
// (written, finite) and masked; their V is zeroed.
#include "ns_kernels.h"

namespace ns {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

}  // namespace

template <int D, int G>
__global__ void __launch_bounds__(64 * G) attn_prefill_kernel(
    const bf16_t* __restrict__ qatt, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_bseq, const int32_t* __restrict__ row_pos,
    const int32_t* __restrict__ btab, bf16_t* __restrict__ out, int maxb, int row0, int n_rows, int nq, int nkv,
    float scale_log2, int osr) {
  constexpr int NCH = D / 8;   // 16-byte chunks per head row
  constexpr int KS = D / 16;   // MFMA steps over d
  constexpr int DT = D / 32;   // 32-wide d tiles of the output
  constexpr int VP = 40;       // LDS row pitch of V^T (fp16), 32 keys + padding
  constexpr long HEAD_BLK = 16L * D;
  __shared__ __attribute__((aligned(16))) _Float16 vt[2][D][VP];

  const int lane = threadIdx.x & 63;
  const int hh = threadIdx.x >> 6;  // query head within the group
  const int g = blockIdx.y;
  const int t0 = row0 + 32 * blockIdx.x;
  if (t0 + 32 > row0 + n_rows || !prefill_tile(row_seq, row_pos, t0, lane)) return;
  const int p0 = row_pos[t0];
  const int last = p0 + 31;  // the tile's last position: every key up to it is written
  const int32_t* __restrict__ bt = btab + (long)(row_bseq ? row_bseq[t0] : t0) * maxb;
  const int q = lane & 31, hl = lane >> 5;

  // Q^T fragments (B operand): query q, d chunk 2 s + hl
  bf16x8_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = *(const bf16x8_t*)(qatt + ((((long)(t0 + q) * nkv + g) * NCH + 2 * s + hl) * G + hh) * 8);

  f32x16_t o[DT];
#pragma unroll
  for (int j = 0; j < DT; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int qpos = p0 + q;

  const int nkb = (last + 32) / 32;
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = 32 * kb;
    _Float16(*vb)[VP] = vt[kb & 1];
    // stage V^T of keys k0 .. k0+31 (fp16) in LDS: the cache holds each
    // block transposed, so a head-dim row's 8 keys are one 16-byte load;
    // keys past the tile's last position are zeroed (they may be unwritten)
    for (int it = threadIdx.x; it < 4 * D; it += 64 * G) {
      const int dd = it >> 2, kg = it & 3;
      const int key0 = k0 + 8 * kg;
      const int kr = min(key0, last);
      const uint4 w = *(const uint4*)(vc + ((long)bt[kr >> 4] * nkv + g) * HEAD_BLK + (long)dd * 16 + (kr & 8));
      const int nvalid = last - key0 + 1;
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
      f16x8_t h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[2 * i] = 2 * i < nvalid ? (_Float16)lo_bf16(wv[i]) : (_Float16)0.f;
        h[2 * i + 1] = 2 * i + 1 < nvalid ? (_Float16)hi_bf16(wv[i]) : (_Float16)0.f;
      }
      *(f16x8_t*)&vb[dd][8 * kg] = h;
    }
    // K fragments (A operand): key k0 + q, d chunk 2 s + hl
    const int kk = min(k0 + q, last);
    const bf16_t* kp = kc + ((long)bt[kk >> 4] * nkv + g) * HEAD_BLK + (long)(kk & 15) * 8;
    f32x16_t st;
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t kf = *(const bf16x8_t*)(kp + (long)(2 * s + hl) * 16 * 8);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
    }
    // lane: query q, keys k0 + 8 (e / 4) + 4 hl + e % 4
    float sv[16];
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0 + 8 * (e >> 2) + 4 * hl + (e & 3);
      sv[e] = key <= qpos ? st[e] * scale_log2 : -INFINITY;
      bm = fmaxf(bm, sv[e]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(m, bm);  // finite: key 0 of block 0 is in every row's range
    const float alpha = exp2f(m - mn);
    m = mn;
    float ps = 0.f;
    uint32_t pk[8];  // fp16 pairs of the 16 probabilities, in e order
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const _Float16 a = (_Float16)exp2f(sv[e] - mn), b = (_Float16)exp2f(sv[e + 1] - mn);
      ps += (float)a + (float)b;
      const f16x2_t v = {a, b};
      pk[e / 2] = __builtin_bit_cast(uint32_t, v);
    }
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[j][e] *= alpha;
    // P^T as the B operand of the two 16-key steps: lane half hl needs keys
    // 16 s' + 8 hl .. +8; the halves swap one group of 4 per step
    f16x8_t pb[2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      const uint32_t* ga = pk + 4 * sp;      // keys 16 s' + 4 hl + 0..3 (e group 2 s')
      const uint32_t* gb = pk + 4 * sp + 2;  // keys 16 s' + 8 + 4 hl + 0..3 (e group 2 s' + 1)
      const uint32_t x0 = hl ? ga[0] : gb[0], x1 = hl ? ga[1] : gb[1];
      const uint32_t r0 = __shfl_xor(x0, 32, 64), r1 = __shfl_xor(x1, 32, 64);
      uint32_t w[4];
      if (hl) {
        w[0] = r0; w[1] = r1; w[2] = gb[0]; w[3] = gb[1];
      } else {
        w[0] = ga[0]; w[1] = ga[1]; w[2] = r0; w[3] = r1;
      }
      pb[sp] = __builtin_bit_cast(f16x8_t, (u32x4_t){w[0], w[1], w[2], w[3]});
    }
    __syncthreads();  // V^T of this block staged by every wavefront
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const f16x8_t va = *(const f16x8_t*)&vb[32 * j + q][16 * sp + 8 * hl];
        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[sp], o[j], 0, 0, 0);
      }
  }
  // lane: query q, d = 32 j + 8 (e / 4) + 4 hl + e % 4
  const float inv = 1.f / l;
#pragma unroll
  for (int j = 0; j < DT; ++j)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d0 = 32 * j + 8 * e4 + 4 * hl;
      uint2 w;
      w.x = pack_bf16(o[j][4 * e4] * inv, o[j][4 * e4 + 1] * inv);
      w.y = pack_bf16(o[j][4 * e4 + 2] * inv, o[j][4 * e4 + 3] * inv);
      // 4 consecutive columns from a multiple of 4: one slab piece
      *(uint2*)(out + act_idx(t0 + q, (g * G + hh) * D + d0, nq * D, osr)) = w;
    }
}

int prefill_supported(int dtype, int d, int G) {
  return dtype == NS_DT_BF16 && (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 7 || G == 8);
}

void launch_attention_prefill(const AttnArgs& a, hipStream_t st) {
  const int G = a.nq / a.nkv;
  if (!a.row_seq || !prefill_supported(a.dtype, a.d, G) || a.n_rows < 32) return;
  const dim3 grid((unsigned)(a.n_rows / 32), (unsigned)a.nkv);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)a.d));
#define NS_PF(DD, GG)                                                                                           \
  if (a.d == DD && G == GG) {                                                                                   \
    hipLaunchKernelGGL((attn_prefill_kernel<DD, GG>), grid, dim3(64 * GG), 0, st, (const bf16_t*)a.q_att,      \
                       (const bf16_t*)a.kc, (const bf16_t*)a.vc, a.row_seq, a.row_bseq, a.row_pos, a.btab,     \
                       (bf16_t*)a.out, a.maxb, a.row0, a.n_rows, a.nq, a.nkv, scale_log2, a.out_slab_rows);                     \
    return;                                                                                                     \
  }
  NS_PF(64, 1) NS_PF(64, 2) NS_PF(64, 4) NS_PF(64, 7) NS_PF(64, 8)
  NS_PF(128, 1) NS_PF(128, 2) NS_PF(128, 4) NS_PF(128, 7) NS_PF(128, 8)
#undef NS_PF
}

}  // namespace ns
