// Dense projections of the decode step on gfx950 matrix cores.
//
// C = A * B^T with A [M, K] (activations) and B [N, K] (a weight stored
// row-major [out, in]), both K-contiguous, bf16 in, fp32 accumulate.  These
// are the "dense" class of the NanoFlow review's operator table (section
// "Four resource classes, one serialized queue": KQV, O, Up, Gate, Down),
// compute-bound at a dense batch and weight-streaming (HBM-bound) at small
// decode batches.
//
// Kernel: a workgroup of 4 wavefronts owns a BM x BN output tile; K advances
// in BK slabs staged through LDS (double buffered: the next slab's global
// loads are in flight while the current slab feeds the MFMAs).  Each
// wavefront owns a (BM / WM) x (BN / WN) sub-tile of 16x16 fragments and
// issues v_mfma_f32_16x16x32_bf16.  LDS rows are padded by 16 bytes so the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks.
//
// Epilogues are fused so that no projection output makes an extra HBM round
// trip: fp32 store (QKV, logits), fp32 residual add (O and Down projections
// write x += y), and the SwiGLU product (the tile loads gate rows and the
// matching up rows, so silu(gate) * up is formed in registers).
#include <type_traits>

#include "ns_kernels.h"

namespace ns {

namespace {

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int BM, int BN, int BK, int WM, int WN, int EPI>
struct GemmCfg {
  static constexpr int NT = 64 * WM * WN;    // threads
  static constexpr int TM = BM / WM;         // wave tile rows
  static constexpr int TN = BN / WN;         // wave tile B rows
  static constexpr int FM = TM / 16;
  static constexpr int FN = TN / 16;
  static constexpr int LDK = BK + 8;         // padded LDS row (elements)
  static constexpr int A_CH = BM * BK / 8;   // 16-byte chunks per A slab
  static constexpr int B_CH = BN * BK / 8;
  static constexpr int A_PT = (A_CH + NT - 1) / NT;
  static constexpr int B_PT = (B_CH + NT - 1) / NT;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole 16x16 fragments");
  static_assert(BK % 32 == 0, "BK must be a multiple of the MFMA depth");
  static_assert(EPI != EPI_SILU_MUL || FN % 2 == 0, "SwiGLU tile needs gate and up fragment pairs");
};

}  // namespace

// BNT: B loads are non-temporal (one row tile covers all M rows, so each B
// element is read by one workgroup).  LAY: bit 0, A is K-slab-major (PK_A);
// bit 1, the SwiGLU output is (PK_C) -- template parameters so that the
// row-major addresses stay the plain ones.
template <int BM, int BN, int BK, int WM, int WN, int EPI, typename OutT, int BNT = 0, int LAY = 0>
__global__ void __launch_bounds__(64 * WM * WN) gemm_bf16_kernel(const bf16_t* __restrict__ A, int lda,
                                                                 const bf16_t* __restrict__ B, int ldb, int M, int N,
                                                                 int K, void* __restrict__ Cv, int ldc, int splits,
                                                                 long slice_stride, int pk) {
  using C = GemmCfg<BM, BN, BK, WM, WN, EPI>;
  constexpr int LDK = C::LDK;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // Output columns per tile: BN, or BN/2 for the SwiGLU pair tile.
  constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? BN / 2 : BN;
  const int n_tiles_n = (N + OUT_BN - 1) / OUT_BN;
  const int tile_m = blockIdx.x / n_tiles_n;
  const int tile_n = blockIdx.x % n_tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * OUT_BN;

  // Global source row of each LDS row (clamped into range; clamped rows only
  // feed outputs that are never stored).
  auto a_row = [&](int r) { int m = m0 + r; return m < M ? m : M - 1; };
  auto b_row = [&](int r) {
    if constexpr (EPI == EPI_SILU_MUL) {
      const int half = BN / 2;
      int n = n0 + (r < half ? r : r - half);
      n = n < N ? n : N - 1;
      return r < half ? n : N + n;
    } else {
      int n = n0 + r;
      return n < N ? n : N - 1;
    }
  };

  u32x4_t ra[C::A_PT], rb[C::B_PT];
  auto load_slab = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_PT; ++i) {
      const int c = tid + i * C::NT;
      if (c < C::A_CH) {
        const int r = c / (BK / 8), k = k0 + (c % (BK / 8)) * 8;
        ra[i] = *(const u32x4_t*)(A + ((LAY & 1) ? ((long)(k >> 5) * lda + a_row(r)) * 32 + (k & 31)
                                                 : (long)a_row(r) * lda + k));
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PT; ++i) {
      const int c = tid + i * C::NT;
      if (c < C::B_CH) {
        const int r = c / (BK / 8), k = k0 + (c % (BK / 8)) * 8;
        const u32x4_t* src = (pk & PK_B) ? (const u32x4_t*)(B + ((long)(k >> 5) * ldb + b_row(r)) * 32 + (k & 31))
                                 : (const u32x4_t*)(B + (long)b_row(r) * ldb + k);
        rb[i] = BNT ? __builtin_nontemporal_load(src) : *src;
      }
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_PT; ++i) {
      const int c = tid + i * C::NT;
      if (c < C::A_CH) {
        const int r = c / (BK / 8), k8 = c % (BK / 8);
        *(u32x4_t*)&As[buf][r * LDK + k8 * 8] = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PT; ++i) {
      const int c = tid + i * C::NT;
      if (c < C::B_CH) {
        const int r = c / (BK / 8), k8 = c % (BK / 8);
        *(u32x4_t*)&Bs[buf][r * LDK + k8 * 8] = rb[i];
      }
    }
  };

  // LDS row of B fragment f of this wave.
  auto b_frag_row = [&](int f) {
    if constexpr (EPI == EPI_SILU_MUL) {
      constexpr int HF = C::FN / 2;  // gate fragments, then the matching up fragments
      const int col = wn * (C::TN / 2) + 16 * (f % HF);
      return (f < HF ? 0 : BN / 2) + col;
    } else {
      return wn * C::TN + 16 * f;
    }
  };

  f32x4_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K slabs [sb, se) of split blockIdx.y (all of K unless EPI_PARTIAL)
  const int slabs = K / BK, split = blockIdx.y;
  const int sb = (int)((long)split * slabs / splits), se = (int)((long)(split + 1) * slabs / splits);
  const int nk = se - sb;
  load_slab(sb * BK);
  store_slab(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;  // fragment row / k offset of this lane
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slab((sb + kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = *(const bf16x8_t*)&As[buf][(wm * C::TM + 16 * i + fr) * LDK + kk + fk];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) bfr[j] = *(const bf16x8_t*)&Bs[buf][(b_frag_row(j) + fr) * LDK + kk + fk];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slab(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Fragment element r of lane l is row 4*(l/16)+r, column l%16.
  const int er = (lane >> 4) * 4, ec = lane & 15;
  if constexpr (EPI == EPI_SILU_MUL) {
    OutT* Cp = (OutT*)Cv;
    constexpr int HF = C::FN / 2;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < HF; ++j) {
        const int col = n0 + wn * (C::TN / 2) + 16 * j + ec;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * C::TM + 16 * i + er + r;
          if (row < M)
            Elem<OutT>::store(Cp, act_idx(row, col, ldc, (LAY & 2) ? ldc : 0),
                              silu_f(acc[i][j][r]) * acc[i][j + HF][r]);
        }
      }
  } else {
    float* Cp = (float*)Cv + (EPI == EPI_PARTIAL ? split * slice_stride : 0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int col = n0 + wn * C::TN + 16 * j + ec;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * C::TM + 16 * i + er + r;
          if (row >= M) continue;
          float* p = Cp + (long)row * ldc + col;
          if constexpr (EPI == EPI_RESID_F32) *p += acc[i][j][r];
          else *p = acc[i][j][r];
        }
      }
  }
}

// Dense-batch projection (M >= 256, K % 32 == 0): a 256 x 256 output tile
// per workgroup of 4 wavefronts in a 2 x 2 grid, each owning a 128 x 128
// sub-tile (4 x 4 fragments of 32 x 32, 256 accumulators per lane): per FLOP
// that needs half the LDS bytes of a 64 x 64 wavefront tile.  The 32x32x16
// bf16 MFMA is used because on gfx950 it sustains the full bf16 rate, about
// twice what the 16x16x32 form reaches.
//
// Slabs of 32 K go global -> LDS with buffer_load_dwordx4 ... lds (no
// register staging, no LDS write instructions): lane l of a wavefront
// instruction lands its 16 bytes at M0 + 16 l, so one instruction fills 16
// rows of 64 bytes.  Each lane's row offset sits in a VGPR for the whole
// kernel and the slab's K offset goes in the scalar offset, so a refill costs
// no vector ALU work.  Rows are unpadded; the 16-byte chunk c of row r is
// stored at position c ^ (((r >> 1) ^ (r >> 2)) & 3), which keeps the
// 32-row fragment reads conflict-free.  Four slab buffers (4 x 32 KB), loads
// issued three slabs ahead.
//
// Software pipeline, two register sets of fragments: while the 32 MFMAs of
// slab k run, slab k+1's fragments are read from LDS into the other set and
// slab k+3's loads go out.  The instruction order within that stream is fixed
// with scheduling groups: 8 MFMAs interleaved with half the loads, the wait
// for slab k+1 and the barrier, then the 16 fragment reads one per MFMA, then
// the other half of the loads spread over the last MFMAs.  One wavefront per
// SIMD, so the MFMA pipe only stays fed if nothing in the stream stalls it.
// Past the last slab the loads re-read the last slab into buffers no one
// reads again (every access stays inside the operands).
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so workgroup b runs on XCD b % 8; giving each XCD a contiguous range
// of tiles, M-fastest, makes the tiles an XCD runs at once share their B
// columns in that XCD's private L2 while walking down A.
//
// Addressing is 32-bit (buffer offsets): the host sends operands whose byte
// span exceeds 4 GiB to the tiled kernel.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// s_waitcnt immediate: vmcnt(vm) lgkmcnt(lgkm), expcnt not waited on
constexpr int waitcnt_imm(int vm, int lgkm) { return ((vm >> 4) << 14) | (lgkm << 8) | 0x70 | (vm & 15); }

// scheduling-group instruction classes (AMDGPU sched_group_barrier masks)
constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100;

constexpr unsigned BUF_RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit dwords, no swizzle

// BNT: the B operand streams with non-temporal loads (set when one row tile
// covers all M rows, so that each B slab is read by one workgroup only).
// NWV: 4 wavefronts (one per SIMD, 128 x 128 outputs each) or 8 (two per
// SIMD, 128 x 64 each); PP (8 only): the two groups of 4 alternate between
// MFMAs and memory work (see the main loop).  Every variant accumulates each
// output over the same k-steps in the same order: the same bits.
template <int EPI, typename OutT, int BM = 256, int BNT = 0, int NWV = 4, int PP = 0>
__global__ void __launch_bounds__(64 * NWV) gemm_big_kernel(const bf16_t* __restrict__ A, int lda,
                                                            const bf16_t* __restrict__ B, int ldb, int M, int N,
                                                            int K, void* __restrict__ Cv, int ldc, int splits,
                                                            long slice_stride, int pk) {
  static_assert(BM == 256 || BM == 128, "tile rows");
  static_assert(NWV == 4 || (NWV == 8 && BM == 256), "wavefronts");
  static_assert(PP == 0 || NWV == 8, "ping-pong takes two wavefronts per SIMD");
  constexpr int BN = 256, BK = 32, NSTAGE = 4;
  // wavefronts in 2 rows of NWV / 2; each owns TM x TN outputs
  constexpr int TM = BM / 2, TN = 2 * BN / NWV, FM = TM / 32, FN = TN / 32;  // 32 x 32 fragments
  constexpr int ROWB = BK * 2;                  // bytes per LDS row
  constexpr int STAGE = (BM + BN) * ROWB;       // bytes per slab buffer (A rows, then B rows)
  constexpr int AG = BM / 16;                   // 16-row load groups of A (then BN / 16 of B)
  constexpr int LOADS = (BM + BN) / 16 / NWV;   // load instructions per wavefront per slab (8, 6 or 4)
  constexpr int NMF = 2 * FM * FN;              // MFMAs per wavefront per slab (32 or 16)
  constexpr int NREAD = 2 * (FM + FN);          // fragment reads per wavefront per slab (16 or 12)
  constexpr int PRE = NMF / 4;                  // MFMAs of a slab before its barrier
  constexpr int LPRE = (BM == 256 && NWV == 4) ? LOADS / 2 : LOADS;  // loads issued before the barrier
  constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? BN / 2 : BN;
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE];  // 128 or 96 KB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NWV / 2), wn = wave % (NWV / 2);
  const int m_tiles = (M + BM - 1) / BM;
  const int n_tiles = (N + OUT_BN - 1) / OUT_BN;
  const int tiles = m_tiles * n_tiles;
  int tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int tile_m = tile % m_tiles, tile_n = tile / m_tiles;
  const int m0 = tile_m * BM, n0 = tile_n * OUT_BN;

  // A's byte span: M rows, or (slab-major) K / 32 - 1 whole slab blocks of
  // lda rows then M rows of the last slab
  const unsigned a_bytes =
      (unsigned)((pk & PK_A) ? ((long)(K / 32 - 1) * lda + M) * 64 : (long)M * lda * 2);
  const unsigned b_bytes =
      (unsigned)((pk & PK_B) ? (long)K * ldb * 2 : (long)((EPI == EPI_SILU_MUL) ? 2 * N : N) * ldb * 2);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)a_bytes, BUF_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)b_bytes, BUF_RSRC_WORD3);
  // Load instruction j of wavefront w fills the 16 LDS rows of group
  // g = w + 4 j (groups 0..AG-1: A rows, then B rows); lane l loads row
  // 16 g' + l / 4 of its operand (g' the group within it), chunk
  // (l & 3) ^ swz(row).  Rows past M or N repeat the last row (their results
  // are never stored).
  // (sized for the largest tile: a value-dependent array size captured by
  // the nested lambdas below stops the host pass from emitting the kernel)
  static_assert(LOADS <= 8 && AG % NWV == 0, "load slots");
  unsigned voff[8];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int g = wave + NWV * j;
    const int r = (g < AG ? g : g - AG) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(r);
    if (g < AG) {
      int m = m0 + r;
      m = m < M ? m : M - 1;
      voff[j] = (pk & PK_A) ? (unsigned)(m * 64 + c * 16) : (unsigned)(((long)m * lda + c * 8) * 2);
    } else {
      int brow;
      if constexpr (EPI == EPI_SILU_MUL) {
        int n = n0 + (r < BN / 2 ? r : r - BN / 2);
        n = n < N ? n : N - 1;
        brow = r < BN / 2 ? n : N + n;
      } else {
        int n = n0 + r;
        brow = n < N ? n : N - 1;
      }
      voff[j] = (pk & PK_B) ? (unsigned)(brow * 64 + c * 16) : (unsigned)(((long)brow * ldb + c * 8) * 2);
    }
  }
  // K slabs [sb, sb + nk) of split blockIdx.y (all of K unless EPI_PARTIAL);
  // kt below counts slabs from sb.
  const int slabs = K / BK, split = blockIdx.y;
  const int sb = (int)((long)split * slabs / splits);
  const int nk = (int)((long)(split + 1) * slabs / splits) - sb;
  // loads j0..j1-1 of slab kt into buffer kt % 4
  auto issue = [&](int kt, int j0, int j1) {
    const int ks = sb + (kt < nk ? kt : nk - 1);
    const unsigned soff = (unsigned)ks * (BK * 2);
    // slab-major operands: slab ks is a contiguous [rows][32] block
    const unsigned soff_a = (pk & PK_A) ? (unsigned)ks * (unsigned)lda * (BK * 2) : soff;
    const unsigned soff_b = (pk & PK_B) ? (unsigned)ks * (unsigned)ldb * (BK * 2) : soff;
    char* base = lds + (kt % NSTAGE) * STAGE;
    // load slots j < AG / NWV carry A rows, the rest B rows (wave < NWV)
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const int g = wave + NWV * j;
      if (j < AG / NWV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(base + g * 16 * ROWB), 16, voff[j], soff_a, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(base + g * 16 * ROWB), 16, voff[j], soff_b, 0,
                                                 BNT ? 2 : 0);  // cache policy: 2 = nt
    }
  };
  // v_mfma_f32_32x32x16_bf16 operands: lane l holds row (or column) l % 32
  // of a fragment and the 8 K values 8 (l / 32) .. +8 of a 16-deep K step.
  // Fragment read offsets within a slab buffer for K step s = 0 / 1.
  const int fr = lane & 31, fq = lane >> 5;
  int aoff[2][FM], boff[2][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * TM + 32 * i + fr;
#pragma unroll
    for (int st = 0; st < 2; ++st) aoff[st][i] = r * ROWB + (((2 * st + fq) ^ swz(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int r;
    if constexpr (EPI == EPI_SILU_MUL) {
      constexpr int HF = FN / 2;
      r = (j < HF ? 0 : BN / 2) + wn * (TN / 2) + 32 * (j % HF) + fr;
    } else {
      r = wn * TN + 32 * j + fr;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) boff[st][j] = BM * ROWB + r * ROWB + (((2 * st + fq) ^ swz(r)) << 4);
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // A bare barrier: a workgroup fence here would also drain the later
  // slabs' loads; the empty asm statements keep the compiler from moving LDS
  // accesses across it.
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  bf16x8_t fa[2][2][FM], fb[2][2][FN];  // [register set][K step][fragment]
  auto read_frags = [&](int kt, int set) {
    const char* base = lds + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[set][st][i] = *(const bf16x8_t*)(base + aoff[st][i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[set][st][j] = *(const bf16x8_t*)(base + boff[st][j]);
    }
  };
  // MFMAs q in [lo, hi) of a slab: K step q / (FM FN), fragment
  // (q / FN % FM, q % FN)
  auto mfmas = [&](int set, int lo, int hi) {
#pragma unroll
    for (int q = lo; q < hi; ++q) {
      const int st = q / (FM * FN), i = (q / FN) % FM, j = q % FN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][st][i], fb[set][st][j], acc[i][j], 0, 0, 0);
    }
  };
  // Slab kt, whose fragments are in register set `set`.
  auto slab = [&](int kt, int set) {
    // Buffer (kt+3) % 4 held slab kt-1: every wavefront completed its reads
    // of it before the barrier of slab kt (lgkmcnt(0) below).
    issue(kt + 3, 0, LPRE);
    mfmas(set, 0, PRE);
    // MFMA q of them followed by its share of the LPRE loads
#pragma unroll
    for (int q = 0; q < PRE; ++q) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
#pragma unroll
      for (int r = q * LPRE / PRE; r < (q + 1) * LPRE / PRE; ++r) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Slab kt+1 landed (the LOADS loads of slab kt+2 and the LPRE of slab
    // kt+3 issued after it may still be in flight) and this wavefront's reads
    // of slab kt completed; after the barrier, the same holds for every
    // wavefront.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(LOADS + LPRE, 0));
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(kt + 1, set ^ 1);
    issue(kt + 3, LPRE, LOADS);
    mfmas(set, PRE, NMF);
    // the NREAD fragment reads one per MFMA, then the remaining loads spread
    // over the MFMAs left
    constexpr int NR = NMF - PRE, LREST = LOADS - LPRE;
    constexpr int DEN = NR > NREAD ? NR - NREAD : 1;
    static_assert(NR >= NREAD && (LREST == 0 || NR > NREAD), "schedule slots");
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 1);
      if (q < NREAD) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 1);
      else if (LREST > 0 && (q - NREAD) * LREST / DEN != (q + 1 - NREAD) * LREST / DEN)
        __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p) issue(p, 0, LOADS);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LOADS, 0));  // slab 0 landed
  barrier();
  if constexpr (PP) {
    // Ping-pong: wavefronts 0..3 and 4..7 (one of each per SIMD) run one
    // barrier interval apart.  In each interval one group issues its MFMAs on
    // the slab whose fragments it read in the previous interval, while the
    // other reads its fragments of a slab and issues its loads of the slab
    // three ahead.  Before every barrier a wavefront waits until its loads
    // of all but the two newest slabs have landed and its LDS reads are done:
    // a slab's loads then land before any group reads it, and a buffer is
    // refilled only after both groups read it.
    const bool late = wave >= NWV / 2;
    auto sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LOADS, 0));
      barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (late) sync();
    for (int kt = 0; kt < nk; ++kt) {
      read_frags(kt, 0);
      issue(kt + 3, 0, LOADS);
      sync();
      mfmas(0, 0, NMF);
      sync();
    }
    if (!late) sync();
  } else {
    read_frags(0, 0);
    // Two slabs per trip so the register sets are compile-time constants.
    // Past the last slab, read_frags reads a buffer whose fragments go unused.
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      slab(kt, 0);
      slab(kt + 1, 1);
    }
    if (kt < nk) mfmas(0, 0, NMF);  // odd slab count: the last slab is in set 0
  }
  // Drain the trailing loads before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  // Epilogue.  32 x 32 fragment element e of lane l: row 8 (e / 4) + 4 (l / 32)
  // + e % 4, column l % 32.
  const int ec = lane & 31, eq = (lane >> 5) * 4;
  if constexpr (EPI == EPI_SILU_MUL) {
    constexpr int HF = FN / 2;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < HF; ++j) {
        const int col = n0 + wn * (TN / 2) + 32 * j + ec;
        if (col >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * TM + 32 * i + 8 * (e >> 2) + eq + (e & 3);
          if (row < M)
            Elem<OutT>::store((OutT*)Cv, act_idx(row, col, ldc, (pk & PK_C) ? ldc : 0),
                              silu_f(acc[i][j][e]) * acc[i][j + HF][e]);
        }
      }
  } else {
    float* Cp = (float*)Cv + (EPI == EPI_PARTIAL ? split * slice_stride : 0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + 32 * j + ec;
        if (col >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * TM + 32 * i + 8 * (e >> 2) + eq + (e & 3);
          if (row >= M) continue;
          float* p = Cp + (long)row * ldc + col;
          if constexpr (EPI == EPI_RESID_F32) *p += acc[i][j][e];
          else *p = acc[i][j][e];
        }
      }
  }
}

// Decode-batch projection (M <= 16 * MF rows, weight-streaming).  A
// workgroup owns 16 * NF output columns (and, for SwiGLU, the matching up
// rows) for all rows; its NW wavefronts split K into contiguous ranges.  Each
// lane loads its fragment of the weight rows straight from global memory into
// MFMA registers, U k-steps at a time, so every wavefront keeps U x 16 x NB
// rows x 64 bytes in flight with no LDS staging.  Each weight byte is read
// once per launch: non-temporal loads (the activations, re-read by every
// workgroup, stay ordinary).  The wavefront partials meet
// in LDS and are summed in wavefront order (deterministic), then wavefront 0
// applies the fused epilogue.  The K partition depends only on K and NW, so a
// row's result does not depend on how many rows share the launch.
//
// With splits > 1 (EPI_PARTIAL) workgroup (tile, s) covers the s-th of
// `splits` contiguous K ranges and stores its fp32 partial tile to slice s
// (C + s * slice_stride); the kernel that next reads these rows sums the
// slices in slice order, so no workgroups ever wait on each other.
template <int MF, int NF, int NW, int U, int EPI, typename OutT, int LAY = 0>
__global__ void __launch_bounds__(64 * NW) gemv_bf16_kernel(const bf16_t* __restrict__ A, int lda,
                                                            const bf16_t* __restrict__ B, int ldb, int M, int N,
                                                            int K, void* __restrict__ Cv, int ldc, int splits,
                                                            long slice_stride, int pk) {
  constexpr int DUAL = (EPI == EPI_SILU_MUL) ? 2 : 1;
  constexpr int NB = NF * DUAL;  // B fragments per k-step (U k-steps in flight)
  __shared__ f32x4_t red[NW][MF * NB][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x / splits, split = blockIdx.x % splits;
  const int n0 = tile * 16 * NF;
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  const bf16_t* brow[NB];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n = n0 + 16 * f + fr;
    n = n < N ? n : N - 1;
#pragma unroll
    for (int dd = 0; dd < DUAL; ++dd) brow[f * DUAL + dd] = B + (long)(dd ? N + n : n) * ((pk & PK_B) ? 32 : ldb) + fk;
  }
  // elements between k-steps of 32: row-major, or one packed slab of ldb rows
  const long bstep = (pk & PK_B) ? (long)ldb * 32 : 32;
  // A K-slab-major (LAY bit 0): a k-step moves one slab block; row-major:
  // 32 elements (a constant, so the loads keep immediate offsets)
  const long astep = (LAY & 1) ? (long)lda * 32 : 32;
  const bf16_t* arow[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    int m = 16 * i + fr;
    m = m < M ? m : M - 1;
    arow[i] = A + (long)m * ((LAY & 1) ? 32 : lda) + fk;
  }
  const int steps = K / 32;
  const int sper = (steps + splits - 1) / splits;       // k-steps of this workgroup's split
  const int g0 = min(steps, split * sper), g1 = min(steps, g0 + sper);
  const int per = (g1 - g0 + NW - 1) / NW;
  const int s0 = min(g1, g0 + wave * per), s1 = min(g1, s0 + per);

  f32x4_t acc[MF][NB];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Rounds of up to U k-steps, every load of a round in flight before its
  // first MFMA; a short last round takes exactly its remaining steps (a
  // uniform switch into straight-line code -- predicated loads would be
  // waited for one by one).
  auto round = [&](auto r_const, int s) {
    constexpr int R = decltype(r_const)::value;
    bf16x8_t bv[R][NB], av[R][MF];
#pragma unroll
    for (int u = 0; u < R; ++u) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bv[u][j] = __builtin_nontemporal_load((const bf16x8_t*)(brow[j] + (s + u) * bstep));
#pragma unroll
      for (int i = 0; i < MF; ++i) av[u][i] = *(const bf16x8_t*)(arow[i] + (s + u) * astep);
    }
    // keep the scheduler from trading loads in flight for registers
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][i], bv[u][j], acc[i][j], 0, 0, 0);
  };
  int s = s0;
  for (; s + U <= s1; s += U) round(std::integral_constant<int, U>{}, s);
#define NS_GEMV_TAIL(R) \
  case R: if constexpr (U > R) round(std::integral_constant<int, (U > R ? R : 1)>{}, s); break;
  switch (s1 - s) {  // 0 .. U-1 steps left
    NS_GEMV_TAIL(1) NS_GEMV_TAIL(2) NS_GEMV_TAIL(3) NS_GEMV_TAIL(4) NS_GEMV_TAIL(5)
    NS_GEMV_TAIL(6) NS_GEMV_TAIL(7) NS_GEMV_TAIL(8) NS_GEMV_TAIL(9) NS_GEMV_TAIL(10)
    NS_GEMV_TAIL(11) NS_GEMV_TAIL(12) NS_GEMV_TAIL(13) NS_GEMV_TAIL(14) NS_GEMV_TAIL(15)
    default: break;
  }
#undef NS_GEMV_TAIL

#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) red[wave][i * NB + j][lane] = acc[i][j];
  __syncthreads();
  if (wave != 0) return;
  // wavefront 0 adds the others' partials in wavefront order (the outer loop
  // stays rolled so only the accumulators are live)
#pragma unroll 1
  for (int w = 1; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] += red[w][i * NB + j][lane];

  // Epilogue.  Fragment element r of lane l is row 4*(l/16)+r, column l%16.
  const int er = (lane >> 4) * 4, ec = lane & 15;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int col = n0 + 16 * f + ec;
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + er + r;
        if (row >= M) continue;
        if constexpr (EPI == EPI_SILU_MUL) {
          Elem<OutT>::store((OutT*)Cv, act_idx(row, col, ldc, (LAY & 2) ? ldc : 0),
                            silu_f(acc[i][2 * f][r]) * acc[i][2 * f + 1][r]);
        } else if constexpr (EPI == EPI_PARTIAL) {
          ((float*)Cv)[split * slice_stride + (long)row * ldc + col] = acc[i][f][r];
        } else {
          float* p = (float*)Cv + (long)row * ldc + col;
          if constexpr (EPI == EPI_RESID_F32) *p += acc[i][f][r];
          else *p = acc[i][f][r];
        }
      }
  }
}

// fp32 GEMM for fp32 models: 16x16 outputs per workgroup, K in LDS slabs.
template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const float* __restrict__ B, int ldb, int M, int N, int K,
                                                       float* __restrict__ Cp, int ldc) {
  __shared__ float As[16][17], Bs[16][17], Bs2[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
  float acc = 0.f, acc2 = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int ar = blockIdx.y * 16 + ty, bcol = blockIdx.x * 16 + ty;
    As[ty][tx] = (ar < M && k0 + tx < K) ? A[(long)ar * lda + k0 + tx] : 0.f;
    Bs[ty][tx] = (bcol < N && k0 + tx < K) ? B[(long)bcol * ldb + k0 + tx] : 0.f;
    if constexpr (EPI == EPI_SILU_MUL)
      Bs2[ty][tx] = (bcol < N && k0 + tx < K) ? B[(long)(N + bcol) * ldb + k0 + tx] : 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      acc = fmaf(As[ty][k], Bs[tx][k], acc);
      if constexpr (EPI == EPI_SILU_MUL) acc2 = fmaf(As[ty][k], Bs2[tx][k], acc2);
    }
    __syncthreads();
  }
  if (row >= M || col >= N) return;
  float* p = Cp + (long)row * ldc + col;
  if constexpr (EPI == EPI_RESID_F32) *p += acc;
  else if constexpr (EPI == EPI_SILU_MUL) *p = silu_f(acc) * acc2;
  else *p = acc;
}

template <int BM, int BN, int BK, int WM, int WN, int EPI>
static void run_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* Cv, int ldc,
                     hipStream_t st, int pk, int splits = 1, long slice_stride = 0) {
  constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? BN / 2 : BN;
  const long tiles = (long)((M + BM - 1) / BM) * ((N + OUT_BN - 1) / OUT_BN);
#define NS_TILE_LAUNCH(BNT_, LAY_)                                                                             \
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, EPI, bf16_t, BNT_, LAY_>),                           \
                     dim3((unsigned)tiles, (unsigned)splits), dim3(64 * WM * WN), 0, st, (const bf16_t*)A, lda, \
                     (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride, pk)
  // one row tile: each weight element is read once (non-temporal B); the
  // SwiGLU output's layout only exists for that epilogue
  const int lay = ((pk & PK_A) ? 1 : 0) | ((EPI == EPI_SILU_MUL && (pk & PK_C)) ? 2 : 0);
  if (M <= BM) {
    if constexpr (EPI == EPI_SILU_MUL) {
      if (lay == 3) NS_TILE_LAUNCH(1, 3);
      else if (lay == 2) NS_TILE_LAUNCH(1, 2);
      else if (lay == 1) NS_TILE_LAUNCH(1, 1);
      else NS_TILE_LAUNCH(1, 0);
    } else {
      if (lay & 1) NS_TILE_LAUNCH(1, 1);
      else NS_TILE_LAUNCH(1, 0);
    }
  } else {
    if constexpr (EPI == EPI_SILU_MUL) {
      if (lay == 3) NS_TILE_LAUNCH(0, 3);
      else if (lay == 2) NS_TILE_LAUNCH(0, 2);
      else if (lay == 1) NS_TILE_LAUNCH(0, 1);
      else NS_TILE_LAUNCH(0, 0);
    } else {
      if (lay & 1) NS_TILE_LAUNCH(0, 1);
      else NS_TILE_LAUNCH(0, 0);
    }
  }
#undef NS_TILE_LAUNCH
}

template <int EPI, int BM = 256>
static void run_big(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* Cv, int ldc,
                    hipStream_t st, int pk, int splits = 1, long slice_stride = 0) {
  constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? 128 : 256;
  const long tiles = (long)((M + BM - 1) / BM) * ((N + OUT_BN - 1) / OUT_BN);
  const dim3 grid((unsigned)tiles, (unsigned)splits);
  // 256-row tiles: 8 wavefronts in two ping-pong groups, the same bits as
  // 4 (measured on MI355X at 2048 rows of the 70B shape: QKV 383.6 -> 369.5,
  // O 261 -> 230.5, gate-up 1693 -> 1665, down 868 -> 847 us; at one row tile
  // of 256 rows, once A is K-slab-major, the 80-layer step 52.0 -> 51.2 ms,
  // where with a row-major A the gate-up projection had lost 7%)
  if (BM == 256 && M <= BM) {  // one row tile: each weight slab is read once (non-temporal)
    hipLaunchKernelGGL((gemm_big_kernel<EPI, bf16_t, 256, 1, 8, 1>), grid, dim3(512), 0, st, (const bf16_t*)A, lda,
                       (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride, pk);
  } else if (M <= BM) {
    hipLaunchKernelGGL((gemm_big_kernel<EPI, bf16_t, BM, 1>), grid, dim3(256), 0, st, (const bf16_t*)A, lda,
                       (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride, pk);
  } else if constexpr (BM == 256) {
    hipLaunchKernelGGL((gemm_big_kernel<EPI, bf16_t, BM, 0, 8, 1>), grid, dim3(512), 0, st, (const bf16_t*)A, lda,
                       (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride, pk);
  } else {
    hipLaunchKernelGGL((gemm_big_kernel<EPI, bf16_t, BM, 0>), grid, dim3(256), 0, st, (const bf16_t*)A, lda,
                       (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride, pk);
  }
}

template <int MF, int NF, int NW, int EPI>
static void run_gemv(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* Cv, int ldc,
                     hipStream_t st, int pk, int splits = 1, long slice_stride = 0) {
  constexpr int NB = NF * (EPI == EPI_SILU_MUL ? 2 : 1);
  // k-steps in flight, as registers allow (1024-thread workgroups get 128
  // VGPRs per lane); with at most 4 fragments per k-step, 16 (up to 256
  // VGPRs), so a wavefront's share of a split (the down projection at 32
  // rows: 10 k-steps) or of the gate-up projection at 17-32 rows (14) is one
  // round of loads (the 0.5B-shaped mix at 32 rows 1.129 -> 1.118 ms against
  // 8 for 4 fragments); up to 6 fragments, 8 (the 33-64-row projections: at
  // 64 rows 1.367 -> 1.341 ms against 4)
  constexpr int U = NW >= 16 ? ((MF + NB) <= 4 ? 4 : 2) : ((MF + NB) <= 4 ? 16 : ((MF + NB) <= 6 ? 8 : 4));
  const unsigned grid = (unsigned)((N + 16 * NF - 1) / (16 * NF) * splits);
#define NS_GEMV_LAUNCH(LAY_)                                                                             \
  hipLaunchKernelGGL((gemv_bf16_kernel<MF, NF, NW, U, EPI, bf16_t, LAY_>), dim3(grid), dim3(64 * NW), 0, st, \
                     (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride, pk)
  // the SwiGLU output's layout only exists for that epilogue
  const int lay = ((pk & PK_A) ? 1 : 0) | ((EPI == EPI_SILU_MUL && (pk & PK_C)) ? 2 : 0);
  if constexpr (EPI == EPI_SILU_MUL) {
    if (lay == 3) NS_GEMV_LAUNCH(3);
    else if (lay == 2) NS_GEMV_LAUNCH(2);
    else if (lay == 1) NS_GEMV_LAUNCH(1);
    else NS_GEMV_LAUNCH(0);
  } else {
    if (lay & 1) NS_GEMV_LAUNCH(1);
    else NS_GEMV_LAUNCH(0);
  }
#undef NS_GEMV_LAUNCH
}

// Tile shapes for M > 64 rows, largest first: 256 x 256 and 128 x 256 (the
// big kernel), 128 x 128 and 64 x 64 (the LDS double-buffered kernel).
enum TileKind { TILE_BIG = 0, TILE_BIG128 = 1, TILE_128 = 2, TILE_64 = 3 };
constexpr int kTileRows[4] = {256, 128, 128, 64};
constexpr int kTileCols[4] = {256, 256, 128, 64};
constexpr int kFillTarget = 256;  // workgroups that fill the chip (one per CU)

// The big kernel addresses its operands with 32-bit buffer offsets.
static bool big_fits(int M, int lda, long b_rows, int ldb, int K, int pk) {
  const long a_span = (pk & PK_A) ? ((long)(K / 32 - 1) * lda + M) * 64 : (long)M * lda * 2;
  return a_span < (1L << 32) && ((pk & PK_B) ? (long)K * ldb : b_rows * ldb) * 2 < (1L << 32);
}

// Output tiles of a launch; SwiGLU tiles hold gate and up columns, so they
// cover half as many output columns.
static long tile_count(int kind, int M, int N, bool swiglu) {
  const int cols = swiglu ? kTileCols[kind] / 2 : kTileCols[kind];
  return (long)((M + kTileRows[kind] - 1) / kTileRows[kind]) * ((N + cols - 1) / cols);
}

// Split-K plan for M > 64 rows: the largest tile whose tiles x splits fill
// the chip with at least 4 K slabs of 32 per split; failing that, the one
// with the most workgroups.
struct PartialPlan {
  int kind, splits;
};
static PartialPlan partial_plan(int M, int N, int K) {
  const int slabs = K / 32;
  const int max_s = std::max(1, std::min(8, slabs / 4));
  PartialPlan best{TILE_64, 1};
  long best_wg = -1;
  for (int kind = (M > 128 ? TILE_BIG : TILE_BIG128); kind <= TILE_64; ++kind) {
    const long tiles = tile_count(kind, M, N, false);
    if (kind <= TILE_BIG128) {
      // one big-tile workgroup per CU: a split count that fills at least 3/4
      // of one wave beats one that spills a few workgroups into a second
      // (70B-shaped QKV at 256 rows: 40 tiles x 6 = 240, not x 7 = 280)
      const int s1 = (int)std::max(1L, std::min((long)max_s, kFillTarget / tiles));
      if (4 * tiles * s1 >= 3 * kFillTarget) return {kind, s1};
    }
    // 64 x 64 tiles take every split K allows: several small workgroups per
    // CU with short K ranges hide latency better than just filling the chip
    // (0.5B-shaped step at 256 rows: down projection 26 -> 20 us in the step,
    // QKV and O 1 us each, the step 2.66 -> 2.48 ms)
    const int s = kind == TILE_64 ? max_s
                                  : (int)std::max(1L, std::min((long)max_s, (kFillTarget + tiles - 1) / tiles));
    if (tiles * s >= kFillTarget) return {kind, s};
    if (tiles * s > best_wg) {
      best_wg = tiles * s;
      best = {kind, s};
    }
  }
  return best;
}

int gemm_partial_splits(int M, int N, int K) {
  if (M <= 64) {  // weight-streaming kernel: 16-column tiles
    const int steps = K / 32;
    const int tiles = (N + 15) / 16;
    return std::max(1, std::min(8, std::min(steps / 8, 512 / std::max(1, tiles))));
  }
  return partial_plan(M, N, K).splits;
}

int launch_gemm_partial(int M, int N, int K, const void* A, int lda, const void* B, int ldb, float* P, int ldp,
                        long slice_stride, int splits, hipStream_t st, int pack) {
  const int pk = pack & (PK_A | PK_B);  // the slices are fp32 row-major
  if (M <= 0 || N <= 0) return 0;
  if (K % 32 != 0 || splits < 1 || splits > K / 32) return -1;
  if (M <= 64) {
    // two wavefronts per workgroup; 32 output columns per workgroup when
    // that still leaves a workgroup per CU (measured best on MI355X at
    // decode sizes)
    const bool nf2 = (long)((N + 31) / 32) * splits >= 256;
#define NS_GEMV_PART(MF)                                                                             \
  do {                                                                                               \
    if (nf2) run_gemv<MF, 2, 2, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride); \
    else run_gemv<MF, 1, 2, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);     \
  } while (0)
    if (M <= 16) NS_GEMV_PART(1);
    else if (M <= 32) NS_GEMV_PART(2);
    else NS_GEMV_PART(4);
#undef NS_GEMV_PART
  } else {
    int kind = partial_plan(M, N, K).kind;
    if ((kind == TILE_BIG || kind == TILE_BIG128) && !big_fits(M, lda, N, ldb, K, pk)) kind = TILE_128;
    if (kind == TILE_BIG) run_big<EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);
    else if (kind == TILE_BIG128)
      run_big<EPI_PARTIAL, 128>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);
    else if (kind == TILE_128)
      run_bf16<128, 128, 32, 2, 2, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);
    // Wide K slabs where every split still gets one: fewer slab syncs
    // (0.5B-shaped mix, down projection at 128 rows: 32-wide 18.5 us, 64-wide
    // 14.6 us, 128-wide 12.2 us)
    else if (K % 128 == 0 && K / 128 >= splits)
      run_bf16<64, 64, 128, 2, 2, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);
    else if (K % 64 == 0 && K / 64 >= splits)
      run_bf16<64, 64, 64, 2, 2, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);
    else run_bf16<64, 64, 32, 2, 2, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, pk, splits, slice_stride);
  }
  return 0;
}

// Decode batches (M <= 64): the weight-streaming kernel.  Wide column tiles
// where N alone gives plenty of workgroups (the LM head: 64 columns and two
// wavefronts at 1..16 and 33..64 rows, 128 and two at 17..32 -- fewer
// re-reads of the activations; measured at 64 rows: 117 -> 84 us against
// four wavefronts); for long K as many
// K-splitting wavefronts as the LDS for their partial sums allows (<= 64 KB).
template <int MF, int EPI>
static void dispatch_gemv_m(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                            hipStream_t st, int pk) {
  constexpr int NB1 = EPI == EPI_SILU_MUL ? 2 : 1;
  constexpr int NW_LONG = (64 / (MF * NB1)) < 16 ? (64 / (MF * NB1)) : 16;
  const bool wide = (long)N / 64 >= 1024;
  if constexpr (EPI != EPI_SILU_MUL) {
    // measured on MI355X (LM head, N 151936, K 896; isolated and in the step)
    if (wide) {
      if constexpr (MF == 1) return run_gemv<MF, 4, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
      else if constexpr (MF == 2) return run_gemv<MF, 8, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
      else return run_gemv<MF, 4, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
    }
  }
  if (K > 2048) run_gemv<MF, 1, NW_LONG, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  else run_gemv<MF, 1, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
}

template <int EPI>
static void dispatch_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                          hipStream_t st, int pk) {
  if (M <= 16) return dispatch_gemv_m<1, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  if (M <= 32) return dispatch_gemv_m<2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  if (M <= 64) return dispatch_gemv_m<4, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  // M > 64: the tile shape with the best estimated throughput -- its
  // relative per-CU rate (measured on MI355X: the 256 x 256 kernel 1.0,
  // 128 x 256 about 0.72, 128 x 128 about 0.55, 64 x 64 about 0.35) times the
  // fill of its last wave of workgroups (256 resident at a time for the big
  // kernel, 512 and 1024 for the LDS-light ones).  The big kernel needs
  // 32-bit offsets, and 256-row tiles more than 128 rows.
  const bool k64 = (K % 64) == 0;
  const long b_rows = (EPI == EPI_SILU_MUL) ? 2L * N : (long)N;
  constexpr double kRate[4] = {1.0, 0.72, 0.55, 0.35};
  constexpr long kSlots[4] = {256, 256, 512, 1024};
  const bool fits = big_fits(M, lda, b_rows, ldb, K, pk);
  int kind = TILE_64;
  double best = -1.0;
  for (int k = (fits ? (M > 128 ? TILE_BIG : TILE_BIG128) : TILE_128); k <= TILE_64; ++k) {
    const long t = tile_count(k, M, N, EPI == EPI_SILU_MUL);
    const double fill = (double)t / (double)(kSlots[k] * ((t + kSlots[k] - 1) / kSlots[k]));
    // a big-tile launch that leaves most of the chip idle loses to smaller
    // tiles spread over more CUs (measured: SwiGLU at 128-256 rows, K 896)
    if (k <= TILE_BIG128 && 2 * t < kSlots[k]) continue;
    if (kRate[k] * fill > best + 1e-9) {
      best = kRate[k] * fill;
      kind = k;
    }
  }
  if (kind == TILE_BIG) return run_big<EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  if (kind == TILE_BIG128) return run_big<EPI, 128>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  if (kind == TILE_128) {
    if (k64) run_bf16<128, 128, 64, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
    else run_bf16<128, 128, 32, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  } else {
    constexpr int BN64 = (EPI == EPI_SILU_MUL) ? 128 : 64;
    // SwiGLU tiles that fit one wave of workgroups take 128-wide K slabs
    // (104 KB of LDS, one workgroup per CU): gate-up at 128 rows of the
    // 0.5B shape 20.8 -> 16.8 us; with more tiles than CUs the second wave
    // costs more than that saves (256 rows: 21 -> 27 us)
    if (EPI == EPI_SILU_MUL && K % 128 == 0 && tile_count(TILE_64, M, N, false) <= kFillTarget)
      run_bf16<64, BN64, 128, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
    else if (k64) run_bf16<64, BN64, 64, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
    else run_bf16<64, BN64, 32, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st, pk);
  }
}

int gemm_supported(int dtype, int K) { return dtype == NS_DT_F32 ? K > 0 : (K > 0 && K % 32 == 0); }

// Row-major [rows, cols] bf16 -> K-slab-major: thread = one 16-byte piece.
__global__ void __launch_bounds__(256) pack_kslab_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                         int rows, int cols) {
  const long c = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = cols / 8;
  if (c >= (long)rows * per_row) return;
  const int n = (int)(c / per_row), k = (int)(c % per_row) * 8;
  *(u32x4_t*)(dst + ((long)(k >> 5) * rows + n) * 32 + (k & 31)) = *(const u32x4_t*)(src + (long)n * cols + k);
}

void launch_pack_kslab(const void* src, void* dst, int rows, int cols, hipStream_t st) {
  const long pieces = (long)rows * (cols / 8);
  if (pieces <= 0) return;
  hipLaunchKernelGGL(pack_kslab_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, (const bf16_t*)src,
                     (bf16_t*)dst, rows, cols);
}

int launch_gemm(int dtype, int epi, int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
                int ldc, hipStream_t st, int pack) {
  if (M <= 0 || N <= 0) return 0;
  if (!gemm_supported(dtype, K) || (pack && dtype != NS_DT_BF16)) return -1;
  // a slab-major C needs whole 32-column slabs and only the SwiGLU epilogue writes bf16
  if ((pack & PK_C) && (epi != EPI_SILU_MUL || N % 32 != 0)) return -1;
  const int pk = pack;
  if (dtype == NS_DT_F32) {
    dim3 grid((N + 15) / 16, (M + 15) / 16);
    const float* a = (const float*)A;
    const float* b = (const float*)B;
    float* c = (float*)C;
    switch (epi) {
      case EPI_STORE_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE_F32>, grid, dim3(256), 0, st, a, lda, b, ldb, M, N, K, c, ldc); break;
      case EPI_RESID_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID_F32>, grid, dim3(256), 0, st, a, lda, b, ldb, M, N, K, c, ldc); break;
      default: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SILU_MUL>, grid, dim3(256), 0, st, a, lda, b, ldb, M, N, K, c, ldc); break;
    }
    return 0;
  }
  switch (epi) {
    case EPI_STORE_F32: dispatch_bf16<EPI_STORE_F32>(M, N, K, A, lda, B, ldb, C, ldc, st, pk); break;
    case EPI_RESID_F32: dispatch_bf16<EPI_RESID_F32>(M, N, K, A, lda, B, ldb, C, ldc, st, pk); break;
    default: dispatch_bf16<EPI_SILU_MUL>(M, N, K, A, lda, B, ldb, C, ldc, st, pk); break;
  }
  return 0;
}

}  // namespace ns
