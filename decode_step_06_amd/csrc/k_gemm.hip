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

template <int BM, int BN, int BK, int WM, int WN, int EPI, typename OutT>
__global__ void __launch_bounds__(64 * WM * WN) gemm_bf16_kernel(const bf16_t* __restrict__ A, int lda,
                                                                 const bf16_t* __restrict__ B, int ldb, int M, int N,
                                                                 int K, void* __restrict__ Cv, int ldc) {
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
        const int r = c / (BK / 8), k8 = c % (BK / 8);
        ra[i] = *(const u32x4_t*)(A + (long)a_row(r) * lda + k0 + k8 * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PT; ++i) {
      const int c = tid + i * C::NT;
      if (c < C::B_CH) {
        const int r = c / (BK / 8), k8 = c % (BK / 8);
        rb[i] = *(const u32x4_t*)(B + (long)b_row(r) * ldb + k0 + k8 * 8);
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

  const int nk = K / BK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;  // fragment row / k offset of this lane
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slab((kt + 1) * BK);
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
          if (row < M) Elem<OutT>::store(Cp, (long)row * ldc + col, silu_f(acc[i][j][r]) * acc[i][j + HF][r]);
        }
      }
  } else {
    float* Cp = (float*)Cv;
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

// Dense-batch projection (M >= 256): a 256 x 256 output tile per workgroup,
// 8 wavefronts in a 2 x 4 grid each owning a 128 x 64 sub-tile (8 x 4
// fragments, 128 accumulators per lane), K in 64-wide slabs through
// double-buffered padded LDS (2 x 72 KB).  A wavefront tile this large needs
// 3/4 of the LDS bytes per MFMA of a 64 x 64 one.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so workgroup b runs on XCD b % 8; giving each XCD a contiguous range
// of tiles, M-fastest, makes the 32 tiles an XCD runs at once share their B
// columns in that XCD's private L2 while walking down A.
template <int EPI, typename OutT>
__global__ void __launch_bounds__(512) gemm_big_kernel(const bf16_t* __restrict__ A, int lda,
                                                       const bf16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                       void* __restrict__ Cv, int ldc) {
  constexpr int BM = 256, BN = 256, BK = 64, LDK = BK + 8;
  constexpr int TM = 128, TN = 64, FM = 8, FN = 4, NT = 512;
  constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? BN / 2 : BN;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * (BM + BN) * LDK];  // 144 KB of the 160 KB
  bf16_t* As = lds;                      // [2][BM * LDK]
  bf16_t* Bs = lds + 2 * BM * LDK;       // [2][BN * LDK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int m_tiles = (M + BM - 1) / BM;
  const int n_tiles = (N + OUT_BN - 1) / OUT_BN;
  const int tiles = m_tiles * n_tiles;
  int tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int tile_m = tile % m_tiles, tile_n = tile / m_tiles;
  const int m0 = tile_m * BM, n0 = tile_n * OUT_BN;

  auto a_row = [&](int r) { int m = m0 + r; return m < M ? m : M - 1; };
  auto b_row = [&](int r) {
    if constexpr (EPI == EPI_SILU_MUL) {
      int n = n0 + (r < BN / 2 ? r : r - BN / 2);
      n = n < N ? n : N - 1;
      return r < BN / 2 ? n : N + n;
    } else {
      int n = n0 + r;
      return n < N ? n : N - 1;
    }
  };
  // 4 A chunks + 4 B chunks of 16 bytes per thread per slab
  constexpr int PT = BM * BK / 8 / NT;
  const bf16_t* ga[PT];
  const bf16_t* gb[PT];
  int la[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3, k8 = c & 7;
    ga[i] = A + (long)a_row(r) * lda + k8 * 8;
    gb[i] = B + (long)b_row(r) * ldb + k8 * 8;
    la[i] = r * LDK + k8 * 8;
  }
  u32x4_t ra[PT], rb[PT];
  auto load_slab = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      ra[i] = *(const u32x4_t*)(ga[i] + k0);
      rb[i] = *(const u32x4_t*)(gb[i] + k0);
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      *(u32x4_t*)&As[buf * BM * LDK + la[i]] = ra[i];
      *(u32x4_t*)&Bs[buf * BN * LDK + la[i]] = rb[i];
    }
  };
  auto b_frag_row = [&](int f) {
    if constexpr (EPI == EPI_SILU_MUL) {
      constexpr int HF = FN / 2;
      return (f < HF ? 0 : BN / 2) + wn * (TN / 2) + 16 * (f % HF);
    } else {
      return wn * TN + 16 * f;
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slab((kt + 1) * BK);
    const bf16_t* Ab = As + buf * BM * LDK;
    const bf16_t* Bb = Bs + buf * BN * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const bf16x8_t*)&Ab[(wm * TM + 16 * i + fr) * LDK + kk + fk];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *(const bf16x8_t*)&Bb[(b_frag_row(j) + fr) * LDK + kk + fk];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slab(buf ^ 1);
    __syncthreads();
  }

  const int er = (lane >> 4) * 4, ec = lane & 15;
  if constexpr (EPI == EPI_SILU_MUL) {
    constexpr int HF = FN / 2;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < HF; ++j) {
        const int col = n0 + wn * (TN / 2) + 16 * j + ec;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * TM + 16 * i + er + r;
          if (row < M)
            Elem<OutT>::store((OutT*)Cv, (long)row * ldc + col, silu_f(acc[i][j][r]) * acc[i][j + HF][r]);
        }
      }
  } else {
    float* Cp = (float*)Cv;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + 16 * j + ec;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * TM + 16 * i + er + r;
          if (row >= M) continue;
          float* p = Cp + (long)row * ldc + col;
          if constexpr (EPI == EPI_RESID_F32) *p += acc[i][j][r];
          else *p = acc[i][j][r];
        }
      }
  }
}

// Decode-batch projection (M <= 16 * MF rows, weight-streaming).  A
// workgroup owns 16 * NF output columns (and, for SwiGLU, the matching up
// rows) for all rows; its NW wavefronts split K into contiguous ranges.  Each
// lane loads its fragment of the weight rows straight from global memory into
// MFMA registers, U k-steps at a time, so every wavefront keeps U x 16 x NB
// rows x 64 bytes in flight with no LDS staging.  The wavefront partials meet
// in LDS and are summed in wavefront order (deterministic), then wavefront 0
// applies the fused epilogue.  The K partition depends only on K and NW, so a
// row's result does not depend on how many rows share the launch.
//
// With splits > 1 (EPI_PARTIAL) workgroup (tile, s) covers the s-th of
// `splits` contiguous K ranges and stores its fp32 partial tile to slice s
// (C + s * slice_stride); the kernel that next reads these rows sums the
// slices in slice order, so no workgroups ever wait on each other.
template <int MF, int NF, int NW, int U, int EPI, typename OutT>
__global__ void __launch_bounds__(64 * NW) gemv_bf16_kernel(const bf16_t* __restrict__ A, int lda,
                                                            const bf16_t* __restrict__ B, int ldb, int M, int N,
                                                            int K, void* __restrict__ Cv, int ldc, int splits,
                                                            long slice_stride) {
  constexpr int DUAL = (EPI == EPI_SILU_MUL) ? 2 : 1;
  constexpr int NB = NF * DUAL;  // B fragments per k-step (U k-steps in flight)
  __shared__ f32x4_t red[NW][MF * NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x / splits, split = blockIdx.x % splits;
  const int n0 = tile * 16 * NF;
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  const bf16_t* brow[NB];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n = n0 + 16 * f + fr;
    n = n < N ? n : N - 1;
#pragma unroll
    for (int dd = 0; dd < DUAL; ++dd) brow[f * DUAL + dd] = B + (long)(dd ? N + n : n) * ldb + fk;
  }
  const bf16_t* arow[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    int m = 16 * i + fr;
    m = m < M ? m : M - 1;
    arow[i] = A + (long)m * lda + fk;
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

  int s = s0;
  for (; s + U <= s1; s += U) {
    bf16x8_t bv[U][NB], av[U][MF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < NB; ++j) bv[u][j] = *(const bf16x8_t*)(brow[j] + (s + u) * 32);
#pragma unroll
      for (int i = 0; i < MF; ++i) av[u][i] = *(const bf16x8_t*)(arow[i] + (s + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][i], bv[u][j], acc[i][j], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    bf16x8_t bv[NB], av[MF];
#pragma unroll
    for (int j = 0; j < NB; ++j) bv[j] = *(const bf16x8_t*)(brow[j] + s * 32);
#pragma unroll
    for (int i = 0; i < MF; ++i) av[i] = *(const bf16x8_t*)(arow[i] + s * 32);
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) red[wave][i * NB + j][lane] = acc[i][j];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      f32x4_t a = red[0][i * NB + j][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) a += red[w][i * NB + j][lane];
      acc[i][j] = a;
    }

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
          Elem<OutT>::store((OutT*)Cv, (long)row * ldc + col, silu_f(acc[i][2 * f][r]) * acc[i][2 * f + 1][r]);
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
                     hipStream_t st) {
  constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? BN / 2 : BN;
  const long tiles = (long)((M + BM - 1) / BM) * ((N + OUT_BN - 1) / OUT_BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, EPI, bf16_t>), dim3((unsigned)tiles), dim3(64 * WM * WN),
                     0, st, (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K, Cv, ldc);
}

template <int MF, int NF, int NW, int EPI>
static void run_gemv(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* Cv, int ldc,
                     hipStream_t st, int splits = 1, long slice_stride = 0) {
  constexpr int NB = NF * (EPI == EPI_SILU_MUL ? 2 : 1);
  constexpr int U = (MF + NB) <= 4 ? 8 : 4;  // k-steps in flight, as registers allow
  const unsigned grid = (unsigned)((N + 16 * NF - 1) / (16 * NF) * splits);
  hipLaunchKernelGGL((gemv_bf16_kernel<MF, NF, NW, U, EPI, bf16_t>), dim3(grid), dim3(64 * NW), 0, st,
                     (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K, Cv, ldc, splits, slice_stride);
}

int gemm_partial_splits(int N, int K) {
  const int steps = K / 32;
  const int tiles = (N + 15) / 16;
  return std::max(1, std::min(8, std::min(steps / 8, 512 / std::max(1, tiles))));
}

int launch_gemm_partial(int M, int N, int K, const void* A, int lda, const void* B, int ldb, float* P, int ldp,
                        long slice_stride, int splits, hipStream_t st) {
  if (M <= 0 || N <= 0) return 0;
  if (M > 64 || K % 32 != 0 || splits < 1) return -1;
  if (M <= 16) run_gemv<1, 1, 4, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, splits, slice_stride);
  else if (M <= 32) run_gemv<2, 1, 4, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, splits, slice_stride);
  else run_gemv<4, 1, 4, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, P, ldp, st, splits, slice_stride);
  return 0;
}

// Decode batches (M <= 64): the weight-streaming kernel.  Wide column tiles
// where N alone gives plenty of workgroups (the LM head); for long K as many
// K-splitting wavefronts as the LDS for their partial sums allows (<= 64 KB).
template <int MF, int EPI>
static void dispatch_gemv_m(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                            hipStream_t st) {
  constexpr int NB1 = EPI == EPI_SILU_MUL ? 2 : 1;
  constexpr int NW_LONG = (64 / (MF * NB1)) < 16 ? (64 / (MF * NB1)) : 16;
  const bool wide = (long)N / 64 >= 1024;
  if constexpr (EPI != EPI_SILU_MUL) {
    if (wide) return run_gemv<MF, 4, 4, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  }
  if (K > 2048) run_gemv<MF, 1, NW_LONG, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  else run_gemv<MF, 1, 4, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
}

template <int EPI>
static void dispatch_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                          hipStream_t st) {
  if (M <= 16) return dispatch_gemv_m<1, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  if (M <= 32) return dispatch_gemv_m<2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  if (M <= 64) return dispatch_gemv_m<4, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  const bool k64 = (K % 64) == 0;
  if (M >= 256 && k64 && N >= 256) {
    constexpr int OUT_BN = (EPI == EPI_SILU_MUL) ? 128 : 256;
    const long tiles = (long)((M + 255) / 256) * ((N + OUT_BN - 1) / OUT_BN);
    hipLaunchKernelGGL((gemm_big_kernel<EPI, bf16_t>), dim3((unsigned)tiles), dim3(512), 0, st, (const bf16_t*)A,
                       lda, (const bf16_t*)B, ldb, M, N, K, C, ldc);
    return;
  }
  // The SwiGLU tile pairs gate and up fragments, so its wave tile needs at
  // least two B fragments.
  constexpr int BN16 = (EPI == EPI_SILU_MUL) ? 128 : 64;
  if (M <= 16) {
    if (k64) run_bf16<16, BN16, 64, 1, 4, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
    else run_bf16<16, BN16, 32, 1, 4, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  } else if (M <= 32) {
    if (k64) run_bf16<32, 64, 64, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
    else run_bf16<32, 64, 32, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  } else if (M <= 64) {
    if (k64) run_bf16<64, 64, 64, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
    else run_bf16<64, 64, 32, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  } else {
    if (k64) run_bf16<128, 128, 64, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
    else run_bf16<128, 128, 32, 2, 2, EPI>(M, N, K, A, lda, B, ldb, C, ldc, st);
  }
}

int gemm_supported(int dtype, int K) { return dtype == NS_DT_F32 ? K > 0 : (K > 0 && K % 32 == 0); }

int launch_gemm(int dtype, int epi, int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
                int ldc, hipStream_t st) {
  if (M <= 0 || N <= 0) return 0;
  if (!gemm_supported(dtype, K)) return -1;
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
    case EPI_STORE_F32: dispatch_bf16<EPI_STORE_F32>(M, N, K, A, lda, B, ldb, C, ldc, st); break;
    case EPI_RESID_F32: dispatch_bf16<EPI_RESID_F32>(M, N, K, A, lda, B, ldb, C, ldc, st); break;
    default: dispatch_bf16<EPI_SILU_MUL>(M, N, K, A, lda, B, ldb, C, ldc, st); break;
  }
  return 0;
}

}  // namespace ns
