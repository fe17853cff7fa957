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

template <int EPI>
static void dispatch_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                          hipStream_t st) {
  const bool k64 = (K % 64) == 0;
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
