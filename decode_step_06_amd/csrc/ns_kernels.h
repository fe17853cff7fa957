// Host-side launchers of the gfx950 decode-step kernels (device code in
// k_*.hip).  Every launcher only enqueues on the given stream; argument
// checking happens in the engine before anything is enqueued.
#pragma once

#include "ns_common.h"

#define NS_DT_F32 0
#define NS_DT_BF16 1

namespace ns {

// GEMM epilogues: C = A * B^T (A [M, K], B [N, K], both K-contiguous).
enum GemmEpi {
  EPI_STORE_F32 = 0,  // C fp32 [M, N] = acc
  EPI_RESID_F32 = 1,  // C fp32 [M, N] += acc              (projection + residual add)
  EPI_SILU_MUL = 2,   // C (dtype) [M, N] = silu(acc_gate) * acc_up, with the gate rows of B at
                      // [0, N) and the up rows at [N, 2N)    (gate-up projection + SwiGLU)
  EPI_PARTIAL = 3,    // C fp32 slice s [M, N] = acc over the s-th K range (split K, decode batches)
};

// Operand layouts (bf16 only), a bit mask:
//  PK_B: B is stored K-slab-major, element (n, k) at ((k / 32) * ldb + n) * 32
//        + k % 32 with ldb = B's row count (N, or 2N for SwiGLU), so each
//        32-wide K slab of every row is one 64-byte piece of a contiguous
//        [rows][32] block; otherwise row-major with row stride ldb.
//  PK_A: A is K-slab-major the same way, lda = the rows of each slab block
//        (at least M; A may point at a row inside the block).
//  PK_C: the SwiGLU epilogue's bf16 C is written K-slab-major, ldc = the
//        rows of each slab block (N % 32 == 0).
enum GemmPack { PK_B = 1, PK_A = 2, PK_C = 4 };

// Returns 0, or -1 when the shape is unsupported (K % 32 != 0 for bf16).
int launch_gemm(int dtype, int epi, int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
                int ldc, hipStream_t st, int pack = 0);
int gemm_supported(int dtype, int K);

// Split-K projection (bf16): slice s of the result (P + s * slice_stride,
// [M, N] with row stride ldp) holds the sum over the s-th of `splits`
// contiguous ranges of K's 32-wide slabs; the consumer sums the slices in
// order.  gemm_partial_splits picks the split count that fills the chip for
// this shape (for M <= 64 from N and K alone).  Any 1 <= splits <= K / 32
// is accepted.  Returns -1 for unsupported shapes.
int gemm_partial_splits(int M, int N, int K);
int launch_gemm_partial(int M, int N, int K, const void* A, int lda, const void* B, int ldb, float* P, int ldp,
                        long slice_stride, int splits, hipStream_t st, int pack = 0);
// Row-major bf16 [rows, cols] -> K-slab-major (cols % 32 == 0).
void launch_pack_kslab(const void* src, void* dst, int rows, int cols, hipStream_t st);

void launch_embed(int dtype, const void* E, const int32_t* tok, float* x, int T, int H, int V, hipStream_t st);
void launch_copy_rows(const float* src, float* dst, long n, hipStream_t st);
void launch_rope_table(const int32_t* pos, float* cosb, float* sinb, int T, int d, float base, hipStream_t st);
// h_slab_rows: 0 = h row-major [T, H]; otherwise h is K-slab-major with that
// many rows per slab block (see act_idx), h pointing at the first row.
void launch_rmsnorm(int dtype, const float* x, const void* g, void* h, int T, int H, float eps, hipStream_t st,
                    int h_slab_rows = 0);
// tokens out[r] = argmax of row r of fp32 logits [n_rows, V] (lowest index
// among equal maxima, NaN never wins, a row of NaN only gives 0)
void launch_argmax_rows(const float* logits, int n_rows, int V, int32_t* out, hipStream_t st);
constexpr int kReadStreamGrid = 2048;  // workgroups of the streaming read (= NS_READ_STREAM_WORDS)
void launch_read_stream(const void* src, long n16, uint32_t* sink, hipStream_t st);
// x[t] += sum_s P[s][t] (slice order; the split-K residual add of the
// previous projection), written back to x, then RMSNorm into h.
void launch_rmsnorm_reduce(int dtype, float* x, const float* P, long slice_stride, int splits, const void* g,
                           void* h, int T, int H, float eps, hipStream_t st, int h_slab_rows = 0);
// out[t] = x[t] + sum_s P[s][t]  (the last layer's residual add, fp32 out)
void launch_reduce_rows(const float* x, const float* P, long slice_stride, int splits, float* out, int T, int H,
                        hipStream_t st);
// Embedding (E non-null) or hidden input already in x, RoPE cos/sin table,
// and layer 0's RMSNorm, one workgroup per row.  Rows whose token id lies
// outside [0, V) gather the nearest valid row and add 1 to *bad_tok (may be
// null).
void launch_step_prologue(int dtype, const void* E, const int32_t* tok, float* x, const int32_t* pos, float* cosb,
                          float* sinb, const void* g0, void* h, int T, int H, int V, int d, float base, float eps,
                          int32_t* bad_tok, hipStream_t st, int h_slab_rows = 0);
// qkv holds `splits` fp32 slices (slice_stride apart) that are summed first.
void launch_rope_kv(int dtype, const float* qkv, long slice_stride, int splits, const float* cosb,
                    const float* sinb, const int32_t* slot, void* q_att, void* kc, void* vc, int T, int nq, int nkv,
                    int d, hipStream_t st);
void launch_kv_scatter(int dtype, const int32_t* slots, const void* k, const void* v, void* kc, void* vc, int n,
                       int nkv, int d, hipStream_t st);
void launch_kv_gather(int dtype, const int32_t* slots, void* k, void* v, const void* kc, const void* vc, int n,
                      int nkv, int d, hipStream_t st);

// Paged GQA decode attention over rows [row0, row0 + n_rows) of the step.
struct AttnArgs {
  int dtype;
  const void* q_att;        // [T][nkv][d/E][G][E]
  const void* kc;           // this layer's K region
  const void* vc;           // this layer's V region
  const int32_t* row_bseq;  // [T] row -> block-table row (-1: padding); null: btab has one row per row
                            // (padding rows: first entry -1)
  const int32_t* row_pos;   // [T]
  const int32_t* btab;      // [n_bseq][maxb]
  int maxb;
  void* out;                // [T][nq * d] (dtype), or K-slab-major when out_slab_rows > 0 (bf16)
  float* part_acc;          // [T * nkv * n_parts][G][d]
  float* part_ml;           // [T * nkv * n_parts][G][2]
  int row0, n_rows;
  int nq, nkv, d;
  int part_tokens;          // P, multiple of 64
  int n_parts;              // partitions per row (max)
  int waves;                // wavefronts per work item: 1, 4 or 8 (fp32: 8 runs as 4)
  int wg_cap;               // 0 = one workgroup per work item
  const int32_t* row_seq;   // [T] sequence of each row (-1: padding), or null: no prefill tiles
  // RoPE and the row's own K/V write fused into the bf16 matrix-core kernel
  // (rows of distinct sequences only): null = q from q_att, the row's K/V
  // already in the cache.
  const float* rope_qkv = nullptr;  // [T][(nq + 2 nkv) d] fp32; slice s at + s * rope_slice_stride
  long rope_slice_stride = 0;
  int rope_splits = 1;
  const float* cosb = nullptr;      // [T][d/2]
  const float* sinb = nullptr;
  const int32_t* slot = nullptr;    // [T] cache slot of each row (-1: none)
  // bf16 matrix-core kernel: the order of its rows, row_order[row0 .. row0 +
  // n_rows) a permutation of those row indices (null: index order).  Rows are
  // independent, so the order changes no result.
  const int32_t* row_order = nullptr;
  // bf16 matrix-core kernel: K/V loads non-temporal (for launches that
  // stream hundreds of MB; see the kernel)
  bool kv_nt = false;
  // bf16 kernels: out is K-slab-major with this many rows per slab block
  // (see act_idx), indexed by absolute row; 0 = row-major
  int out_slab_rows = 0;
};
int attention_supported(int dtype, int d, int G);
// Rows are taken in tiles of 32 from row0; a tile of one sequence at
// consecutive positions (a prefill chunk) goes to the MFMA prefill kernel and
// the decode kernel skips its rows (when row_seq is set and the shape is
// supported), every other row to the decode kernel.
void launch_attention(const AttnArgs& a, hipStream_t st);
int prefill_supported(int dtype, int d, int G);
void launch_attention_prefill(const AttnArgs& a, hipStream_t st);

}  // namespace ns
