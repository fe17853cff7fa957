/*
 * ns.h -- C ABI of the MI355X (gfx950) batched GQA decode step.
 *
 * One decode iteration of a pre-norm grouped-query-attention transformer
 * stack over a paged KV cache, as hand-written HIP kernels behind plain C
 * entry points: pointers and sizes only, no C++ or framework types.
 *
 * Sources (the pages describe the problem; none gives an interface):
 *  - page "gpu-waiting-not-working" (nanoserve notes), section "What I
 *    changed because of it" and its changes table: paged KV cache with
 *    per-sequence block tables, token -> cache-slot mapping, one pinned
 *    host-to-device copy of the step metadata, RoPE cos/sin built once per
 *    step, fused RMSNorm, GQA without an expanded K/V copy; section "Where
 *    this leaves nanoserve": the decode step captured once as a graph and
 *    replayed;
 *  - page "NanoFlow: LLM Serving Is Compute Bound, and Your GPU Is Half
 *    Idle", section "Nano-batching: manufacturing independence": the dense
 *    batch split into nano-batches whose compute-bound projections overlap
 *    memory-bound decode attention, ordered by events across streams
 *    (section "Runtime details that keep the pipeline fed" and the closing
 *    implementation note);
 *  - page "The chef who calls out every order: SMs, CUDA streams and CUDA
 *    graphs", sections on streams and on graphs captured per batch size.
 *
 * Conventions
 *  - Every call returns NS_OK (0) or a negative status; nothing throws or
 *    aborts across the ABI.  ns_last_error() gives a message for the last
 *    failing call on this thread.
 *  - Arguments are validated before any state changes or any work is
 *    enqueued: a failing call has no side effects (except NS_EHIP, which
 *    reports a HIP runtime failure that may have left work enqueued).
 *  - "device" pointers are GPU memory the caller owns (e.g. torch tensors);
 *    "host" pointers are ordinary CPU memory read or written before the call
 *    returns.  The library owns only its opaque objects, its second stream,
 *    its events and its pinned staging buffers, released by *_destroy.
 *  - All device work goes to the caller's stream; work forked to the
 *    library's second stream joins back before the call returns.
 *  - One host thread per engine.  KV-manager and slot-map calls are
 *    host-only and need no GPU.
 */
#ifndef NS_H
#define NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
enum {
  NS_OK = 0,
  NS_EINVAL = -1,     /* null pointer, out-of-range id, bad descriptor      */
  NS_ENOBLOCKS = -2,  /* KV pool exhausted                                   */
  NS_ESHAPE = -3,     /* size beyond what the object was created for         */
  NS_ESTATE = -4,     /* call not valid in the object's current state        */
  NS_EHIP = -5        /* HIP runtime error (message from the runtime)        */
};

/* Message for the last failing ns_* call on this thread (never NULL). */
const char* ns_last_error(void);

/* ------------------------------------------------------------ model */
enum { NS_F32 = 0, NS_BF16 = 1 };
#define NS_BLOCK_SIZE 16   /* KV slots per cache block */

typedef struct {
  int32_t n_layers;
  int32_t hidden;       /* H                                                   */
  int32_t n_q_heads;    /* nq                                                  */
  int32_t n_kv_heads;   /* nkv; nq % nkv == 0, group G = nq / nkv in {1..8}    */
  int32_t head_dim;     /* d in {32, 64, 128}                                  */
  int32_t ffn;          /* F (SwiGLU width)                                    */
  int32_t vocab;        /* V; 0 = no embedding / LM head (hidden in and out)   */
  int32_t tied;         /* LM head is the embedding matrix                      */
  float rms_eps;
  float rope_base;
  int32_t dtype;        /* NS_F32 or NS_BF16: storage of weights, activations
                           and KV cache (accumulation is always fp32)          */
} ns_model_desc;

/* Device pointers to the weights (element type = dtype), [out, in]:
 *   attn_norm[l], mlp_norm[l]: [H]
 *   wqkv[l]: [(nq + 2 nkv) d, H]   rows: all q heads, then k heads, then v heads
 *   wo[l]:   [H, nq d]
 *   wgu[l]:  [2F, H]               rows: gate (F rows) then up (F rows)
 *   wdown[l]:[H, F]
 *   final_norm: [H]; embed: [V, H]; lm_head: [V, H].
 * Layout: embed and every fp32 model's matrices are row-major (an fp32
 * model's lm_head may equal embed).  In a bf16 model wqkv, wo, wgu, wdown
 * and lm_head are K-slab-major instead (a tied bf16 model passes a packed
 * copy of embed as lm_head): element
 * (row r, column k) of a [R, K] matrix sits at ((k / 32) * R + r) * 32 +
 * k % 32, so the 32 columns k0 .. k0+31 of all R rows form one contiguous
 * [R][32] block and each row's piece of it is a whole 64-byte segment (the
 * projection kernels then read whole cache lines; row-major rows of a
 * 32-wide K slab cover half of each 128-byte line).  ns_pack_weight converts
 * a row-major matrix.  The per-layer arrays are host arrays of n_layers
 * device pointers; the engine copies them at creation. */
typedef struct {
  const void* const* attn_norm;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* mlp_norm;
  const void* const* wgu;
  const void* const* wdown;
  const void* final_norm;
  const void* embed;
  const void* lm_head;
} ns_weights;

/* ------------------------------------------------------------ KV cache manager
 * Paged KV cache (nanoserve notes, changes table and the paragraph after
 * it: block tables and token -> slot mapping).  Host-side block manager
 * over device memory the caller owns.
 *
 * Device layout (element type = dtype, E = 16 bytes / element size):
 *   for layer l: K region then V region, each num_blocks * nkv * 16 * d
 *   elements;
 *   K: [num_blocks][nkv][d / E][16][E]  (16-byte chunks of a block's 16
 *      tokens interleaved, so one wavefront reads a whole block's chunk
 *      contiguously);
 *   V, fp32: [num_blocks][nkv][16][d]   (token rows);
 *   V, bf16: [num_blocks][nkv][d][16]   (each block transposed, so the 16
 *      tokens of one head-dim element are 32 contiguous bytes).
 * Slot s lives in block s / 16 at row s % 16. */
typedef struct ns_kv ns_kv;

/* Bytes of device memory the cache needs for all layers. */
size_t ns_kv_bytes(const ns_model_desc* desc, int32_t num_blocks);

/* Create a manager of num_blocks blocks for sequence ids 0..max_seqs-1, each
 * holding at most max_blocks_per_seq blocks.  free_order: host [num_blocks]
 * permutation giving the initial free-list order (NULL = 0..num_blocks-1).
 * Errors: NS_EINVAL (bad sizes, free_order not a permutation). */
int ns_kv_create(const ns_model_desc* desc, int32_t num_blocks, int32_t max_seqs,
                 int32_t max_blocks_per_seq, const int32_t* free_order, ns_kv** out);

/* Grow sequence seq to hold n_tokens tokens (ceil(n_tokens / 16) blocks),
 * taking blocks from the head of the free list.  All or nothing.
 * Errors: NS_EINVAL (bad seq / n_tokens), NS_ESHAPE (more than
 * max_blocks_per_seq blocks), NS_ENOBLOCKS (pool exhausted; table unchanged). */
int ns_kv_alloc(ns_kv* kv, int32_t seq, int32_t n_tokens);

/* Return all blocks of seq to the tail of the free list, in table order. */
int ns_kv_free_seq(ns_kv* kv, int32_t seq);

/* Copy the block tables to host out[max_seqs][max_blocks_per_seq], -1 padded. */
int ns_kv_block_table(const ns_kv* kv, int32_t* out);

/* Tokens sequence seq can hold (blocks * 16) and free blocks in the pool. */
int ns_kv_capacity(const ns_kv* kv, int32_t seq, int32_t* tokens_out);
int ns_kv_num_free(const ns_kv* kv, int32_t* out);

void ns_kv_destroy(ns_kv* kv);

/* Token -> slot mapping (nanoserve notes, paragraph after the changes table):
 * slot_out[i] = table[seq[i]][pos[i] / 16] * 16 + pos[i] % 16, or -1 when
 * seq[i] == -1 (a padding row).  Host arrays of n_tok entries.
 * Errors: NS_EINVAL (seq out of range), NS_ESHAPE (pos beyond what the
 * sequence's blocks hold); slot_out is untouched on error. */
int ns_slot_map(const ns_kv* kv, int32_t n_tok, const int32_t* seq, const int32_t* pos,
                int32_t* slot_out);

/* ------------------------------------------------------------ engine */

/* Nano-batch schedule (NanoFlow review, "Nano-batching: manufacturing
 * independence"; its 70B schedule uses four nano-ops at KQV).
 *   n_nano / nano_rows: the rows split into up to 4 consecutive nano-batches
 *     for the O projection and the MLP; the last takes any remainder
 *     (n_nano <= 1: one batch).
 *   n_qkv / qkv_rows: the same for norm + QKV projection + RoPE/cache write
 *     and attention (n_qkv <= 1: use the nano-batches).
 *   overlap: 0 = every kernel in order on the caller's stream; 1 = attention
 *     nano-ops on the library's second stream, ordered by events, so they
 *     run beside the projections of other nano-batches.  Results are
 *     bit-identical either way.
 *   attn_wg_cap: 0 = no cap; else the attention kernel runs at most this
 *     many workgroups (a persistent loop), the graph-safe way to bound the
 *     share of the GPU that attention takes.
 *   cu_mask_frac: must be 0 (NS_EINVAL otherwise).  Restricting the
 *     second stream to a fraction of the compute units
 *     (hipExtStreamCreateWithCUMask) is switched off: on its first GPU run
 *     the masked stream's work did not complete, for a reason not yet
 *     known.  attn_wg_cap bounds the attention's share instead.
 *   prefill_tiles: 0 = every row's attention on the decode kernel; 1 = rows
 *     taken in tiles of 32 from the start of each attention launch, and a
 *     tile of one sequence at 32 consecutive positions (a chunk of a prompt
 *     topping up the dense batch: NanoFlow review, "Runtime details that keep
 *     the pipeline fed") computed on matrix cores (fp16 probabilities);
 *     costs an extra launch and a per-row check, so leave it 0 for batches
 *     of decode rows only.  Captured graphs keep the value they were
 *     captured with.
 *   decode_rows_first: 0 = nano-ops in row order; 1 = the batch holds its
 *     decode rows (long cached contexts) first and prompt chunks after them
 *     (NanoFlow review, "Runtime details that keep the pipeline fed"): the
 *     first QKV part's attention is queued after the other parts' and the
 *     O projection + MLP nano-batches run last-first, so the prompt rows'
 *     projections run beside the decode rows' memory-bound attention
 *     ("Nano-batching: manufacturing independence").  Results are
 *     bit-identical either way.
 *   fuse_rope_attention: 0 = RoPE and the cache write of each row's own K/V
 *     run as their own kernel before attention; 1 = (bf16 models) inside the
 *     attention kernel, one launch fewer per layer (streams-and-graphs
 *     page, "Knob 9 -- Fused kernels": fusing removes launches; the nanoserve
 *     notes' paged-attention kernel took over the ops around it).  The rows of
 *     a step must then belong to distinct sequences (a decode batch): a row
 *     reads no K/V that another row of the same step writes.  Steps and
 *     replays of graphs captured with it reject a batch that repeats a
 *     sequence (NS_EINVAL).  Excludes prefill_tiles.  Steps of 2048 or more
 *     (row, KV head) attention items keep the separate kernel: there the
 *     items alone fill the chip and the prologue would serialise in front of
 *     every item's K/V stream.  Results are bit-identical either way. */
typedef struct {
  int32_t n_nano;
  int32_t nano_rows[4];
  int32_t n_qkv;
  int32_t qkv_rows[4];
  int32_t overlap;
  int32_t attn_wg_cap;
  float cu_mask_frac;
  int32_t prefill_tiles;
  int32_t decode_rows_first;
  int32_t fuse_rope_attention;
} ns_sched;

/* One step's rows.  token_ids (host, [n_tok]) for models with a vocabulary,
 * else hidden_in (device fp32 [n_tok, H]).  seq (host) is the sequence of
 * each row, -1 for a padding row; pos (host) its position.  A decode row has
 * pos = context length - 1; the row's own K/V are written to the cache
 * before attention, so attention covers positions 0..pos.  Rows of one
 * sequence must be in increasing position order.
 *
 * token_ids_dev (device int32 [n_tok], may be NULL): when set, the step takes
 * its token ids from this device buffer instead of token_ids, so the tokens
 * a previous step sampled on the device (ns_sample_greedy) feed the next
 * step with no host round trip, and the host can form step i+1's rows while
 * step i still runs (NanoFlow review, "Runtime details that keep the
 * pipeline fed").  The ids are copied on the step's stream after the
 * metadata; the host cannot check them before the step runs: an id outside
 * [0, vocab) gathers the nearest valid embedding row and is counted on the
 * device.  The count is copied back after each such step, and a later
 * ns_decode_step / ns_graph_replay on this engine (the first one that finds
 * that copy complete, without waiting for it) returns NS_EINVAL, with no
 * other effect, saying how many ids were out of range. */
typedef struct {
  int32_t n_tok;
  const int32_t* token_ids;
  const void* hidden_in;
  const int32_t* seq;
  const int32_t* pos;
  const int32_t* token_ids_dev;
} ns_batch;

typedef struct ns_engine ns_engine;
typedef struct ns_graph ns_graph;

/* Device workspace the engine needs for batches of up to max_tokens rows
 * and sequences of up to max_blocks_per_seq blocks. */
size_t ns_workspace_bytes(const ns_model_desc* desc, int32_t max_tokens,
                          int32_t max_blocks_per_seq);

/* Create an engine over caller-owned weights, KV memory (kv_dev, kv_bytes >=
 * ns_kv_bytes) and workspace (ws_bytes >= ns_workspace_bytes).  sched may be
 * NULL (serial, one batch).  Checks the device is gfx950.
 * Errors: NS_EINVAL, NS_ESHAPE, NS_EHIP. */
int ns_engine_create(const ns_model_desc* desc, const ns_weights* weights, ns_kv* kv,
                     void* kv_dev, size_t kv_bytes, void* workspace, size_t ws_bytes,
                     int32_t max_tokens, const ns_sched* sched, ns_engine** out);
/* Release an engine: waits (at most 30 s) for the work it enqueued on its
 * second stream and for its event-guarded copies, then frees its stream,
 * events and pinned staging.  NULL is a no-op.  Errors: NS_EHIP when that
 * work has not finished within the wait; the engine's resources then stay
 * allocated (the work in flight still uses them) and the handle must not be
 * used again. */
int ns_engine_destroy(ns_engine* eng);

/* Replace the engine's schedule (not the CU mask).  Graphs captured earlier
 * keep the schedule they were captured with. */
int ns_engine_set_sched(ns_engine* eng, const ns_sched* sched);

/* One eager decode step: each kernel is its own launch on `stream`
 * (a hipStream_t; NULL = the null stream).  out_dev (device fp32) receives
 * logits [n_tok, V], or the final hidden state [n_tok, H] when vocab == 0.
 * Every row's slot must already be allocated (ns_kv_alloc).
 * Errors: NS_EINVAL, NS_ESHAPE (n_tok > max_tokens, pos beyond the
 * sequence's blocks), NS_EHIP. */
int ns_decode_step(ns_engine* eng, const ns_batch* batch, void* out_dev, void* stream);

/* Capture the whole step for batches of exactly `bucket` rows as a hipGraph
 * (capture once per batch size, replay per step).  out_dev is fixed at
 * capture.  The capture enqueues nothing that runs.  Errors: NS_EINVAL,
 * NS_ESHAPE (bucket > max_tokens), NS_EHIP. */
int ns_graph_capture(ns_engine* eng, int32_t bucket, void* out_dev, void* stream,
                     ns_graph** out);

/* Replay: one host-to-device copy of the step metadata from pinned staging,
 * then one graph launch, both on `stream`.  batch->n_tok <= bucket; rows
 * beyond n_tok are padding (their output rows are unspecified).
 * Errors: as ns_decode_step. */
int ns_graph_replay(ns_graph* g, const ns_batch* batch, void* stream);

void ns_graph_destroy(ns_graph* g);

/* Bucketed capture ("The chef who calls out every order", CUDA graphs
 * section and "Knob 3 — Capture buckets": one graph per batch-size bucket,
 * the real batch padded up to the next bucket and the output trimmed).
 * ns_graph_set_capture captures one graph per entry of `buckets` (strictly
 * increasing, each in [1, max_tokens], at most 64 entries), all writing
 * out_dev.  ns_graph_set_replay replays the smallest bucket >= batch->n_tok:
 * rows n_tok..bucket-1 are padding, so only the first n_tok output rows are
 * meaningful; *bucket_used (may be NULL) receives the bucket.  Errors:
 * NS_EINVAL (bad bucket list, null argument), NS_ESHAPE (n_tok above the
 * largest bucket), and those of ns_graph_capture / ns_graph_replay; a failed
 * capture releases the graphs already captured. */
typedef struct ns_graph_set ns_graph_set;
int ns_graph_set_capture(ns_engine* eng, const int32_t* buckets, int32_t n_buckets, void* out_dev,
                         void* stream, ns_graph_set** out);
int ns_graph_set_replay(ns_graph_set* set, const ns_batch* batch, void* stream, int32_t* bucket_used);
void ns_graph_set_destroy(ns_graph_set* set);

/* Greedy sampling on the device: the argmax of each row of the step's
 * logits, one of the per-step pieces of fixed cost the roofline page lists
 * beside the kernels ("The roofline flips", section "The point of the title:
 * why it flips in SLMs": the argmax and the copy of the token back).
 * logits: device fp32 [n_rows, vocab], row-major.  tokens_out: device int32
 * [n_rows]; tokens_out[r] is the lowest index v with logits[r][v] equal to
 * the row's maximum over its non-NaN entries (NaN never wins; a row of NaN
 * only gives 0).  Enqueued on `stream`; nothing is synchronised or copied
 * to the host.  Errors: NS_EINVAL (null pointer, n_rows or vocab < 1),
 * NS_EHIP. */
int ns_sample_greedy(const float* logits, int32_t n_rows, int32_t vocab, int32_t* tokens_out, void* stream);

/* Streaming read, for measuring the memory ceiling of the roofline: the
 * pages take the ceiling as the datasheet bandwidth and note that real
 * kernels reach only part of it (roofline page, "The roofline flips", section
 * "The bare mechanism: what the roofline says"); timing this call gives the
 * read rate a kernel reaches on this chip, beside which the attention's
 * bytes per second are read.  Reads every byte of src (device, 16-byte
 * aligned; bytes a positive multiple of 16) once and writes
 * NS_READ_STREAM_WORDS words to sink (device uint32, sink_words of room):
 * their XOR equals the XOR of all 32-bit words of src.  Enqueued on
 * `stream`.  Errors: NS_EINVAL (null pointer, misaligned src, bytes not a
 * positive multiple of 16, sink too small), NS_EHIP. */
#define NS_READ_STREAM_WORDS 2048
int ns_read_stream(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

/* ------------------------------------------------------------ helpers */

/* Write n cached positions into the KV cache of one layer: k, v are device
 * [n, nkv, d] (element type = dtype) in logical order, slots a device int32
 * [n] (entries < 0 skipped).  For setting up context that earlier steps
 * would have written.  Enqueued on `stream`. */
int ns_kv_scatter(ns_engine* eng, int32_t layer, int32_t n, const int32_t* slots_dev,
                  const void* k_dev, const void* v_dev, void* stream);

/* Read n cached positions of one layer back in logical order (device
 * k_out, v_out [n, nkv, d]); slots < 0 give zeros. */
int ns_kv_gather(ns_engine* eng, int32_t layer, int32_t n, const int32_t* slots_dev,
                 void* k_out, void* v_out, void* stream);

/* Kernels launched by the last ns_decode_step (for launch counting). */
int ns_engine_last_launches(const ns_engine* eng, int32_t* out);

/* Profiling of eager steps (measurement only).  When enabled, a serial
 * (overlap = 0) ns_decode_step records a HIP event after every launch on
 * the caller's stream.  ns_engine_profile_read waits for the last one and
 * returns, for the first min(cap, n) launches, the kernel class and the
 * device time since the previous event in microseconds; *n_out = launches
 * recorded.  Classes: 0 embedding, 1 RoPE table, 2 RMSNorm, 3 QKV
 * projection, 4 RoPE + cache write, 5 attention (with its combine),
 * 6 O projection, 7 gate-up projection, 8 down projection, 9 LM head,
 * 10 output copy.  Graph capture ignores the setting. */
int ns_engine_profile(ns_engine* eng, int32_t enable);
int ns_engine_profile_read(ns_engine* eng, int32_t cap, int32_t* kinds, float* us, int32_t* n_out);

/* ------------------------------------------------------------ single kernels
 * The hot kernels on their own, for kernel-level checks and roofline
 * timing.  All pointers are device memory; work goes to `stream`. */

enum { NS_EPI_STORE = 0, NS_EPI_RESID = 1, NS_EPI_SILU = 2 };

/* Dense projection C = A * B^T (NanoFlow review, operator table: the dense
 * class).  A [M, K], B [N, K] row-major, element type dtype, fp32
 * accumulation.  epi NS_EPI_STORE: C fp32 [M, N] = result; NS_EPI_RESID:
 * C fp32 [M, N] += result; NS_EPI_SILU: B is [2N, K] (gate rows then up
 * rows) and C (dtype) [M, N] = silu(gate) * up.  bf16 needs K % 32 == 0
 * (NS_ESHAPE otherwise). */
int ns_op_gemm(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, const void* B,
               void* C, void* stream);

/* The same with B K-slab-major (the layout of a bf16 model's projection
 * weights, see ns_weights): bf16 only (NS_EINVAL otherwise). */
int ns_op_gemm_packed(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A,
                      const void* B, void* C, void* stream);

/* The same projection (bf16) with every operand in the layout a bf16
 * engine's step keeps (NanoFlow review, operator table: the dense class):
 * A K-slab-major with a_rows (>= M) rows per 32-column slab block, element
 * (m, k) at ((k / 32) * a_rows + m) * 32 + k % 32; B K-slab-major as for
 * ns_op_gemm_packed; for NS_EPI_SILU, C (bf16) K-slab-major over its N
 * columns with c_rows (>= M) rows per block (N % 32 == 0); for NS_EPI_STORE
 * and NS_EPI_RESID, C fp32 [M, N] row-major (c_rows unused).  ns_pack_weight
 * of a row-major [a_rows, K] matrix gives such an A.  Errors: NS_EINVAL (bad
 * epilogue or sizes, null pointer, a_rows or c_rows < M), NS_ESHAPE
 * (K % 32 != 0). */
int ns_op_gemm_slab(int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, int32_t a_rows, const void* B,
                    void* C, int32_t c_rows, void* stream);

/* RMSNorm of each row (nanoserve notes, changes table: the fused RMSNorm;
 * the final norm in front of the LM head): out[r] = x[r] / sqrt(mean(x[r]^2)
 * + eps) * gain, computed in fp32 and stored as dtype.  x: device fp32
 * [n_rows, hidden]; gain: device [hidden] (dtype); out: device [n_rows,
 * hidden] (dtype).  The same kernel the step uses for a norm with no split-K
 * slices to add.  Errors: NS_EINVAL (bad dtype or sizes, eps < 0, null
 * pointer with n_rows > 0). */
int ns_op_rmsnorm(int32_t dtype, int32_t n_rows, int32_t hidden, const float* x, const void* gain, float eps,
                  void* out, void* stream);
/* Convert a row-major bf16 matrix [rows, cols] (device) into the K-slab-major
 * layout of ns_weights (device, a separate buffer of the same size), on
 * `stream`.  Errors: NS_EINVAL (null or equal pointers, rows < 1, cols not a
 * positive multiple of 32). */
int ns_pack_weight(const void* src, void* dst, int32_t rows, int32_t cols, void* stream);

/* Paged GQA decode attention (nanoserve notes, changes table; NanoFlow
 * review, operator table: decode attention).  Row i (query position
 * row_pos[i] of the sequence whose block-table row is row_bseq[i], -1 for a
 * padding row) attends over positions 0..row_pos[i] with scale 1/sqrt(d).
 *   q_att: [n_rows][nkv][d/E][G][E] (E = 16 bytes / element size): the G
 *     query heads of each KV head, 16-byte chunk by chunk;
 *   kv_layer: one layer of the cache (layout as in ns_kv_bytes);
 *   btab: [*][max_blocks_per_seq] block ids; out: [n_rows][nq * d];
 *   ws: ns_op_attention_ws_bytes() bytes for split-context partials;
 *   wg_cap: 0 or the maximum number of workgroups. */
size_t ns_op_attention_ws_bytes(const ns_model_desc* desc, int32_t n_rows, int32_t max_blocks_per_seq);
int ns_op_attention(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                    int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos, const int32_t* btab,
                    int32_t max_blocks_per_seq, void* out, void* ws, size_t ws_bytes, int32_t wg_cap,
                    void* stream);

/* The same with prefill tiles on (see ns_sched.prefill_tiles): rows are
 * taken in tiles of 32 from row 0, and a tile whose rows are one sequence
 * (row_bseq) at consecutive positions goes to the matrix-core prefill kernel.
 * Arguments and errors as ns_op_attention. */
int ns_op_attention_prefill(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                    int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos, const int32_t* btab,
                    int32_t max_blocks_per_seq, void* out, void* ws, size_t ws_bytes, int32_t wg_cap,
                    void* stream);

/* Paged GQA decode attention that allocates nothing, for callers that
 * cannot call hipMalloc or take a workspace: code under graph capture, tight
 * serving loops, harnesses that forbid allocation.  Arguments, layout and
 * results as ns_op_attention, without ws / ws_bytes: the split-context
 * partials live in a static device array of NS_ATTENTION_STATIC_SCRATCH_BYTES
 * (5 MiB) that the library holds on every GPU it runs on until the process
 * ends (looked up once per device on the first call there).  Contexts are
 * split only while the split work items' wavefronts stay within 4096, at 4
 * or 8 wavefronts per item, so at most 1024 split items and partials of at
 * most 4 MiB + 64 KiB for any supported shape (G * d <= 1024).  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (two
 * streams, or two host threads) race and give wrong results; the partials
 * are written before they are read within each call, so nothing needs
 * clearing.  Errors: those of ns_op_attention, and NS_ESHAPE when the
 * partials (ns_op_attention_ws_bytes) exceed the static array. */
#define NS_ATTENTION_STATIC_SCRATCH_BYTES ((size_t)5 << 20)
int ns_op_attention_static(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                           int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos,
                           const int32_t* btab, int32_t max_blocks_per_seq, void* out, int32_t wg_cap,
                           void* stream);
#ifdef __cplusplus
}
#endif
#endif /* NS_H */
