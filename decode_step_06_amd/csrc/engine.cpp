// Engine of the decode step: workspace plan, step metadata, the kernel
// sequence of one step (shared by eager execution and graph capture), the
// nano-batch schedule over two streams, and graph capture / replay.
//
// Sources: page "gpu-waiting-not-working" (nanoserve notes) -- changes table
// (one pinned host-to-device copy of the step metadata; RoPE cos/sin built
// once per step) and section "Where this leaves nanoserve" (capture the
// decode step once and replay it); page "NanoFlow: LLM Serving Is Compute
// Bound, and Your GPU Is Half Idle" -- section "Nano-batching: manufacturing
// independence" (split rows into nano-batches so projections of one overlap
// attention of another) and its implementation note (events order the
// nano-ops across streams); page "The chef who calls out every order: SMs,
// CUDA streams and CUDA graphs" -- streams as in-order queues that overlap
// each other, and one graph per batch size.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "ns_internal.h"
#include "ns_kernels.h"

namespace ns {
int check_desc(const ns_model_desc* d);
size_t kv_layer_bytes(const ns_model_desc* d, int32_t num_blocks);
}  // namespace ns

#define HIP_TRY(expr)                                                                                  \
  do {                                                                                                 \
    hipError_t _e = (expr);                                                                            \
    if (_e != hipSuccess) NS_FAIL(NS_EHIP, "%s failed: %s", #expr, hipGetErrorString(_e));             \
  } while (0)

namespace {

constexpr int kMaxParts = 4;
constexpr int kSplitRows = 256;  // steps of at most this many rows use the split-K projections
constexpr int kMaxSlices = 8;
constexpr long kOrderItems = 1024;  // attention work items from which rows go longest first
// One layer's K/V region from which the attention streams the cache with
// non-temporal loads (an upper bound on what one launch reads).  Measured on
// MI355X, one box, both ways: the 70B shape (1.04 GiB per layer) gains with
// the hint (attention at 256 rows 192.5 -> 180.2 us, the 80-layer step 56.9 ->
// 56.5 ms); the 0.5B shape (at most 146 MB per layer) loses at every batch
// (B = 32 step 0.924 -> 0.975 ms, the mix at B = 1 0.816 -> 0.955 ms,
// B = 256 2.363 -> 2.443 ms).
constexpr size_t kKvStreamBytes = 512ul << 20;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int elem_size(int32_t dtype) { return dtype == NS_BF16 ? 2 : 4; }

// Attention launch shape for a batch of n_rows rows when sequences hold at
// most cap_tokens tokens: partition size (tokens, a multiple of 64),
// partitions per row, and wavefronts per work item (row, KV head,
// partition).  A wavefront's 64-token pass costs about 1 us of memory
// latency and the combine launch of a split context about 6 us, so:
// 8 wavefronts per item while items are few (<= 256, at most 2048
// wavefronts: more passes in flight per row), 4 up to 4095 items, 1 once
// the items alone fill the chip twice over; the context is split (in
// halves, repeatedly) only while a wavefront would take more than 8 passes
// and the split items stay within 4096 wavefronts.  The shape depends only
// on the whole batch's row count and the capacity, so nano-batched and
// unsplit steps, eager and captured, compute identically.  (Fitted to
// timings of the matrix-core kernel on MI355X: batch 1..512, contexts
// 128..2048, head_dim 64 with 7 query heads per KV head and 128 with 8; at
// 256 rows of 8 KV heads with contexts 512..1536, 4 wavefronts on whole
// contexts took 200 us against 226 us for 1 wavefront on contexts split in
// two, whose short rows leave their second part empty.)
void attn_partition(int n_rows, int nkv, int cap_tokens, int* part_tokens, int* n_parts, int* waves) {
  const int chunks = std::max(1, (cap_tokens + 63) / 64);
  const long items = std::max(1L, (long)n_rows * nkv);
  const int w = items >= 4096 ? 1 : (items <= 256 ? 8 : 4);
  int parts = 1;
  auto passes = [&](int p) { return ((chunks + p - 1) / p + w - 1) / w; };
  while (parts < chunks && passes(parts) > 8 && items * parts * 2 * w <= 4096) parts *= 2;
  const int per = (chunks + parts - 1) / parts;
  *waves = w;
  *part_tokens = 64 * per;
  *n_parts = (chunks + per - 1) / per;
}

struct Plan {
  size_t x, h, qkv, q_att, o, act, cosb, sinb, meta, part_acc, part_ml, part_qkv, part_res, bad_tok, total;
  int tdec;  // rows of the split-K slice buffers (steps of at most 256 rows)
  size_t meta_ints;  // int32 entries of the metadata block
};

// Rows of a slab block of the K-slab-major bf16 activations (see
// act_slab_rows): the capacity rounded up to an odd count, so that
// consecutive blocks do not start at the same offset modulo a power of two.
int slab_rows(int max_tokens) { return max_tokens | 1; }

Plan make_plan(const ns_model_desc* d, int T, int maxb) {
  Plan p{};
  const size_t es = elem_size(d->dtype);
  const int G = d->n_q_heads / d->n_kv_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  p.x = take((size_t)T * d->hidden * 4);
  // the bf16 projections' inputs: slab blocks of slab_rows(T) rows
  p.h = take((size_t)slab_rows(T) * d->hidden * es);
  p.qkv = take((size_t)T * (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim * 4);
  p.q_att = take((size_t)T * d->n_q_heads * d->head_dim * es);
  p.o = take((size_t)slab_rows(T) * d->n_q_heads * d->head_dim * es);
  p.act = take((size_t)slab_rows(T) * d->ffn * es);
  p.cosb = take((size_t)T * d->head_dim / 2 * 4);
  p.sinb = take((size_t)T * d->head_dim / 2 * 4);
  p.meta_ints = 5 * (size_t)T + (size_t)T * maxb;
  p.meta = take(p.meta_ints * 4);
  long items = 0;
  for (int n = 1; n <= T; ++n) {
    int P, np, nw;
    attn_partition(n, d->n_kv_heads, maxb * NS_BLOCK_SIZE, &P, &np, &nw);
    if (np > 1) items = std::max(items, (long)n * d->n_kv_heads * np);
  }
  p.part_acc = take((size_t)items * G * d->head_dim * 4);
  p.part_ml = take((size_t)items * G * 2 * 4);
  // split-K slices of steps of at most 256 rows (bf16 models): the QKV
  // result, and the O / down projections' residual adds (up to 8 slices each)
  p.tdec = std::min(T, kSplitRows);
  const int qkv_w = (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  const bool dec = d->dtype == NS_BF16;
  p.part_qkv = take(dec ? (size_t)kMaxSlices * p.tdec * qkv_w * 4 : 0);
  p.part_res = take(dec ? (size_t)kMaxSlices * p.tdec * d->hidden * 4 : 0);
  p.bad_tok = take(sizeof(int32_t));  // running count of out-of-range device-fed token ids
  p.total = off;
  return p;
}

// Row ranges of a split: up to 4 consecutive parts; the last takes the rest.
std::vector<std::pair<int, int>> row_parts(int n_tok, int n, const int32_t* rows) {
  std::vector<std::pair<int, int>> out;
  if (n <= 1) {
    out.push_back({0, n_tok});
    return out;
  }
  int r = 0;
  for (int i = 0; i < n && r < n_tok; ++i) {
    int len = (i == n - 1) ? n_tok - r : std::min(std::max(rows[i], 0), n_tok - r);
    if (len <= 0) continue;
    out.push_back({r, r + len});
    r += len;
  }
  if (r < n_tok) {
    if (out.empty()) out.push_back({r, n_tok});
    else out.back().second = n_tok;
  }
  return out;
}

}  // namespace

struct ns_engine {
  ns_model_desc d{};
  int es = 2;
  int G = 1;
  std::vector<const void*> attn_norm, wqkv, wo, mlp_norm, wgu, wdown;
  const void* final_norm = nullptr;
  const void* embed = nullptr;
  const void* lm_head = nullptr;
  ns_kv* kv = nullptr;
  char* kv_dev = nullptr;
  size_t kv_layer = 0;
  int num_blocks = 0;
  int max_tokens = 0;
  int maxb = 0;
  int ncu = 256;  // compute units: workgroups of one dispatch round
  char* ws = nullptr;
  Plan plan{};
  ns_sched sched{};
  hipStream_t s2 = nullptr;
  hipEvent_t ev_qkv[kMaxParts] = {};
  hipEvent_t ev_att[kMaxParts] = {};
  hipEvent_t ev_join = nullptr;  // joins the second stream back into a capture that failed half-way
  int32_t* staging[2] = {nullptr, nullptr};
  hipEvent_t staging_ev[2] = {};
  bool staging_used[2] = {false, false};
  int staging_next = 0;
  int last_launches = 0;
  // out-of-range device-fed token ids: the device count, copied to pinned
  // host memory after each step fed from device memory, and the count the
  // host has reported so far
  int32_t* bad_tok_host = nullptr;
  hipEvent_t bad_tok_ev = nullptr;
  bool bad_tok_copied = false;
  int32_t bad_tok_reported = 0;
  // profiling: an event after every launch of an eager serial step
  bool prof = false;
  hipEvent_t prof_start = nullptr;
  std::vector<hipEvent_t> prof_ev;
  std::vector<int32_t> prof_kind;
  int prof_n = 0;

  float* x() const { return (float*)(ws + plan.x); }
  void* h() const { return ws + plan.h; }
  float* qkv() const { return (float*)(ws + plan.qkv); }
  void* q_att() const { return ws + plan.q_att; }
  void* o() const { return ws + plan.o; }
  void* act() const { return ws + plan.act; }
  float* cosb() const { return (float*)(ws + plan.cosb); }
  float* sinb() const { return (float*)(ws + plan.sinb); }
  int32_t* meta() const { return (int32_t*)(ws + plan.meta); }
  // metadata block: tokens[T] | row index (-1: padding)[T] | pos[T] | slot[T] | btab[T][maxb] (one block-table
  // row per step row)
  int32_t* m_tok() const { return meta(); }
  int32_t* m_seq() const { return meta() + max_tokens; }
  int32_t* m_pos() const { return meta() + 2 * max_tokens; }
  int32_t* m_slot() const { return meta() + 3 * max_tokens; }
  int32_t* m_order() const { return meta() + 4 * max_tokens; }
  int32_t* m_btab() const { return meta() + 5 * max_tokens; }
  int32_t* bad_tok() const { return (int32_t*)(ws + plan.bad_tok); }
  float* part_qkv() const { return (float*)(ws + plan.part_qkv); }
  float* part_res() const { return (float*)(ws + plan.part_res); }
  char* k_layer(int l) const { return kv_dev + (size_t)l * kv_layer; }
  char* v_layer(int l) const { return kv_dev + (size_t)l * kv_layer + kv_layer / 2; }
};

struct ns_graph {
  ns_engine* e = nullptr;
  int bucket = 0;
  bool fused_rope = false;  // captured with RoPE fused into attention: one row per sequence
  ns_sched sched{};         // the schedule captured (its attention parts order the rows at replay)
  void* out = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

struct ns_graph_set {
  std::vector<ns_graph*> graphs;  // increasing buckets
};

namespace {

int check_sched(const ns_sched* s) {
  if (!s) return NS_OK;
  if (s->n_nano < 0 || s->n_nano > kMaxParts || s->n_qkv < 0 || s->n_qkv > kMaxParts)
    NS_FAIL(NS_EINVAL, "at most %d nano-batches", kMaxParts);
  if (s->attn_wg_cap < 0) NS_FAIL(NS_EINVAL, "attn_wg_cap must be >= 0");
  if (s->cu_mask_frac < 0.f || s->cu_mask_frac > 1.f) NS_FAIL(NS_EINVAL, "cu_mask_frac must be in [0, 1]");
  // The CU-masked second stream is switched off: its first GPU run (40% of
  // the CUs, overlapped nano-batches) left work on that stream that never
  // completed, and the cause is not known.
  if (s->cu_mask_frac != 0.f)
    NS_FAIL(NS_EINVAL, "cu_mask_frac is disabled (a CU-masked second stream did not complete its work); use "
                       "attn_wg_cap to bound the attention's share");
  if (s->prefill_tiles != 0 && s->prefill_tiles != 1) NS_FAIL(NS_EINVAL, "prefill_tiles must be 0 or 1");
  if (s->decode_rows_first != 0 && s->decode_rows_first != 1) NS_FAIL(NS_EINVAL, "decode_rows_first must be 0 or 1");
  if (s->fuse_rope_attention != 0 && s->fuse_rope_attention != 1)
    NS_FAIL(NS_EINVAL, "fuse_rope_attention must be 0 or 1");
  if (s->fuse_rope_attention && s->prefill_tiles)
    NS_FAIL(NS_EINVAL, "fuse_rope_attention and prefill_tiles exclude each other");
  return NS_OK;
}

// RoPE + the row's own K/V write run inside the bf16 attention kernel.
bool fused_rope(const ns_engine* e, const ns_sched& s) { return s.fuse_rope_attention != 0 && e->d.dtype == NS_BF16; }

// Validate a batch against the engine and the KV manager; no side effects.
int check_batch(const ns_engine* e, const ns_batch* b, int max_rows, bool one_row_per_seq) {
  if (!b) NS_FAIL(NS_EINVAL, "null batch");
  if (b->n_tok <= 0) NS_FAIL(NS_EINVAL, "batch must have at least one row");
  if (b->n_tok > max_rows) NS_FAIL(NS_ESHAPE, "batch of %d rows exceeds %d", b->n_tok, max_rows);
  if (!b->seq || !b->pos) NS_FAIL(NS_EINVAL, "null seq/pos arrays");
  if (e->d.vocab > 0 && !b->token_ids && !b->token_ids_dev)
    NS_FAIL(NS_EINVAL, "model has a vocabulary: token_ids or token_ids_dev required");
  if (e->d.vocab == 0 && !b->hidden_in) NS_FAIL(NS_EINVAL, "model has no vocabulary: hidden_in required");
  const ns_kv* kv = e->kv;
  std::vector<int32_t> last_pos(kv->max_seqs, -1);
  for (int i = 0; i < b->n_tok; ++i) {
    const int32_t s = b->seq[i], p = b->pos[i];
    if (s == -1) continue;
    if (s < 0 || s >= kv->max_seqs) NS_FAIL(NS_EINVAL, "row %d: sequence %d out of range", i, s);
    if (p < 0 || (int64_t)p >= (int64_t)kv->tables[s].size() * NS_BLOCK_SIZE)
      NS_FAIL(NS_ESHAPE, "row %d: position %d not covered by sequence %d's blocks", i, p, s);
    if ((int)kv->tables[s].size() > e->maxb)
      NS_FAIL(NS_ESHAPE, "sequence %d holds more blocks than the engine's table rows", s);
    if (one_row_per_seq && last_pos[s] >= 0)
      NS_FAIL(NS_EINVAL, "sequence %d has more than one row; the fused RoPE/attention schedule takes one", s);
    if (p <= last_pos[s]) NS_FAIL(NS_EINVAL, "rows of sequence %d must have increasing positions", s);
    last_pos[s] = p;
    if (e->d.vocab > 0 && !b->token_ids_dev && (b->token_ids[i] < 0 || b->token_ids[i] >= e->d.vocab))
      NS_FAIL(NS_EINVAL, "row %d: token id %d out of range", i, b->token_ids[i]);
  }
  return NS_OK;
}

// The row ranges of a step's attention launches: the QKV parts when the QKV
// projection is split, else the nano-batches.
std::vector<std::pair<int, int>> attn_row_parts(const ns_sched& sc, int n_tok) {
  return sc.n_qkv > 1 ? row_parts(n_tok, sc.n_qkv, sc.qkv_rows) : row_parts(n_tok, sc.n_nano, sc.nano_rows);
}

// Pack the step metadata for `rows` rows (rows >= n_tok are padding) of a
// step run under schedule sc into pinned staging and copy it to the device
// with one transfer.
// How an attention launch of n_rows rows (per_row work items each) orders
// its rows.  From kOrderItems items: longest context first (more items than
// the chip holds at once; the dispatch hands the short ones to the CUs that
// free up first: 256 rows of the 70B shape with contexts 512..1536, 202 ->
// 192 us in isolation).  Between one and two dispatch rounds (more items
// than CUs, all resident at once, two workgroups on the busiest CUs):
// zig-zag, so the workgroups that share a CU pair a long row with a short
// one.  Fewer items: none (one round, each item on a CU of its own; the order
// would only add a dependent load in front of each).
enum { kOrderNone = 0, kOrderLongest = 1, kOrderZigzag = 2 };
int attn_row_order(const ns_engine* e, long n_rows, long per_row) {
  const long items = n_rows * per_row;
  if (items >= kOrderItems) return kOrderLongest;
  if (items > e->ncu && items <= 2L * e->ncu) return kOrderZigzag;
  return kOrderNone;
}

int upload_meta(ns_engine* e, const ns_batch* b, int rows, const ns_sched& sc, hipStream_t st) {
  const int k = e->staging_next;
  e->staging_next ^= 1;
  if (e->staging_used[k]) HIP_TRY(hipEventSynchronize(e->staging_ev[k]));
  int32_t* m = e->staging[k];
  const int T = e->max_tokens;
  int32_t* tok = m;
  int32_t* rowb = m + T;  // sequence of each row (-1: padding)
  int32_t* pos = m + 2 * T;
  int32_t* slot = m + 3 * T;
  int32_t* order = m + 4 * T;  // attention's row order within each of its parts
  int32_t* btab = m + 5 * T;
  // one block-table row per step row (attention then reads its blocks
  // without first looking up the row's sequence)
  for (int i = 0; i < rows; ++i) {
    const bool real = i < b->n_tok && b->seq[i] != -1;
    tok[i] = (i < b->n_tok && b->token_ids && !b->token_ids_dev) ? b->token_ids[i] : 0;
    pos[i] = real ? b->pos[i] : 0;
    int32_t* row = btab + (size_t)i * e->maxb;
    if (!real) {
      rowb[i] = -1;
      slot[i] = -1;
      std::fill(row, row + e->maxb, -1);
      continue;
    }
    const int32_t s = b->seq[i];
    const auto& tab = e->kv->tables[s];
    for (int j = 0; j < e->maxb; ++j) row[j] = j < (int)tab.size() ? tab[j] : -1;
    rowb[i] = s;
    const int32_t p = b->pos[i];
    slot[i] = tab[p / NS_BLOCK_SIZE] * NS_BLOCK_SIZE + p % NS_BLOCK_SIZE;
  }
  // longest context first within each attention part (padding rows last);
  // ties in row order.  Parts whose work items fill two dispatch rounds are
  // zig-zagged instead: the rows of the first round longest first, the rest
  // shortest first, so each CU's second workgroup (a short row) joins a long
  // one (attn_row_order says which parts use the order at all).
  int pt = 0, np = 0, wv = 0;
  attn_partition(rows, e->d.n_kv_heads, e->maxb * NS_BLOCK_SIZE, &pt, &np, &wv);
  for (const auto& pr : attn_row_parts(sc, rows)) {
    for (int i = pr.first; i < pr.second; ++i) order[i] = i;
    std::stable_sort(order + pr.first, order + pr.second, [&](int32_t a, int32_t c) {
      const int32_t ka = rowb[a] < 0 ? -1 : pos[a], kc = rowb[c] < 0 ? -1 : pos[c];
      return ka > kc;
    });
    const long per_row = (long)e->d.n_kv_heads * np;
    if (attn_row_order(e, pr.second - pr.first, per_row) == kOrderZigzag) {
      const long first = (e->ncu + per_row - 1) / per_row;  // rows of the first round
      if (first < pr.second - pr.first) std::reverse(order + pr.first + first, order + pr.second);
    }
  }
  const size_t head = 5 * (size_t)T * sizeof(int32_t);
  const size_t bytes = head + (size_t)rows * e->maxb * sizeof(int32_t);
  HIP_TRY(hipMemcpyAsync(e->meta(), m, bytes, hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(e->staging_ev[k], st));
  e->staging_used[k] = true;
  // device-resident token ids (on-device feedback) overwrite the token slots
  if (e->d.vocab > 0 && b->token_ids_dev)
    HIP_TRY(hipMemcpyAsync(e->meta(), b->token_ids_dev, (size_t)b->n_tok * sizeof(int32_t), hipMemcpyDeviceToDevice,
                           st));
  return NS_OK;
}

// bf16 models keep the projections' bf16 inputs (h, the attention output o
// and the SwiGLU activation) K-slab-major, each 32-column slab a contiguous
// block of slab_rows(max_tokens) rows: the layout of the weights, so that a
// GEMM's 16-row load of one slab reads 1 KB contiguous instead of 16
// separate 64-byte pieces (measured on MI355X, one box, same bits: the
// 80-layer 70B-shaped step 54.1 -> 51.9 ms, the 2048-row layer 3.62 -> 3.55
// ms, the 0.5B-shaped mix at 64 rows 1.565 -> 1.371 ms).  fp32 models stay
// row-major.  Steps of at most kPackMinRows rows keep them row-major too:
// their projections load one 16-row fragment per k-step, which the layout
// cannot widen, and the row-major loads keep their constant offsets.
constexpr int kPackMinRows = 16;
int act_slab_rows(const ns_engine* e, int n_tok) {
  return e->d.dtype == NS_BF16 && n_tok > kPackMinRows ? slab_rows(e->max_tokens) : 0;
}

void attn_args(const ns_engine* e, int layer, int r0, int r1, int n_tok, ns::AttnArgs* a) {
  a->dtype = e->d.dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32;
  a->q_att = e->q_att();
  a->kc = e->k_layer(layer);
  a->vc = e->v_layer(layer);
  a->row_bseq = nullptr;  // the step's table has one row per row
  a->row_pos = e->m_pos();
  a->btab = e->m_btab();
  a->maxb = e->maxb;
  a->out = e->o();
  a->part_acc = (float*)(e->ws + e->plan.part_acc);
  a->part_ml = (float*)(e->ws + e->plan.part_ml);
  a->row0 = r0;
  a->n_rows = r1 - r0;
  a->nq = e->d.n_q_heads;
  a->nkv = e->d.n_kv_heads;
  a->d = e->d.head_dim;
  attn_partition(n_tok, e->d.n_kv_heads, e->maxb * NS_BLOCK_SIZE, &a->part_tokens,
                 &a->n_parts, &a->waves);
  a->wg_cap = e->sched.attn_wg_cap;
  a->row_seq = e->sched.prefill_tiles ? e->m_seq() : nullptr;
  a->kv_nt = e->kv_layer >= kKvStreamBytes;
  a->out_slab_rows = act_slab_rows(e, n_tok);
  if (attn_row_order(e, r1 - r0, (long)a->nkv * a->n_parts) != kOrderNone) a->row_order = e->m_order();
}

// The kernel sequence of one step over n_tok rows (metadata already on the
// device, x already holding the hidden input for models without a
// vocabulary).  Used unchanged by eager steps and by graph capture.
// Kernel classes reported by the profiling mode.
enum { K_EMBED = 0, K_ROPE_TABLE, K_NORM, K_QKV, K_ROPE_KV, K_ATTN, K_O, K_GU, K_DOWN, K_LM_HEAD, K_COPY };

int enqueue_step(ns_engine* e, const ns_sched& sc, int n_tok, void* out, hipStream_t st, bool capturing) {
  const ns_model_desc& d = e->d;
  const int dt = d.dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32;
  const int H = d.hidden, nq = d.n_q_heads, nkv = d.n_kv_heads, hd = d.head_dim, F = d.ffn;
  const int QKV = (nq + 2 * nkv) * hd, DQ = nq * hd;
  const size_t es = e->es;
  const bool overlap = sc.overlap != 0;
  auto nano = row_parts(n_tok, sc.n_nano, sc.nano_rows);
  auto qparts = attn_row_parts(sc, n_tok);
  int launches = 0;
  hipStream_t sa = overlap ? e->s2 : st;
  const bool prof = e->prof && !capturing && !overlap;
  e->prof_n = 0;
  if (prof) HIP_TRY(hipEventRecord(e->prof_start, st));
  auto mark = [&](int kind) -> int {
    if (!prof) return NS_OK;
    if (e->prof_n >= (int)e->prof_ev.size()) {
      hipEvent_t ev;
      HIP_TRY(hipEventCreate(&ev));
      e->prof_ev.push_back(ev);
      e->prof_kind.push_back(0);
    }
    HIP_TRY(hipEventRecord(e->prof_ev[e->prof_n], st));
    e->prof_kind[e->prof_n++] = kind;
    return NS_OK;
  };
#define MARK(k)                 \
  do {                          \
    int _rc = mark(k);          \
    if (_rc) return _rc;        \
  } while (0)

  // embedding (or the hidden input already in x), RoPE table, layer 0's norm
  ns::launch_step_prologue(dt, d.vocab > 0 ? e->embed : nullptr, e->m_tok(), e->x(), e->m_pos(), e->cosb(),
                           e->sinb(), e->attn_norm[0], e->h(), n_tok, H, d.vocab, hd, d.rope_base, d.rms_eps,
                           e->bad_tok(), st, act_slab_rows(e, n_tok));
  ++launches;
  MARK(K_EMBED);

  char* h = (char*)e->h();
  char* o = (char*)e->o();
  char* act = (char*)e->act();
  // activation rows from r0 of a `width`-column matrix, its leading
  // dimension for the GEMMs, and their layout flag
  const int ar = act_slab_rows(e, n_tok);
  auto arow = [&](char* buf, int r0, int width) { return buf + (ar ? (size_t)r0 * 32 : (size_t)r0 * width) * es; };
  auto ald = [&](int width) { return ar ? ar : width; };
  const int apk = ar ? ns::PK_A : 0;
  float* x = e->x();
  float* qkv = e->qkv();
  // Steps of at most 256 rows (bf16): the QKV, O and down projections split
  // K across workgroups so that their few output tiles still fill the chip
  // (at <= 64 rows they stream the weights); each split writes an fp32 slice
  // and the next kernel on those rows (RoPE/cache write, or the next
  // RMSNorm, or the output) sums the slices in order -- the residual add of
  // the O and down projections happens there.  The split counts follow the
  // whole step's row count, so every nano-batch's slices match their
  // consumers.
  const bool dec = dt == NS_DT_BF16 && n_tok <= e->plan.tdec;
  const long sq = (long)e->plan.tdec * QKV, sr = (long)e->plan.tdec * H;  // slice strides
  const int S_qkv = dec ? std::min(kMaxSlices, ns::gemm_partial_splits(n_tok, QKV, H)) : 1;
  const int S_o = dec ? std::min(kMaxSlices, ns::gemm_partial_splits(n_tok, H, DQ)) : 1;
  const int S_d = dec ? std::min(kMaxSlices, ns::gemm_partial_splits(n_tok, H, F)) : 1;
  float* pq = e->part_qkv();
  float* pr = e->part_res();
  // bf16 models' projection weights are K-slab-major: their "leading
  // dimension" is the row count; fp32 weights are row-major
  const int pk = dt == NS_DT_BF16 ? ns::PK_B : 0;
  auto wld = [&](int rows, int cols) { return pk ? rows : cols; };
  // decode rows first (the dense batch's order): the first QKV part's long
  // attention is queued after the other parts' and the O/MLP nano-batches
  // run last-first, so the later rows' projections run beside it.  Attention
  // part j reads only K/V written by parts <= j, all finished before QKV part
  // j's event, so any launch order of the attention parts is valid.
  // fused only below 2048 work items (rows x KV heads), where the launches
  // are latency-bound and a work item's wavefronts share the RoPE prologue;
  // at 2048 items and more the prologue serialises in front of every item's
  // K/V stream while the separate kernel runs wide (80-layer 70B-shaped step
  // at 256 rows: 55.8 ms separate, 58.7 ms fused), so the separate kernel
  // runs there
  int a_pt = 0, a_np = 0, a_waves = 1;
  attn_partition(n_tok, nkv, e->maxb * NS_BLOCK_SIZE, &a_pt, &a_np, &a_waves);
  const bool fuse = fused_rope(e, sc) && a_waves > 1 && (long)n_tok * nkv < 2048;
  const bool late_first = sc.decode_rows_first != 0 && nano.size() > 1;
  const bool defer0 = sc.decode_rows_first != 0 && qparts.size() > 1;
  int layer = 0;
  auto attend = [&](size_t j) -> int {
    const int r0 = qparts[j].first, n = qparts[j].second - r0;
    ns::AttnArgs a;
    attn_args(e, layer, r0, r0 + n, n_tok, &a);
    if (fuse) {
      a.rope_qkv = dec ? pq : qkv;
      a.rope_slice_stride = dec ? sq : 0;
      a.rope_splits = S_qkv;
      a.cosb = e->cosb();
      a.sinb = e->sinb();
      a.slot = e->m_slot();
      a.row_seq = nullptr;
    }
    if (overlap) HIP_TRY(hipStreamWaitEvent(sa, e->ev_qkv[j], 0));
    ns::launch_attention(a, sa);
    launches += a.n_parts > 1 ? 2 : 1;
    MARK(K_ATTN);
    if (overlap) HIP_TRY(hipEventRecord(e->ev_att[j], sa));
    return NS_OK;
  };
  for (int l = 0; l < d.n_layers; ++l) {
    layer = l;
    for (size_t j = 0; j < qparts.size(); ++j) {
      const int r0 = qparts[j].first, n = qparts[j].second - r0;
      if (l > 0) {  // layer 0's norm ran in the prologue
        if (dec)      // finishing the previous layer's down projection
          ns::launch_rmsnorm_reduce(dt, x + (size_t)r0 * H, pr + (size_t)r0 * H, sr, S_d, e->attn_norm[l],
                                    arow(h, r0, H), n, H, d.rms_eps, st, ar);
        else
          ns::launch_rmsnorm(dt, x + (size_t)r0 * H, e->attn_norm[l], arow(h, r0, H), n, H, d.rms_eps, st, ar);
        ++launches;
        MARK(K_NORM);
      }
      if (dec) {
        if (ns::launch_gemm_partial(n, QKV, H, arow(h, r0, H), ald(H), e->wqkv[l], QKV, pq + (size_t)r0 * QKV, QKV,
                                    sq, S_qkv, st, pk | apk))
          NS_FAIL(NS_ESHAPE, "unsupported QKV projection shape");
      } else if (ns::launch_gemm(dt, ns::EPI_STORE_F32, n, QKV, H, arow(h, r0, H), ald(H), e->wqkv[l], wld(QKV, H),
                                 qkv + (size_t)r0 * QKV, QKV, st, pk | apk)) {
        NS_FAIL(NS_ESHAPE, "unsupported QKV projection shape");
      }
      MARK(K_QKV);
      ++launches;
      if (!fuse) {
        ns::launch_rope_kv(dt, (dec ? pq : qkv) + (size_t)r0 * QKV, dec ? sq : 0, S_qkv,
                           e->cosb() + (size_t)r0 * hd / 2, e->sinb() + (size_t)r0 * hd / 2, e->m_slot() + r0,
                           (char*)e->q_att() + (size_t)r0 * DQ * es, e->k_layer(l), e->v_layer(l), n, nq, nkv, hd,
                           st);
        MARK(K_ROPE_KV);
        ++launches;
      }
      if (overlap) HIP_TRY(hipEventRecord(e->ev_qkv[j], st));
      // the decode part's attention waits until the other parts' is queued
      if (!(defer0 && j == 0)) {
        int rc = attend(j);
        if (rc) return rc;
      }
    }
    if (defer0) {
      int rc = attend(0);
      if (rc) return rc;
    }
    for (size_t ii = 0; ii < nano.size(); ++ii) {
      const size_t i = late_first ? nano.size() - 1 - ii : ii;
      const int r0 = nano[i].first, r1 = nano[i].second, n = r1 - r0;
      if (overlap)
        for (size_t j = 0; j < qparts.size(); ++j)
          if (qparts[j].first < r1 && qparts[j].second > r0) HIP_TRY(hipStreamWaitEvent(st, e->ev_att[j], 0));
      if (dec) {
        if (ns::launch_gemm_partial(n, H, DQ, arow(o, r0, DQ), ald(DQ), e->wo[l], H, pr + (size_t)r0 * H, H, sr, S_o,
                                    st, pk | apk))
          NS_FAIL(NS_ESHAPE, "unsupported O projection shape");
      } else if (ns::launch_gemm(dt, ns::EPI_RESID_F32, n, H, DQ, arow(o, r0, DQ), ald(DQ), e->wo[l], wld(H, DQ),
                                 x + (size_t)r0 * H, H, st, pk | apk)) {
        NS_FAIL(NS_ESHAPE, "unsupported O projection shape");
      }
      MARK(K_O);
      if (dec)
        ns::launch_rmsnorm_reduce(dt, x + (size_t)r0 * H, pr + (size_t)r0 * H, sr, S_o, e->mlp_norm[l],
                                  arow(h, r0, H), n, H, d.rms_eps, st, ar);
      else
        ns::launch_rmsnorm(dt, x + (size_t)r0 * H, e->mlp_norm[l], arow(h, r0, H), n, H, d.rms_eps, st, ar);
      MARK(K_NORM);
      if (ns::launch_gemm(dt, ns::EPI_SILU_MUL, n, F, H, arow(h, r0, H), ald(H), e->wgu[l], wld(2 * F, H),
                          arow(act, r0, F), ald(F), st, pk | apk | (ar ? ns::PK_C : 0)))
        NS_FAIL(NS_ESHAPE, "unsupported gate-up projection shape");
      MARK(K_GU);
      if (dec) {
        if (ns::launch_gemm_partial(n, H, F, arow(act, r0, F), ald(F), e->wdown[l], H, pr + (size_t)r0 * H, H, sr,
                                    S_d, st, pk | apk))
          NS_FAIL(NS_ESHAPE, "unsupported down projection shape");
      } else if (ns::launch_gemm(dt, ns::EPI_RESID_F32, n, H, F, arow(act, r0, F), ald(F), e->wdown[l], wld(H, F),
                                 x + (size_t)r0 * H, H, st, pk | apk)) {
        NS_FAIL(NS_ESHAPE, "unsupported down projection shape");
      }
      MARK(K_DOWN);
      launches += 4;
    }
  }
  if (d.vocab > 0) {
    if (dec)
      ns::launch_rmsnorm_reduce(dt, x, pr, sr, S_d, e->final_norm, h, n_tok, H, d.rms_eps, st, ar);
    else
      ns::launch_rmsnorm(dt, x, e->final_norm, h, n_tok, H, d.rms_eps, st, ar);
    MARK(K_NORM);
    if (ns::launch_gemm(dt, ns::EPI_STORE_F32, n_tok, d.vocab, H, h, ald(H), e->lm_head, wld(d.vocab, H), out,
                        d.vocab, st, pk | apk))
      NS_FAIL(NS_ESHAPE, "unsupported LM head shape");
    MARK(K_LM_HEAD);
    launches += 2;
  } else {
    if (dec) ns::launch_reduce_rows(x, pr, sr, S_d, (float*)out, n_tok, H, st);
    else ns::launch_copy_rows(x, (float*)out, (long)n_tok * H, st);
    ++launches;
    MARK(K_COPY);
  }
#undef MARK
  HIP_TRY(hipGetLastError());
  e->last_launches = launches;
  return NS_OK;
}

int make_second_stream(ns_engine* e, float frac) {
  if (frac > 0.f) {
    int ncu = 0;
    HIP_TRY(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
    int use = std::max(1, std::min(ncu, (int)(frac * ncu + 0.5f)));
    std::vector<uint32_t> mask((ncu + 31) / 32, 0u);
    for (int i = 0; i < use; ++i) mask[i / 32] |= 1u << (i % 32);
    HIP_TRY(hipExtStreamCreateWithCUMask(&e->s2, (uint32_t)mask.size(), mask.data()));
  } else {
    HIP_TRY(hipStreamCreateWithFlags(&e->s2, hipStreamNonBlocking));
  }
  return NS_OK;
}

// A device-fed step's out-of-range token ids: reported by a later call once
// the count copied after that step has arrived (no waiting).
int check_bad_tokens(ns_engine* e) {
  if (!e->bad_tok_copied || hipEventQuery(e->bad_tok_ev) != hipSuccess) return NS_OK;
  const int32_t n = *e->bad_tok_host;
  if (n > e->bad_tok_reported) {
    const int32_t fresh = n - e->bad_tok_reported;
    e->bad_tok_reported = n;
    NS_FAIL(NS_EINVAL, "%d device-fed token id(s) of an earlier step lay outside [0, %d); those rows gathered the "
                       "nearest valid embedding row",
            fresh, e->d.vocab);
  }
  return NS_OK;
}

// After a step that took its token ids from device memory: copy the count.
int copy_bad_tokens(ns_engine* e, const ns_batch* b, hipStream_t st) {
  if (e->d.vocab == 0 || !b->token_ids_dev) return NS_OK;
  HIP_TRY(hipMemcpyAsync(e->bad_tok_host, e->bad_tok(), sizeof(int32_t), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipEventRecord(e->bad_tok_ev, st));
  e->bad_tok_copied = true;
  return NS_OK;
}

constexpr double kDrainSeconds = 30.0;  // longest wait for the engine's work at teardown

// Poll `query` (a stream or event query) until it stops reporting work in
// flight or kDrainSeconds pass; true when it drained (or reported an error,
// which leaves nothing to wait for).
template <typename Q>
bool wait_drained(Q query) {
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    if (query() != hipErrorNotReady) return true;
    if (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > kDrainSeconds) return false;
    std::this_thread::sleep_for(std::chrono::milliseconds(1));
  }
}

}  // namespace

extern "C" {

size_t ns_workspace_bytes(const ns_model_desc* desc, int32_t max_tokens, int32_t max_blocks_per_seq) {
  if (ns::check_desc(desc) != NS_OK || max_tokens <= 0 || max_blocks_per_seq <= 0) return 0;
  return make_plan(desc, max_tokens, max_blocks_per_seq).total;
}

int ns_engine_create(const ns_model_desc* desc, const ns_weights* w, ns_kv* kv, void* kv_dev, size_t kv_bytes,
                     void* workspace, size_t ws_bytes, int32_t max_tokens, const ns_sched* sched,
                     ns_engine** out) {
  if (!out) NS_FAIL(NS_EINVAL, "null output pointer");
  int rc = ns::check_desc(desc);
  if (rc) return rc;
  if ((rc = check_sched(sched))) return rc;
  if (!w || !kv || !kv_dev || !workspace) NS_FAIL(NS_EINVAL, "null weights, kv manager, kv memory or workspace");
  if (memcmp(&kv->desc, desc, sizeof *desc) != 0) NS_FAIL(NS_EINVAL, "kv manager was created for another model");
  if (max_tokens <= 0) NS_FAIL(NS_EINVAL, "max_tokens must be positive");
  const int G = desc->n_q_heads / desc->n_kv_heads;
  const int dt = desc->dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32;
  if (!ns::attention_supported(dt, desc->head_dim, G))
    NS_FAIL(NS_EINVAL, "no attention kernel for head_dim %d, group %d", desc->head_dim, G);
  const int QKV = (desc->n_q_heads + 2 * desc->n_kv_heads) * desc->head_dim;
  if (!ns::gemm_supported(dt, desc->hidden) || !ns::gemm_supported(dt, desc->ffn) ||
      !ns::gemm_supported(dt, desc->n_q_heads * desc->head_dim) || QKV <= 0)
    NS_FAIL(NS_EINVAL, "bf16 projections need K dimensions that are multiples of 32");
  const size_t need_kv = ns_kv_bytes(desc, kv->num_blocks);
  if (kv_bytes < need_kv) NS_FAIL(NS_ESHAPE, "kv memory of %zu bytes < %zu needed", kv_bytes, need_kv);
  const Plan plan = make_plan(desc, max_tokens, kv->max_blocks);
  if (ws_bytes < plan.total) NS_FAIL(NS_ESHAPE, "workspace of %zu bytes < %zu needed", ws_bytes, plan.total);
  for (int l = 0; l < desc->n_layers; ++l)
    if (!w->attn_norm || !w->wqkv || !w->wo || !w->mlp_norm || !w->wgu || !w->wdown || !w->attn_norm[l] ||
        !w->wqkv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->wgu[l] || !w->wdown[l])
      NS_FAIL(NS_EINVAL, "missing weights of layer %d", l);
  if (desc->vocab > 0 && (!w->final_norm || !w->embed || !w->lm_head))
    NS_FAIL(NS_EINVAL, "missing embedding, final norm or LM head");

  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    NS_FAIL(NS_EINVAL, "built for gfx950 (MI355X); device is %s", prop.gcnArchName);

  ns_engine* e = new ns_engine;
  e->d = *desc;
  e->ncu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  e->es = elem_size(desc->dtype);
  e->G = G;
  for (int l = 0; l < desc->n_layers; ++l) {
    e->attn_norm.push_back(w->attn_norm[l]);
    e->wqkv.push_back(w->wqkv[l]);
    e->wo.push_back(w->wo[l]);
    e->mlp_norm.push_back(w->mlp_norm[l]);
    e->wgu.push_back(w->wgu[l]);
    e->wdown.push_back(w->wdown[l]);
  }
  e->final_norm = w->final_norm;
  e->embed = w->embed;
  e->lm_head = w->lm_head;
  e->kv = kv;
  e->kv_dev = (char*)kv_dev;
  e->kv_layer = ns::kv_layer_bytes(desc, kv->num_blocks);
  e->num_blocks = kv->num_blocks;
  e->max_tokens = max_tokens;
  e->maxb = kv->max_blocks;
  e->ws = (char*)workspace;
  e->plan = plan;
  if (sched) e->sched = *sched;
  auto fail = [&](int code) {
    (void)ns_engine_destroy(e);
    return code;
  };
  if ((rc = make_second_stream(e, e->sched.cu_mask_frac))) return fail(rc);
  for (int i = 0; i < kMaxParts; ++i) {
    if (hipEventCreateWithFlags(&e->ev_qkv[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&e->ev_att[i], hipEventDisableTiming) != hipSuccess) {
      ns::set_error("hipEventCreate failed");
      return fail(NS_EHIP);
    }
  }
  if (hipEventCreateWithFlags(&e->ev_join, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&e->bad_tok_ev, hipEventDisableTiming) != hipSuccess) {
    ns::set_error("hipEventCreate failed");
    return fail(NS_EHIP);
  }
  if (hipHostMalloc((void**)&e->bad_tok_host, sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
      hipMemset(e->bad_tok(), 0, sizeof(int32_t)) != hipSuccess) {
    ns::set_error("token-id counter set-up failed");
    return fail(NS_EHIP);
  }
  *e->bad_tok_host = 0;
  for (int k = 0; k < 2; ++k) {
    if (hipHostMalloc((void**)&e->staging[k], plan.meta_ints * sizeof(int32_t), hipHostMallocDefault) !=
            hipSuccess ||
        hipEventCreateWithFlags(&e->staging_ev[k], hipEventDisableTiming) != hipSuccess) {
      ns::set_error("pinned staging allocation failed");
      return fail(NS_EHIP);
    }
    memset(e->staging[k], 0, plan.meta_ints * sizeof(int32_t));
  }
  *out = e;
  return NS_OK;
}

int ns_engine_destroy(ns_engine* e) {
  if (!e) return NS_OK;
  // work that may still use the engine's stream, events and pinned staging
  bool drained = !e->s2 || wait_drained([&] { return hipStreamQuery(e->s2); });
  if (drained && e->bad_tok_ev) drained = wait_drained([&] { return hipEventQuery(e->bad_tok_ev); });
  for (int k = 0; k < 2 && drained; ++k)
    if (e->staging_ev[k]) drained = wait_drained([&] { return hipEventQuery(e->staging_ev[k]); });
  if (!drained)  // leave everything allocated: the work in flight still uses it
    NS_FAIL(NS_EHIP, "engine work still in flight after %.0f s; its stream, events and staging stay allocated",
            kDrainSeconds);
  if (e->s2) (void)hipStreamDestroy(e->s2);
  for (int i = 0; i < kMaxParts; ++i) {
    if (e->ev_qkv[i]) (void)hipEventDestroy(e->ev_qkv[i]);
    if (e->ev_att[i]) (void)hipEventDestroy(e->ev_att[i]);
  }
  if (e->ev_join) (void)hipEventDestroy(e->ev_join);
  if (e->bad_tok_ev) (void)hipEventDestroy(e->bad_tok_ev);
  if (e->bad_tok_host) (void)hipHostFree(e->bad_tok_host);
  for (hipEvent_t ev : e->prof_ev) (void)hipEventDestroy(ev);
  if (e->prof_start) (void)hipEventDestroy(e->prof_start);
  for (int k = 0; k < 2; ++k) {
    if (e->staging_ev[k]) (void)hipEventDestroy(e->staging_ev[k]);
    if (e->staging[k]) (void)hipHostFree(e->staging[k]);
  }
  delete e;
  return NS_OK;
}

int ns_engine_set_sched(ns_engine* e, const ns_sched* sched) {
  if (!e || !sched) NS_FAIL(NS_EINVAL, "null argument");
  int rc = check_sched(sched);
  if (rc) return rc;
  const float frac = e->sched.cu_mask_frac;
  e->sched = *sched;
  e->sched.cu_mask_frac = frac;
  return NS_OK;
}

int ns_decode_step(ns_engine* e, const ns_batch* b, void* out, void* stream) {
  if (!e || !out) NS_FAIL(NS_EINVAL, "null engine or output");
  int rc = check_batch(e, b, e->max_tokens, fused_rope(e, e->sched));
  if (rc) return rc;
  if ((rc = check_bad_tokens(e))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_meta(e, b, b->n_tok, e->sched, st))) return rc;
  if (e->d.vocab == 0)
    HIP_TRY(hipMemcpyAsync(e->x(), b->hidden_in, (size_t)b->n_tok * e->d.hidden * 4, hipMemcpyDeviceToDevice, st));
  if ((rc = enqueue_step(e, e->sched, b->n_tok, out, st, false))) return rc;
  return copy_bad_tokens(e, b, st);
}

int ns_graph_capture(ns_engine* e, int32_t bucket, void* out, void* stream, ns_graph** gout) {
  if (!e || !out || !gout) NS_FAIL(NS_EINVAL, "null argument");
  if (!stream) NS_FAIL(NS_EINVAL, "graph capture needs a non-null stream");
  if (bucket <= 0) NS_FAIL(NS_EINVAL, "bucket must be positive");
  if (bucket > e->max_tokens) NS_FAIL(NS_ESHAPE, "bucket %d exceeds max_tokens %d", bucket, e->max_tokens);
  hipStream_t st = (hipStream_t)stream;
  ns_graph* g = new ns_graph;
  g->e = e;
  g->bucket = bucket;
  g->out = out;
  g->fused_rope = fused_rope(e, e->sched);
  g->sched = e->sched;
  hipError_t he = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
  if (he != hipSuccess) {
    delete g;
    NS_FAIL(NS_EHIP, "hipStreamBeginCapture: %s", hipGetErrorString(he));
  }
  int rc = enqueue_step(e, e->sched, bucket, out, st, true);
  if (rc != NS_OK && e->sched.overlap) {
    // a step that failed after forking to the second stream: join that
    // stream back into the capture so that the capture can end
    (void)hipEventRecord(e->ev_join, e->s2);
    (void)hipStreamWaitEvent(st, e->ev_join, 0);
  }
  he = hipStreamEndCapture(st, &g->graph);
  if (rc != NS_OK || he != hipSuccess) {
    if (g->graph) (void)hipGraphDestroy(g->graph);
    delete g;
    if (rc != NS_OK) return rc;
    NS_FAIL(NS_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(he));
  }
  he = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (he != hipSuccess) {
    (void)hipGraphDestroy(g->graph);
    delete g;
    NS_FAIL(NS_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(he));
  }
  *gout = g;
  return NS_OK;
}

int ns_graph_replay(ns_graph* g, const ns_batch* b, void* stream) {
  if (!g) NS_FAIL(NS_EINVAL, "null graph");
  ns_engine* e = g->e;
  int rc = check_batch(e, b, g->bucket, g->fused_rope);
  if (rc) return rc;
  if ((rc = check_bad_tokens(e))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_meta(e, b, g->bucket, g->sched, st))) return rc;
  if (e->d.vocab == 0)
    HIP_TRY(hipMemcpyAsync(e->x(), b->hidden_in, (size_t)b->n_tok * e->d.hidden * 4, hipMemcpyDeviceToDevice, st));
  HIP_TRY(hipGraphLaunch(g->exec, st));
  return copy_bad_tokens(e, b, st);
}

int ns_graph_set_capture(ns_engine* e, const int32_t* buckets, int32_t n, void* out, void* stream,
                         ns_graph_set** sout) {
  if (!e || !buckets || !out || !sout) NS_FAIL(NS_EINVAL, "null argument");
  if (n < 1 || n > 64) NS_FAIL(NS_EINVAL, "bucket count %d outside 1..64", n);
  for (int i = 0; i < n; ++i) {
    if (buckets[i] < 1 || buckets[i] > e->max_tokens)
      NS_FAIL(NS_EINVAL, "bucket %d outside 1..max_tokens (%d)", buckets[i], e->max_tokens);
    if (i > 0 && buckets[i] <= buckets[i - 1]) NS_FAIL(NS_EINVAL, "buckets must be strictly increasing");
  }
  ns_graph_set* set = new ns_graph_set;
  for (int i = 0; i < n; ++i) {
    ns_graph* g = nullptr;
    const int rc = ns_graph_capture(e, buckets[i], out, stream, &g);
    if (rc != NS_OK) {
      ns_graph_set_destroy(set);
      return rc;
    }
    set->graphs.push_back(g);
  }
  *sout = set;
  return NS_OK;
}

int ns_graph_set_replay(ns_graph_set* set, const ns_batch* b, void* stream, int32_t* bucket_used) {
  if (!set || !b) NS_FAIL(NS_EINVAL, "null argument");
  if (b->n_tok <= 0) NS_FAIL(NS_EINVAL, "batch must have at least one row");
  for (ns_graph* g : set->graphs) {
    if (g->bucket < b->n_tok) continue;
    const int rc = ns_graph_replay(g, b, stream);
    if (rc == NS_OK && bucket_used) *bucket_used = g->bucket;
    return rc;
  }
  NS_FAIL(NS_ESHAPE, "batch of %d rows exceeds the largest bucket %d", b->n_tok, set->graphs.back()->bucket);
}

void ns_graph_set_destroy(ns_graph_set* set) {
  if (!set) return;
  for (ns_graph* g : set->graphs) ns_graph_destroy(g);
  delete set;
}

int ns_sample_greedy(const float* logits, int32_t n_rows, int32_t vocab, int32_t* tokens_out, void* stream) {
  if (!logits || !tokens_out) NS_FAIL(NS_EINVAL, "null argument");
  if (n_rows < 1 || vocab < 1) NS_FAIL(NS_EINVAL, "n_rows and vocab must be positive");
  ns::launch_argmax_rows(logits, n_rows, vocab, tokens_out, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

int ns_read_stream(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  static_assert(ns::kReadStreamGrid == NS_READ_STREAM_WORDS, "one sink word per workgroup");
  if (!src || !sink) NS_FAIL(NS_EINVAL, "null argument");
  if (bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    NS_FAIL(NS_EINVAL, "src must be 16-byte aligned and bytes a positive multiple of 16 (got %zu)", bytes);
  if (sink_words < NS_READ_STREAM_WORDS)
    NS_FAIL(NS_EINVAL, "sink holds %zu words, needs %d", sink_words, NS_READ_STREAM_WORDS);
  ns::launch_read_stream(src, (long)(bytes / 16), sink, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

void ns_graph_destroy(ns_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

int ns_kv_scatter(ns_engine* e, int32_t layer, int32_t n, const int32_t* slots, const void* k, const void* v,
                  void* stream) {
  if (!e || (n > 0 && (!slots || !k || !v))) NS_FAIL(NS_EINVAL, "null argument");
  if (layer < 0 || layer >= e->d.n_layers || n < 0) NS_FAIL(NS_EINVAL, "bad layer or count");
  ns::launch_kv_scatter(e->d.dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32, slots, k, v, e->k_layer(layer),
                        e->v_layer(layer), n, e->d.n_kv_heads, e->d.head_dim, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

int ns_kv_gather(ns_engine* e, int32_t layer, int32_t n, const int32_t* slots, void* k, void* v, void* stream) {
  if (!e || (n > 0 && (!slots || !k || !v))) NS_FAIL(NS_EINVAL, "null argument");
  if (layer < 0 || layer >= e->d.n_layers || n < 0) NS_FAIL(NS_EINVAL, "bad layer or count");
  ns::launch_kv_gather(e->d.dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32, slots, k, v, e->k_layer(layer),
                       e->v_layer(layer), n, e->d.n_kv_heads, e->d.head_dim, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

int ns_engine_profile(ns_engine* e, int32_t enable) {
  if (!e) NS_FAIL(NS_EINVAL, "null engine");
  if (enable && !e->prof_start) HIP_TRY(hipEventCreate(&e->prof_start));
  e->prof = enable != 0;
  e->prof_n = 0;
  return NS_OK;
}

int ns_engine_profile_read(ns_engine* e, int32_t cap, int32_t* kinds, float* us, int32_t* n_out) {
  if (!e || !n_out || (cap > 0 && (!kinds || !us))) NS_FAIL(NS_EINVAL, "null argument");
  const int n = std::min(cap, e->prof_n);
  if (n > 0) HIP_TRY(hipEventSynchronize(e->prof_ev[e->prof_n - 1]));
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, i ? e->prof_ev[i - 1] : e->prof_start, e->prof_ev[i]));
    kinds[i] = e->prof_kind[i];
    us[i] = ms * 1e3f;
  }
  *n_out = e->prof_n;
  return NS_OK;
}

int ns_engine_last_launches(const ns_engine* e, int32_t* out) {
  if (!e || !out) NS_FAIL(NS_EINVAL, "null argument");
  *out = e->last_launches;
  return NS_OK;
}

// ---------------------------------------------------------------- single ops
namespace {
int op_gemm(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, const void* B, void* C,
            void* stream, bool packed) {
  if (dtype != NS_F32 && dtype != NS_BF16) NS_FAIL(NS_EINVAL, "bad dtype");
  if (packed && dtype != NS_BF16) NS_FAIL(NS_EINVAL, "the K-slab-major layout is bf16 only");
  if (epi < 0 || epi > 2) NS_FAIL(NS_EINVAL, "bad epilogue");
  if (M < 0 || N < 0 || K <= 0) NS_FAIL(NS_EINVAL, "bad sizes");
  if ((M > 0 && N > 0) && (!A || !B || !C)) NS_FAIL(NS_EINVAL, "null matrix");
  const int dt = dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32;
  if (!ns::gemm_supported(dt, K)) NS_FAIL(NS_ESHAPE, "K = %d unsupported (bf16 needs K %% 32 == 0)", K);
  const int b_rows = epi == NS_EPI_SILU ? 2 * N : N;
  ns::launch_gemm(dt, epi, M, N, K, A, K, B, packed ? b_rows : K, C, N, (hipStream_t)stream, packed ? 1 : 0);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}
}  // namespace

int ns_op_gemm(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, const void* B, void* C,
               void* stream) {
  return op_gemm(dtype, epi, M, N, K, A, B, C, stream, false);
}

int ns_op_gemm_packed(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, const void* B,
                      void* C, void* stream) {
  return op_gemm(dtype, epi, M, N, K, A, B, C, stream, true);
}

int ns_op_gemm_slab(int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, int32_t a_rows, const void* B,
                    void* C, int32_t c_rows, void* stream) {
  if (epi < 0 || epi > 2) NS_FAIL(NS_EINVAL, "bad epilogue");
  if (M < 0 || N < 0 || K <= 0) NS_FAIL(NS_EINVAL, "bad sizes");
  if (M == 0 || N == 0) return NS_OK;
  if (!A || !B || !C) NS_FAIL(NS_EINVAL, "null matrix");
  if (K % 32 != 0) NS_FAIL(NS_ESHAPE, "K = %d unsupported (the slab layouts need K %% 32 == 0)", K);
  if (a_rows < M) NS_FAIL(NS_EINVAL, "a_rows %d is less than M %d", a_rows, M);
  const bool slab_c = epi == NS_EPI_SILU;
  if (slab_c && (N % 32 != 0 || c_rows < M))
    NS_FAIL(NS_EINVAL, "a slab-major SwiGLU output needs N %% 32 == 0 and c_rows >= M");
  const int b_rows = epi == NS_EPI_SILU ? 2 * N : N;
  if (ns::launch_gemm(NS_DT_BF16, epi, M, N, K, A, a_rows, B, b_rows, C, slab_c ? c_rows : N, (hipStream_t)stream,
                      ns::PK_A | ns::PK_B | (slab_c ? ns::PK_C : 0)))
    NS_FAIL(NS_ESHAPE, "unsupported shape");
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

int ns_op_rmsnorm(int32_t dtype, int32_t n_rows, int32_t hidden, const float* x, const void* gain, float eps, void* out,
                  void* stream) {
  if (dtype != NS_F32 && dtype != NS_BF16) NS_FAIL(NS_EINVAL, "bad dtype");
  if (n_rows < 0 || hidden <= 0) NS_FAIL(NS_EINVAL, "bad sizes");
  if (!(eps >= 0.f)) NS_FAIL(NS_EINVAL, "eps must be >= 0");
  if (n_rows > 0 && (!x || !gain || !out)) NS_FAIL(NS_EINVAL, "null argument");
  ns::launch_rmsnorm(dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32, x, gain, out, n_rows, hidden, eps,
                     (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

int ns_pack_weight(const void* src, void* dst, int32_t rows, int32_t cols, void* stream) {
  if (!src || !dst || src == dst) NS_FAIL(NS_EINVAL, "null or equal source and destination");
  if (rows < 1 || cols < 32 || cols % 32 != 0) NS_FAIL(NS_EINVAL, "bad shape [%d, %d]", rows, cols);
  ns::launch_pack_kslab(src, dst, rows, cols, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}

size_t ns_op_attention_ws_bytes(const ns_model_desc* desc, int32_t n_rows, int32_t max_blocks_per_seq) {
  if (ns::check_desc(desc) != NS_OK || n_rows <= 0 || max_blocks_per_seq <= 0) return 0;
  int P, np, nw;
  attn_partition(n_rows, desc->n_kv_heads, max_blocks_per_seq * NS_BLOCK_SIZE, &P, &np, &nw);
  const int G = desc->n_q_heads / desc->n_kv_heads;
  const size_t items = (size_t)n_rows * desc->n_kv_heads * np;
  return align_up(items * G * desc->head_dim * 4, 256) + align_up(items * G * 2 * 4, 256);
}

namespace {
// Argument checks shared by the attention ops (nothing enqueued).
int check_attention_args(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                         int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos, const int32_t* btab,
                         int32_t max_blocks_per_seq, void* out, int32_t wg_cap) {
  int rc = ns::check_desc(desc);
  if (rc) return rc;
  if (n_rows <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || wg_cap < 0) NS_FAIL(NS_EINVAL, "bad sizes");
  if (!q_att || !kv_layer || !row_bseq || !row_pos || !btab || !out) NS_FAIL(NS_EINVAL, "null argument");
  const int G = desc->n_q_heads / desc->n_kv_heads;
  const int dt = desc->dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32;
  if (!ns::attention_supported(dt, desc->head_dim, G))
    NS_FAIL(NS_EINVAL, "no attention kernel for head_dim %d, group %d", desc->head_dim, G);
  return NS_OK;
}

int op_attention(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                 int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos, const int32_t* btab,
                 int32_t max_blocks_per_seq, void* out, void* ws, size_t ws_bytes, int32_t wg_cap, void* stream,
                 bool tiles) {
  int rc = check_attention_args(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab,
                                max_blocks_per_seq, out, wg_cap);
  if (rc) return rc;
  const int G = desc->n_q_heads / desc->n_kv_heads;
  const int dt = desc->dtype == NS_BF16 ? NS_DT_BF16 : NS_DT_F32;
  const size_t need = ns_op_attention_ws_bytes(desc, n_rows, max_blocks_per_seq);
  if (ws_bytes < need || (need > 0 && !ws)) NS_FAIL(NS_ESHAPE, "workspace of %zu bytes < %zu", ws_bytes, need);
  ns::AttnArgs a;
  a.dtype = dt;
  a.q_att = q_att;
  a.kc = kv_layer;
  a.vc = (const char*)kv_layer + ns::kv_layer_bytes(desc, num_blocks) / 2;
  a.kv_nt = ns::kv_layer_bytes(desc, num_blocks) >= kKvStreamBytes;
  a.row_bseq = row_bseq;
  a.row_pos = row_pos;
  a.btab = btab;
  a.maxb = max_blocks_per_seq;
  a.out = out;
  a.row0 = 0;
  a.n_rows = n_rows;
  a.nq = desc->n_q_heads;
  a.nkv = desc->n_kv_heads;
  a.d = desc->head_dim;
  attn_partition(n_rows, desc->n_kv_heads, max_blocks_per_seq * NS_BLOCK_SIZE, &a.part_tokens, &a.n_parts,
                 &a.waves);
  const int G2 = G;
  const size_t items = (size_t)n_rows * desc->n_kv_heads * a.n_parts;
  a.part_acc = (float*)ws;
  a.part_ml = (float*)((char*)ws + align_up(items * G2 * desc->head_dim * 4, 256));
  a.wg_cap = wg_cap;
  a.row_seq = tiles ? row_bseq : nullptr;  // row_bseq is the sequence of each row
  ns::launch_attention(a, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return NS_OK;
}
}  // namespace

int ns_op_attention(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                    int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos, const int32_t* btab,
                    int32_t max_blocks_per_seq, void* out, void* ws, size_t ws_bytes, int32_t wg_cap,
                    void* stream) {
  return op_attention(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab, max_blocks_per_seq, out, ws,
                      ws_bytes, wg_cap, stream, false);
}

// ---------------------------------------------------------------- attention without allocation
// ns_op_attention_static keeps its split-context partials in `scratch`, a
// file-scope device array: every GPU the library runs on holds its own copy
// from module load until the process ends.  In host code the array's name
// is only a stand-in, so the device address of the current GPU's copy is
// looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive.
namespace {
constexpr size_t kStaticScratchBytes = NS_ATTENTION_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) NS_FAIL(NS_EINVAL, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) NS_FAIL(NS_EHIP, "hipGetSymbolAddress gave a null address for the static scratch");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return NS_OK;
}
}  // namespace

int ns_op_attention_static(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                           int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos, const int32_t* btab,
                           int32_t max_blocks_per_seq, void* out, int32_t wg_cap, void* stream) {
  int rc = check_attention_args(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab,
                                max_blocks_per_seq, out, wg_cap);
  if (rc) return rc;
  const size_t need = ns_op_attention_ws_bytes(desc, n_rows, max_blocks_per_seq);
  if (need > kStaticScratchBytes)
    NS_FAIL(NS_ESHAPE, "split-context partials of %zu bytes exceed the static scratch of %zu bytes (%d rows, %d blocks "
                       "per sequence); use ns_op_attention with a workspace",
            need, kStaticScratchBytes, n_rows, max_blocks_per_seq);
  void* ws = nullptr;
  if (need > 0 && (rc = static_scratch(&ws))) return rc;
  return op_attention(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab, max_blocks_per_seq, out, ws,
                      need, wg_cap, stream, false);
}

int ns_op_attention_prefill(const ns_model_desc* desc, int32_t n_rows, const void* q_att, const void* kv_layer,
                            int32_t num_blocks, const int32_t* row_bseq, const int32_t* row_pos,
                            const int32_t* btab, int32_t max_blocks_per_seq, void* out, void* ws, size_t ws_bytes,
                            int32_t wg_cap, void* stream) {
  return op_attention(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab, max_blocks_per_seq, out, ws,
                      ws_bytes, wg_cap, stream, true);
}

}  // extern "C"
