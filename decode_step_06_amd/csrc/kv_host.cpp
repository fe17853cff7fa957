// Paged KV-cache block manager and token -> slot mapping (host only).
//
// Page "gpu-waiting-not-working" (nanoserve notes), changes table and the
// paragraph after it: each sequence owns a table of fixed-size cache blocks
// and every token is mapped to a cache slot through it.  The policy is a FIFO
// free list in a caller-given initial order: a sequence grows by taking
// blocks from the head (all or nothing) and a freed sequence returns its
// blocks to the tail in table order.  slot = table[seq][pos / 16] * 16 +
// pos % 16.
#include <stdio.h>
#include <string.h>

#include <string>

#include "ns_internal.h"

namespace ns {

static thread_local std::string g_last_error = "no error";

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

const char* last_error() { return g_last_error.c_str(); }

static int elem_bytes(int32_t dtype) { return dtype == NS_BF16 ? 2 : 4; }

int check_desc(const ns_model_desc* d) {
  if (!d) NS_FAIL(NS_EINVAL, "null model descriptor");
  if (d->n_layers <= 0 || d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->ffn <= 0 ||
      d->vocab < 0)
    NS_FAIL(NS_EINVAL, "model sizes must be positive");
  if (d->n_q_heads % d->n_kv_heads) NS_FAIL(NS_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
    NS_FAIL(NS_EINVAL, "head_dim must be 32, 64 or 128 (got %d)", d->head_dim);
  if (d->n_q_heads / d->n_kv_heads > 8) NS_FAIL(NS_EINVAL, "query heads per KV head must be <= 8");
  if (d->dtype != NS_F32 && d->dtype != NS_BF16) NS_FAIL(NS_EINVAL, "dtype must be NS_F32 or NS_BF16");
  if (!(d->rms_eps > 0.f) || !(d->rope_base > 1.f)) NS_FAIL(NS_EINVAL, "rms_eps must be > 0, rope_base > 1");
  return NS_OK;
}

size_t kv_layer_bytes(const ns_model_desc* d, int32_t num_blocks) {
  return 2ull * (size_t)num_blocks * d->n_kv_heads * NS_BLOCK_SIZE * d->head_dim * elem_bytes(d->dtype);
}

}  // namespace ns

extern "C" {

const char* ns_last_error(void) { return ns::last_error(); }

size_t ns_kv_bytes(const ns_model_desc* desc, int32_t num_blocks) {
  if (ns::check_desc(desc) != NS_OK || num_blocks <= 0) return 0;
  return ns::kv_layer_bytes(desc, num_blocks) * (size_t)desc->n_layers;
}

int ns_kv_create(const ns_model_desc* desc, int32_t num_blocks, int32_t max_seqs, int32_t max_blocks_per_seq,
                 const int32_t* free_order, ns_kv** out) {
  if (!out) NS_FAIL(NS_EINVAL, "null output pointer");
  int rc = ns::check_desc(desc);
  if (rc) return rc;
  if (num_blocks <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0)
    NS_FAIL(NS_EINVAL, "num_blocks, max_seqs and max_blocks_per_seq must be positive");
  if ((int64_t)num_blocks * NS_BLOCK_SIZE >= (1ll << 31)) NS_FAIL(NS_EINVAL, "slot ids must fit int32");
  std::vector<int32_t> order(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) NS_FAIL(NS_EINVAL, "free_order is not a permutation of the pool");
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  ns_kv* kv = new ns_kv;
  kv->desc = *desc;
  kv->num_blocks = num_blocks;
  kv->max_seqs = max_seqs;
  kv->max_blocks = max_blocks_per_seq;
  kv->free_list.assign(order.begin(), order.end());
  kv->tables.assign(max_seqs, {});
  *out = kv;
  return NS_OK;
}

int ns_kv_alloc(ns_kv* kv, int32_t seq, int32_t n_tokens) {
  if (!kv) NS_FAIL(NS_EINVAL, "null kv manager");
  if (seq < 0 || seq >= kv->max_seqs) NS_FAIL(NS_EINVAL, "sequence %d out of range [0, %d)", seq, kv->max_seqs);
  if (n_tokens < 0) NS_FAIL(NS_EINVAL, "negative token count");
  const int64_t want = ((int64_t)n_tokens + NS_BLOCK_SIZE - 1) / NS_BLOCK_SIZE;
  if (want > kv->max_blocks)
    NS_FAIL(NS_ESHAPE, "sequence %d needs %lld blocks, table rows hold %d", seq, (long long)want, kv->max_blocks);
  auto& tab = kv->tables[seq];
  const int64_t extra = want - (int64_t)tab.size();
  if (extra <= 0) return NS_OK;
  if (extra > (int64_t)kv->free_list.size())
    NS_FAIL(NS_ENOBLOCKS, "pool exhausted: need %lld blocks, %zu free", (long long)extra, kv->free_list.size());
  for (int64_t i = 0; i < extra; ++i) {
    tab.push_back(kv->free_list.front());
    kv->free_list.pop_front();
  }
  return NS_OK;
}

int ns_kv_free_seq(ns_kv* kv, int32_t seq) {
  if (!kv) NS_FAIL(NS_EINVAL, "null kv manager");
  if (seq < 0 || seq >= kv->max_seqs) NS_FAIL(NS_EINVAL, "sequence %d out of range [0, %d)", seq, kv->max_seqs);
  for (int32_t b : kv->tables[seq]) kv->free_list.push_back(b);
  kv->tables[seq].clear();
  return NS_OK;
}

int ns_kv_block_table(const ns_kv* kv, int32_t* out) {
  if (!kv || !out) NS_FAIL(NS_EINVAL, "null argument");
  for (int32_t s = 0; s < kv->max_seqs; ++s) {
    const auto& tab = kv->tables[s];
    int32_t* row = out + (size_t)s * kv->max_blocks;
    for (int32_t j = 0; j < kv->max_blocks; ++j) row[j] = j < (int32_t)tab.size() ? tab[j] : -1;
  }
  return NS_OK;
}

int ns_kv_capacity(const ns_kv* kv, int32_t seq, int32_t* tokens_out) {
  if (!kv || !tokens_out) NS_FAIL(NS_EINVAL, "null argument");
  if (seq < 0 || seq >= kv->max_seqs) NS_FAIL(NS_EINVAL, "sequence %d out of range [0, %d)", seq, kv->max_seqs);
  *tokens_out = (int32_t)kv->tables[seq].size() * NS_BLOCK_SIZE;
  return NS_OK;
}

int ns_kv_num_free(const ns_kv* kv, int32_t* out) {
  if (!kv || !out) NS_FAIL(NS_EINVAL, "null argument");
  *out = (int32_t)kv->free_list.size();
  return NS_OK;
}

void ns_kv_destroy(ns_kv* kv) { delete kv; }

int ns_slot_map(const ns_kv* kv, int32_t n_tok, const int32_t* seq, const int32_t* pos, int32_t* slot_out) {
  if (!kv) NS_FAIL(NS_EINVAL, "null kv manager");
  if (n_tok < 0) NS_FAIL(NS_EINVAL, "negative row count");
  if (n_tok > 0 && (!seq || !pos || !slot_out)) NS_FAIL(NS_EINVAL, "null array");
  for (int32_t i = 0; i < n_tok; ++i) {  // validate first: no partial output
    if (seq[i] == -1) continue;
    if (seq[i] < 0 || seq[i] >= kv->max_seqs) NS_FAIL(NS_EINVAL, "row %d: sequence %d out of range", i, seq[i]);
    if (pos[i] < 0 || (int64_t)pos[i] >= (int64_t)kv->tables[seq[i]].size() * NS_BLOCK_SIZE)
      NS_FAIL(NS_ESHAPE, "row %d: position %d beyond the %zu blocks of sequence %d", i, pos[i],
              kv->tables[seq[i]].size(), seq[i]);
  }
  for (int32_t i = 0; i < n_tok; ++i) {
    if (seq[i] == -1) {
      slot_out[i] = -1;
      continue;
    }
    const int32_t p = pos[i];
    slot_out[i] = kv->tables[seq[i]][p / NS_BLOCK_SIZE] * NS_BLOCK_SIZE + p % NS_BLOCK_SIZE;
  }
  return NS_OK;
}

}  // extern "C"
