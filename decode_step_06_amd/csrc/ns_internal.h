// Internal host-side declarations shared by the C ABI translation units.
#pragma once

#include <stdarg.h>
#include <stdint.h>

#include <deque>
#include <vector>

#include "../../include/ns.h"

namespace ns {

// Record the message returned by ns_last_error() for this thread.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace ns

#define NS_FAIL(code, ...)      \
  do {                          \
    ns::set_error(__VA_ARGS__); \
    return (code);              \
  } while (0)

// Host block manager behind ns_kv_*.
struct ns_kv {
  ns_model_desc desc;
  int32_t num_blocks;
  int32_t max_seqs;
  int32_t max_blocks;  // per sequence
  std::deque<int32_t> free_list;
  std::vector<std::vector<int32_t>> tables;
};
