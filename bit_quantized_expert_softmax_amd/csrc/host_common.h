// Host-side helpers shared by the C-ABI entry points: thread-local error
// text, status returns and argument checks. No HIP dependency.
#pragma once

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "moedecode.h"

namespace moe {

std::string& last_error_text();

inline moe_status fail(moe_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error_text() = buf;
  return code;
}

// Copies the whole state of one cache into another of the same size.
void cache_assign(moe_cache* dst, const moe_cache* src);
// Empties one slot (expert -1, frequency 0, never used), as if it had never
// been filled; the counters and the step are unchanged.
void cache_clear_slot(moe_cache* c, int32_t slot);

inline void clear_error() { last_error_text().clear(); }

// Whether a store holds layer `layer` of n_experts blobs of blob_bytes each.
bool store_fits(const moe_store* s, int layer, int n_experts, int64_t blob_bytes);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace moe
