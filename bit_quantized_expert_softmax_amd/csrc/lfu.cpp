// LFU expert-slot cache, one per layer, host side.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", section "Qual é o principal truque da
// arquitetura": the program checks a local expert cache of 16 slots managed
// with an LFU algorithm before loading a missing expert. "Show HN: mecanismo
// de código aberto executando Gemma 4 26B em 2 GB de RAM", section
// "Abordagem técnica": more slots use more memory and improve speed.
//
// The pages give no tie-breaks. Policy implemented here, so that the event
// trace of a given id sequence is unique:
//   hit  : frequency + 1, last use = current step;
//   miss : lowest-index empty slot, else the slot with the smallest
//          (frequency, last use, slot index) among slots holding none of the
//          current token's ids; the new entry starts at frequency 1;
//   hits are applied before misses; events are reported in the ids' order.
// A policy variant for comparisons (LRU) takes the smallest (last use, slot
// index) instead. Plain C++ with no HIP dependency.
#include <string.h>

#include <vector>

#include "host_common.h"

struct moe_cache {
  int32_t n_slots = 0, n_experts = 0;
  int32_t policy = MOE_POLICY_LFU;
  std::vector<int32_t> expert;  // slot -> expert, -1 = empty
  std::vector<int32_t> freq;
  std::vector<int64_t> last;
  std::vector<int32_t> where;   // expert -> slot, -1 = absent
  int64_t tick = 0, hits = 0, misses = 0;
};

namespace moe {
std::string& last_error_text() {
  static thread_local std::string s;
  return s;
}
void cache_assign(moe_cache* dst, const moe_cache* src) { *dst = *src; }
void cache_clear_slot(moe_cache* c, int32_t slot) {
  if (slot < 0 || slot >= c->n_slots) return;
  const int32_t e = c->expert[slot];
  if (e >= 0) c->where[e] = -1;
  c->expert[slot] = -1;
  c->freq[slot] = 0;
  c->last[slot] = -1;
}
}  // namespace moe

using moe::fail;

extern "C" {

const char* moe_last_error(void) { return moe::last_error_text().c_str(); }

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_cache_create(int32_t n_slots, int32_t n_experts, moe_cache** out) {
  return moe_cache_create_policy(n_slots, n_experts, MOE_POLICY_LFU, out);
}

moe_status moe_cache_create_policy(int32_t n_slots, int32_t n_experts, int32_t policy, moe_cache** out) {
  moe::clear_error();
  if (!out) return fail(MOE_EINVAL, "moe_cache_create: out is NULL");
  if (policy != MOE_POLICY_LFU && policy != MOE_POLICY_LRU)
    return fail(MOE_EINVAL, "moe_cache_create: unknown policy %d", policy);
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ESHAPE, "moe_cache_create: n_experts %d outside [1, %d]", n_experts, MOE_MAX_EXPERTS);
  if (n_slots < 1 || n_slots > n_experts)
    return fail(MOE_ESHAPE, "moe_cache_create: n_slots %d outside [1, n_experts=%d]", n_slots, n_experts);
  moe_cache* c = new (std::nothrow) moe_cache;
  if (!c) return fail(MOE_ENOMEM, "moe_cache_create: out of host memory");
  c->n_slots = n_slots;
  c->n_experts = n_experts;
  c->policy = policy;
  c->expert.assign(n_slots, -1);
  c->freq.assign(n_slots, 0);
  c->last.assign(n_slots, -1);
  c->where.assign(n_experts, -1);
  *out = c;
  return MOE_OK;
}

void moe_cache_destroy(moe_cache* c) { delete c; }

moe_status moe_cache_reset(moe_cache* c) {
  moe::clear_error();
  if (!c) return fail(MOE_EINVAL, "moe_cache_reset: NULL cache");
  c->expert.assign(c->n_slots, -1);
  c->freq.assign(c->n_slots, 0);
  c->last.assign(c->n_slots, -1);
  c->where.assign(c->n_experts, -1);
  c->tick = c->hits = c->misses = 0;
  return MOE_OK;
}

moe_status moe_cache_step(moe_cache* c, const int32_t* ids, int32_t k, moe_cache_event* ev,
                          int32_t* n_miss) {
  moe::clear_error();
  if (!c || !ids || !ev) return fail(MOE_EINVAL, "moe_cache_step: NULL argument");
  if (k < 1 || k > c->n_slots || k > MOE_MAX_TOPK)
    return fail(MOE_ESHAPE, "moe_cache_step: k=%d must be in [1, min(n_slots=%d, %d)]", k, c->n_slots,
                MOE_MAX_TOPK);
  bool seen[MOE_MAX_EXPERTS];
  for (int j = 0; j < k; ++j) {
    if (ids[j] < 0 || ids[j] >= c->n_experts)
      return fail(MOE_EINVAL, "moe_cache_step: id %d out of range [0, %d)", ids[j], c->n_experts);
  }
  for (int e = 0; e < c->n_experts; ++e) seen[e] = false;
  for (int j = 0; j < k; ++j) {
    if (seen[ids[j]]) return fail(MOE_EINVAL, "moe_cache_step: duplicate id %d", ids[j]);
    seen[ids[j]] = true;
  }
  const int64_t t = c->tick;
  bool done[MOE_MAX_TOPK];
  int misses = 0;
  for (int j = 0; j < k; ++j) {
    const int s = c->where[ids[j]];
    done[j] = s >= 0;
    if (s >= 0) {
      c->freq[s] += 1;
      c->last[s] = t;
      ev[j] = moe_cache_event{ids[j], s, 1, -1};
    }
  }
  for (int j = 0; j < k; ++j) {
    if (done[j]) continue;
    int victim = -1;
    for (int s = 0; s < c->n_slots; ++s)
      if (c->expert[s] < 0) { victim = s; break; }
    if (victim < 0) {
      for (int s = 0; s < c->n_slots; ++s) {
        if (seen[c->expert[s]]) continue;  // holds an id of this token
        if (victim < 0) {
          victim = s;
          continue;
        }
        const bool better = c->policy == MOE_POLICY_LRU
                                ? c->last[s] < c->last[victim]
                                : c->freq[s] < c->freq[victim] ||
                                      (c->freq[s] == c->freq[victim] && c->last[s] < c->last[victim]);
        if (better) victim = s;  // scanning upward keeps the lower index on full ties
      }
    }
    const int old = c->expert[victim];
    if (old >= 0) c->where[old] = -1;
    c->expert[victim] = ids[j];
    c->freq[victim] = 1;
    c->last[victim] = t;
    c->where[ids[j]] = victim;
    ev[j] = moe_cache_event{ids[j], victim, 0, old};
    ++misses;
  }
  c->hits += k - misses;
  c->misses += misses;
  c->tick += 1;
  if (n_miss) *n_miss = misses;
  return MOE_OK;
}

moe_status moe_cache_slots(const moe_cache* c, int32_t* expert, int32_t* freq, int64_t* last,
                           int32_t n) {
  moe::clear_error();
  if (!c) return fail(MOE_EINVAL, "moe_cache_slots: NULL cache");
  if (n != c->n_slots) return fail(MOE_ESHAPE, "moe_cache_slots: n=%d but n_slots=%d", n, c->n_slots);
  for (int s = 0; s < n; ++s) {
    if (expert) expert[s] = c->expert[s];
    if (freq) freq[s] = c->freq[s];
    if (last) last[s] = c->last[s];
  }
  return MOE_OK;
}

moe_status moe_cache_counters(const moe_cache* c, int64_t* hits, int64_t* misses, int64_t* steps) {
  moe::clear_error();
  if (!c) return fail(MOE_EINVAL, "moe_cache_counters: NULL cache");
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (steps) *steps = c->tick;
  return MOE_OK;
}

}  // extern "C"
