// Reads "n_slots n_experts k T" then T lines of k ids from stdin, runs the
// library's LFU cache and prints one line per event: step expert slot hit evicted.
// Built with g++ and the address/undefined-behaviour sanitizers by the tests.
#include <stdio.h>

#include <vector>

#include "moedecode.h"

int main() {
  int S, E, k, T;
  if (scanf("%d %d %d %d", &S, &E, &k, &T) != 4) return 2;
  moe_cache* c = nullptr;
  if (moe_cache_create(S, E, &c) != MOE_OK) return 3;
  std::vector<int32_t> ids(k);
  std::vector<moe_cache_event> ev(k);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j)
      if (scanf("%d", &ids[j]) != 1) return 4;
    int32_t nm = 0;
    const moe_status st = moe_cache_step(c, ids.data(), k, ev.data(), &nm);
    if (st != MOE_OK) {
      printf("ERR %d %d\n", t, st);
      continue;
    }
    for (int j = 0; j < k; ++j)
      printf("%d %d %d %d %d\n", t, ev[j].expert, ev[j].slot, ev[j].hit, ev[j].evicted);
  }
  int64_t h, m, s;
  moe_cache_counters(c, &h, &m, &s);
  printf("END %lld %lld %lld\n", (long long)h, (long long)m, (long long)s);
  moe_cache_destroy(c);
  return 0;
}
