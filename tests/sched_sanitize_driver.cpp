// Host driver for the scheduler under AddressSanitizer and UBSan: random
// configurations (policies, block sizes, pool sizes down to zero, item counts
// down to one), several calls per state, a rejected bad query after each
// call, and a read of the pools.  Built and run by tests/test_schedule.py with
// g++ (host code only; the scheduler has no device code).
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <random>
#include "bat.h"
int main() {
  std::mt19937 g(1);
  for (int trial = 0; trial < 300; ++trial) {
    bat_sched_config c{};
    c.policy = trial % 2;
    c.item_tokens = 1 + g() % 8;
    c.user_block = 1 + g() % 64;
    c.item_capacity = g() % 40;
    c.user_capacity_blocks = g() % 200;
    c.num_users = 1 + g() % 50;
    c.num_items = 1 + g() % 120;
    std::vector<int32_t> ul(c.num_users);
    for (auto &x : ul) x = g() % 2000;
    size_t n = bat_sched_state_size(&c);
    std::vector<uint64_t> st((n + 7) / 8);
    if (bat_sched_init(&c, ul.data(), st.data(), n) != BAT_OK) { printf("init fail\n"); return 1; }
    int m = g() % (c.num_items < 16 ? c.num_items + 1 : 16);
    for (int call = 0; call < 5; ++call) {
      int R = g() % 200;
      std::vector<int32_t> u(R), it((size_t)R * m), slot((size_t)R * m);
      for (auto &x : u) x = g() % c.num_users;
      for (int r = 0; r < R; ++r) {
        std::vector<int> perm(c.num_items);
        for (int i = 0; i < c.num_items; ++i) perm[i] = i;
        for (int j = 0; j < m; ++j) { int k = j + g() % (c.num_items - j); std::swap(perm[j], perm[k]); it[(size_t)r * m + j] = perm[j]; }
      }
      std::vector<uint8_t> mode(R), uh(R); std::vector<int32_t> ih(R); std::vector<int64_t> pt(R), stt(R), pr(R);
      if (bat_sched_step(st.data(), R, m, u.data(), it.data(), mode.data(), uh.data(), ih.data(), pt.data(), stt.data(), pr.data(), slot.data()) != BAT_OK) { printf("step fail\n"); return 1; }
      // a bad query must be rejected
      if (R > 0) { int32_t bad = c.num_users; if (bat_sched_step(st.data(), 1, m, &bad, it.data(), 0,0,0,0,0,0,0) != BAT_ERR_INVALID_ARG) { printf("no reject\n"); return 1; } }
    }
    std::vector<int32_t> ru(c.num_users), si(c.item_capacity + 1); int32_t nr = 0;
    if (bat_sched_pools(st.data(), ru.data(), &nr, si.data()) != BAT_OK) return 1;
  }
  printf("asan driver ok\n");
  return 0;
}
