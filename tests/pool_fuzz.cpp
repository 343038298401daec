// Random alloc / free / claim_run / release_run sequences against the host page pool, with the free
// count checked after each step and refusals probed (pages out of range, a page listed twice, a
// range that is not a claimed run, part of a run).  tests/test_pool_sanitizer.py builds it with g++
// under AddressSanitizer and UBSan together with the pool's source.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <vector>
#include <algorithm>
#include <random>
extern "C" {
size_t paged_pool_state_bytes(int32_t n_pages);
int paged_pool_init(void* state, size_t state_size, int32_t n_pages);
int paged_pool_alloc(void* state, int32_t n, int32_t* pages);
int paged_pool_free(void* state, const int32_t* pages, int32_t n);
int paged_pool_claim_run(void* state, int32_t k, int32_t* first);
int paged_pool_release_run(void* state, int32_t first, int32_t k);
int32_t paged_pool_free_count(const void* state);
}
int main() {
  std::mt19937 rng(7);
  long ops = 0;
  for (int trial = 0; trial < 300; ++trial) {
    const int n = 1 + rng() % 300;
    std::vector<uint64_t> st((paged_pool_state_bytes(n) + 7) / 8);
    if (paged_pool_init(st.data(), st.size() * 8, n) != 0) { puts("init failed"); return 1; }
    std::vector<int32_t> held;
    std::vector<std::pair<int, int>> runs;
    for (int step = 0; step < 2000; ++step, ++ops) {
      const int op = rng() % 6;
      if (op == 0) {
        const int k = 1 + rng() % 8;
        std::vector<int32_t> p(k);
        if (paged_pool_alloc(st.data(), k, p.data()) == 0) held.insert(held.end(), p.begin(), p.end());
      } else if (op == 1 && !held.empty()) {
        std::shuffle(held.begin(), held.end(), rng);
        const int k = 1 + rng() % std::min<int>(8, held.size());
        if (paged_pool_free(st.data(), held.data() + held.size() - k, k) != 0) { puts("free refused"); return 1; }
        held.resize(held.size() - k);
      } else if (op == 2) {
        const int k = 1 + rng() % 16;
        int32_t f;
        if (paged_pool_claim_run(st.data(), k, &f) == 0) runs.push_back({f, k});
      } else if (op == 3 && !runs.empty()) {
        const int i = rng() % runs.size();
        if (paged_pool_release_run(st.data(), runs[i].first, runs[i].second) != 0) { puts("release refused"); return 1; }
        runs.erase(runs.begin() + i);
      } else if (op == 4) {  // refusals: bad pages, bad runs, double free
        int32_t bad[2] = {(int32_t)(rng() % (2 * n)) - n / 2, n + (int32_t)(rng() % 5)};
        paged_pool_free(st.data(), bad, 2);
        {
          const int32_t f = (rng() & 1) ? n + (int32_t)(rng() % 5) : -1 - (int32_t)(rng() % 5);
          if (paged_pool_release_run(st.data(), f, 1 + rng() % 4) == 0) { puts("bad release accepted"); return 1; }
          // a range of pages handed out singly is not a run either
          if (!held.empty() && paged_pool_release_run(st.data(), held.back(), 1) == 0) { puts("page released as a run"); return 1; }
          if (!runs.empty() && runs[0].second >= 2) {
            if (paged_pool_release_run(st.data(), runs[0].first + 1, runs[0].second - 1) == 0) { puts("part of a run released"); return 1; }
            if (paged_pool_release_run(st.data(), runs[0].first, runs[0].second - 1) == 0) { puts("short release accepted"); return 1; }
          }
        }
        if (!held.empty()) { int32_t d[2] = {held[0], held[0]}; if (paged_pool_free(st.data(), d, 2) == 0) { puts("double free accepted"); return 1; } }
      } else {
        int32_t fc = paged_pool_free_count(st.data());
        long used = (long)held.size(); for (auto& r : runs) used += r.second;
        if (fc != n - used) { printf("count %d vs %ld\n", fc, n - used); return 1; }
      }
    }
  }
  printf("ok, %ld operations\n", ops);
  return 0;
}
