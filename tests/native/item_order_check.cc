// Host check of the grouped GEMM's item orders (item_order.h) on random
// plans: experts with 0..40 m-tiles, 1..70 n-tiles per m-tile.
//   * plain and blocked orders both visit every (m-tile, n-tile) exactly once
//     over q = 0 .. tiles * nt_n - 1, and item q stays within the expert of
//     m-tile q / nt_n (so a workgroup's next-item weights are that expert's);
//   * in the blocked order, any 32 consecutive items inside one n-group of an
//     expert with at least 8 m-tiles span at most 9 m-tiles and 4 n-tiles.
// Prints "ok <plans>" or the first failures.
#include <cstdio>
#include <cstdint>
#include <random>
#include <set>
#include <vector>

#include "item_order.h"

static long fails = 0;
#define CHECK(c, ...)                                            \
  do {                                                           \
    if (!(c)) {                                                  \
      if (fails < 20) { printf(__VA_ARGS__); printf("\n"); }     \
      ++fails;                                                   \
    }                                                            \
  } while (0)

int main() {
  std::mt19937 rng(12345);
  int plans = 0;
  for (int trial = 0; trial < 400; ++trial) {
    const int E = 1 + rng() % 12;
    const int nt_n = trial < 200 ? 20 : 1 + rng() % 70;
    std::vector<int32_t> expert, first, count;
    for (int e = 0; e < E; ++e) {
      const int M = rng() % 4 == 0 ? 0 : (rng() % 3 == 0 ? 8 + rng() % 33 : 1 + rng() % 3);
      const int f = (int)expert.size();
      for (int m = 0; m < M; ++m) {
        expert.push_back(e);
        first.push_back(f);
        count.push_back(M);
      }
    }
    const int tiles = (int)expert.size();
    const int total = tiles * nt_n;
    for (int blocked = 0; blocked < 2; ++blocked) {
      std::vector<int> seen((size_t)total, 0);
      for (int q = 0; q < total; ++q) {
        int t, n;
        beam::item_of(q, nt_n, blocked ? first.data() : nullptr, blocked ? count.data() : nullptr, t, n);
        CHECK(t >= 0 && t < tiles && n >= 0 && n < nt_n, "out of range q%d", q);
        if (t < 0 || t >= tiles || n < 0 || n >= nt_n) continue;
        CHECK(expert[t] == expert[q / nt_n], "q%d left its expert", q);
        ++seen[(size_t)t * nt_n + n];
      }
      for (int i = 0; i < total; ++i) CHECK(seen[i] == 1, "item %d visited %d times (blocked %d)", i, seen[i], blocked);
    }
    // block shape of hot experts in the blocked order
    for (int t = 0; t < tiles; t += count[t]) {
      const int M = count[t];
      if (M < 8) continue;
      const int base = t * nt_n, groups = nt_n / beam::kGroupN;
      for (int g = 0; g < groups; ++g)
        for (int s = 0; s + 32 <= beam::kGroupN * M; ++s) {
          std::set<int> ms, ns;
          for (int k = 0; k < 32; ++k) {
            int tt, n;
            beam::item_of(base + g * beam::kGroupN * M + s + k, nt_n, first.data(), count.data(), tt, n);
            ms.insert(tt);
            ns.insert(n);
          }
          CHECK(ms.size() <= 9 && ns.size() <= 4, "window of expert at tile %d: %zu m-tiles %zu n-tiles", t, ms.size(), ns.size());
        }
    }
    ++plans;
  }
  if (fails) {
    printf("FAILED %ld\n", fails);
    return 1;
  }
  printf("ok %d\n", plans);
  return 0;
}
