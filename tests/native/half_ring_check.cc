// Host check of the grouped GEMM's half-stage load schedule (half_ring.h).
//
// The schedule is simulated directly: every load a wave issues is appended
// to a list in issue order (front weight sub-steps, prologue, then the loop),
// each wait point records how many loads were issued before it, and the
// exact number of loads younger than what a sub-step needs is read off the
// list.  Checked for every schedule shape in a grid and every loop length:
//   * younger() and younger_fast() equal the exact count;
//   * for schedules with head_ok(), the count the kernel waits with never
//     exceeds it
//     (a larger count would let a sub-step start before its data landed);
//   * every load fills a slot whose previous contents were read before the
//     barrier that precedes the load (lag 0: the wave waits for its own LDS
//     reads before each barrier; lag 1: it does not, and a read is known
//     complete only once the MFMAs that use it were issued, i.e. by the
//     barrier after the one that follows the read);
//   * every weight sub-step and A stage is loaded exactly once, before the
//     wait that needs it.
// Prints "ok <cases>" or the first failures.
#include <cstdio>
#include <initializer_list>
#include <vector>

#include "half_ring.h"

using namespace beam::half_ring;

struct Load {
  bool a;     // A stage (else weight sub-step)
  int idx;    // stage / sub-step
  int iter;   // loop iteration that issued it (prologue: negative, front: -1000)
};

static long fails = 0;
#define CHECK(c, ...)                                  \
  do {                                                 \
    if (!(c)) {                                        \
      if (fails < 20) { printf(__VA_ARGS__); printf("\n"); } \
      ++fails;                                         \
    }                                                  \
  } while (0)

int main() {
  long cases = 0;
  for (int L = 0; L <= 1; ++L)
  for (int SA = 2; SA <= 4; ++SA)
    for (int SB = 3; SB <= 8; ++SB)
      for (int KP = 0; KP < SB; ++KP)
        for (int nbl = 1; nbl <= 2; ++nbl)
          for (int na2 = 0; na2 <= 4; na2 += 2) {
            // the kernel's rule for a wave with na2 A loads per stage whose
            // workgroup also has waves with na2 + 2 (or na2 - 2): the larger
            // tail length and minimum depth of the pair
            const bool ok_head = head_ok(SA, SB, KP, L, nbl, na2);
            if (SB < L + 2 || 2 * SA < L + 3) continue;  // a load would be issued after its wait
            int dmin = deep_min(SA, SB, KP, L, nbl, na2), T = steady_tail(SA, SB, KP, L, nbl, na2);
            for (int o : {na2 - 2, na2 + 2})
              if (o >= 0) {
                dmin = dmin > deep_min(SA, SB, KP, L, nbl, o) ? dmin : deep_min(SA, SB, KP, L, nbl, o);
                T = T > steady_tail(SA, SB, KP, L, nbl, o) ? T : steady_tail(SA, SB, KP, L, nbl, o);
              }
            const int st[2] = {steady(SA, SB, KP, L, nbl, na2, 0), steady(SA, SB, KP, L, nbl, na2, 1)};
            int tail[130];
            for (int d = 1; d < 130; ++d) tail[d] = tail_count(SA, SB, KP, L, nbl, na2, d);
            for (int nk = 4; nk <= 120; nk += 2) {
              const int nst = nk / 2;
              std::vector<Load> loads;
              std::vector<int> b_slot_owner(SB, -1), a_slot_owner(SA, -1);
              std::vector<int> b_count(nk, 0), a_count(nst, 0);
              // Operands of sub-step s are read in iteration s - 1 (s = 0:
              // before the loop) and used by the MFMAs of iteration s.  A
              // slot may be refilled in iteration kt if its owner's last
              // reading sub-step is <= kt - L.
              auto add_b = [&](int s, int iter) {
                const int slot = s % SB;
                if (b_slot_owner[slot] >= 0)
                  CHECK(b_slot_owner[slot] <= iter - L, "B slot reuse L%d SA%d SB%d KP%d nk%d s%d", L, SA, SB, KP, nk, s);
                b_slot_owner[slot] = s;
                ++b_count[s];
                loads.push_back({false, s, iter});
              };
              auto add_a = [&](int q, int iter) {
                const int slot = q % SA;
                if (a_slot_owner[slot] >= 0)  // stage q' read by sub-steps 2q' and 2q'+1
                  CHECK(2 * a_slot_owner[slot] + 1 <= iter - L, "A slot reuse L%d SA%d SB%d nk%d q%d", L, SA, SB, nk, q);
                a_slot_owner[slot] = q;
                ++a_count[q];
                loads.push_back({true, q, iter});
              };
              // front weight sub-steps (slots free: the previous item is done)
              for (int s = 0; s < KP && s < nk; ++s) add_b(s, -1000);
              // prologue: model iterations that precede the loop's first
              auto model = [&](int j, int iter) {
                if (j % 2 != 0 && (j - 1) / 2 + SA >= 0 && (j - 1) / 2 + SA < nst) add_a((j - 1) / 2 + SA, iter);
                if (j + SB >= KP && j + SB < nk) add_b(j + SB, iter);
              };
              for (int j = first_iter(SA, SB); j < -L; ++j) model(j, -1000);
              // waits[s] = loads issued when sub-step s's wait happens
              std::vector<size_t> issued_at(nk, 0);
              issued_at[0] = loads.size();
              for (int kt = 0; kt < nk; ++kt) {
                if (kt + 1 < nk) issued_at[kt + 1] = loads.size();  // wait precedes this iteration's issues
                model(kt - L, kt);
              }
              for (int s = 0; s < nk; ++s) CHECK(b_count[s] == 1, "B%d loaded %d times", s, b_count[s]);
              for (int q = 0; q < nst; ++q) CHECK(a_count[q] == 1, "A%d loaded %d times", q, a_count[q]);
              for (int s = 0; s < nk; ++s) {
                // youngest needed load among those issued before the wait
                int youngest = -1;
                for (size_t i = 0; i < issued_at[s]; ++i)
                  if ((!loads[i].a && loads[i].idx == s) || (loads[i].a && s % 2 == 0 && loads[i].idx == s / 2))
                    youngest = (int)i;
                bool have_b = false, have_a = s % 2 != 0;
                for (size_t i = 0; i < issued_at[s]; ++i) {
                  if (!loads[i].a && loads[i].idx == s) have_b = true;
                  if (loads[i].a && s % 2 == 0 && loads[i].idx == s / 2) have_a = true;
                }
                CHECK(have_b && have_a, "sub-step %d waited before its loads were issued (SA%d SB%d KP%d nk%d)", s, SA, SB, KP, nk);
                int exact = 0;
                for (size_t i = youngest + 1; i < issued_at[s]; ++i) exact += loads[i].a ? na2 : nbl;
                const int last = last_of(s, L);
                const int y = younger(SA, SB, KP, nbl, na2, nk, s, last);
                const int yf = younger_fast(SA, SB, KP, nbl, na2, nk, s, last);
                CHECK(y == exact && yf == exact, "count L%d SA%d SB%d KP%d nbl%d na2%d nk%d s%d: exact %d younger %d fast %d",
                      L, SA, SB, KP, nbl, na2, nk, s, exact, y, yf);
                if (ok_head && s >= 1) {
                  const int p = nk < dmin ? 0 : s + T < nk ? st[s & 1] : tail[nk - s];
                  CHECK(p <= exact, "policy L%d SA%d SB%d KP%d nbl%d na2%d nk%d s%d: waits for %d > exact %d",
                        L, SA, SB, KP, nbl, na2, nk, s, p, exact);
                }
                ++cases;
              }
            }
          }
  // the shapes the kernel runs (3 A slots; 7, 5 and 4 weight slots at 128-,
  // 192- and 256-row tiles; 2 front sub-steps; either lag; 2 weight loads per
  // sub-step; 0, 2 or 4 A loads per stage) pass the head check
  for (int L = 0; L <= 1; ++L)
    for (int SB : {7, 5, 4})
      for (int na2 : {0, 2, 4})
        CHECK(head_ok(3, SB, 2, L, 2, na2), "kernel shape L%d SB%d na2%d fails head_ok", L, SB, na2);
  if (fails) {
    printf("FAILED %ld of %ld\n", fails, cases);
    return 1;
  }
  printf("ok %ld\n", cases);
  return 0;
}
