// Load schedule of the grouped GEMM's bf16 pipeline for 128..256-row tiles,
// and the vmcnt wait counts it implies.  Plain constexpr C++ (no HIP types),
// so that a host program can check the counts against a simulation of the
// schedule.
//
// The k loop runs sub-steps kt = 0 .. nk-1 of 32 k.  Weights (B) sit in a ring
// of SB half-stage slots (one 32-k sub-step each), activations (A) in a ring of
// SA slots of one 64-k stage (two sub-steps) each.  Iteration kt of the loop
// waits for the operands of sub-step kt + 1, passes one workgroup barrier and
// then refills the slots that sub-step j = kt - L's operands came from ("model
// iteration" j):
//
//   j odd:   A stage (j - 1) / 2 + SA   into A slot ((j - 1) / 2) % SA
//   always:  B sub-step j + SB          into B slot j % SB
//
// (A first, then B), each only if it exists (A stage < nk / 2, B sub-step <
// nk).  Lag L = 0: the barrier must follow the wave's wait for its own LDS
// reads of sub-step kt's operands (issued in iteration kt - 1).  L = 1: the
// slots refilled are those of sub-step kt - 1, whose operand reads every wave
// completed before issuing that sub-step's MFMAs, so no such wait is needed;
// each ring looks one sub-step less ahead.  The prologue issues what model
// iterations jmin .. -1 - L would have issued by the same rule, except that
// the first KP weight sub-steps come before everything else ("front" loads:
// for every item but a workgroup's first they are issued by the workgroup's
// previous item, before its epilogue).
//
// A wave's vector memory loads complete in issue order, so "everything a
// sub-step needs has landed" is "at most N loads remain outstanding", N being
// the number of loads issued after the youngest load the sub-step needs.  Each
// B sub-step is nbl loads per wave, each A stage na2 loads.
#pragma once

#ifndef BEAM_HD
#if defined(__HIPCC__)
#define BEAM_HD __host__ __device__
#else
#define BEAM_HD
#endif
#endif

namespace beam {
namespace half_ring {

constexpr int kFront = -(1 << 20);  // positions of the front loads: before all others

// first emulated prologue iteration: the one that issues A stage 0 or, if
// earlier, B sub-step 0
BEAM_HD constexpr int first_iter(int SA, int SB) {
  return (1 - 2 * SA) < -SB ? (1 - 2 * SA) : -SB;
}

// Position of B sub-step s / A stage q in the issue order: 2 j for iteration
// j's A load, 2 j + 1 for its B load, kFront + s for a front load.
BEAM_HD constexpr int pos_b(int SB, int KP, int s) { return s < KP ? kFront + s : 2 * (s - SB) + 1; }
BEAM_HD constexpr int pos_a(int SA, int q) { return 2 * (2 * (q - SA) + 1); }

// Loads issued after the youngest load that sub-step s needs (B sub-step s
// and, for even s, A stage s / 2), once model iterations up to `last` have
// issued: last_of(s, L) (s - 2 - L for the wait in iteration s - 1, -1 - L for
// sub-step 0, after the prologue).
BEAM_HD constexpr int last_of(int s, int L) { return (s == 0 ? -1 : s - 2) - L; }
BEAM_HD constexpr int younger(int SA, int SB, int KP, int nbl, int na2, int nk, int s, int last) {
  const int nst = nk / 2;
  int target = pos_b(SB, KP, s);
  if (s % 2 == 0) {
    const int pa = pos_a(SA, s / 2);
    target = pa > target ? pa : target;
  }
  int n = 0;
  const int nfront = KP < nk ? KP : nk;
  for (int i = 0; i < nfront; ++i)
    if (kFront + i > target) n += nbl;
  for (int j = first_iter(SA, SB); j <= last; ++j) {
    if (j % 2 != 0) {  // odd (also for negative j)
      const int qa = (j - 1) / 2 + SA;
      if (qa >= 0 && qa < nst && 2 * j > target) n += na2;
    }
    const int sb = j + SB;
    if (sb >= KP && sb < nk && 2 * j + 1 > target) n += nbl;
  }
  return n;
}

// younger() in closed form (what the kernel evaluates): the B loads after
// the target are those of a range of iterations, the A loads those of the odd
// iterations in a range, the front loads a range of indices.
BEAM_HD constexpr int count_in(int lo, int hi) { return hi >= lo ? hi - lo + 1 : 0; }
BEAM_HD constexpr int odd_upto(int x) { return (x + 1) >> 1; }  // odd integers in [0, x], or minus those in [x + 1, -1]
BEAM_HD constexpr int imax(int a, int b) { return a > b ? a : b; }
BEAM_HD constexpr int imin(int a, int b) { return a < b ? a : b; }
BEAM_HD constexpr int younger_fast(int SA, int SB, int KP, int nbl, int na2, int nk, int s, int last) {
  const int nst = nk >> 1;
  const int pb = s < KP ? kFront + s : 2 * (s - SB) + 1;
  const int target = (s & 1) == 0 ? imax(pb, 2 * (2 * ((s >> 1) - SA) + 1)) : pb;
  const int first = first_iter(SA, SB);
  const int nb = count_in(imax(imax(first, KP - SB), ((target - 1) >> 1) + 1), imin(last, nk - 1 - SB));
  const int alo = imax(imax(first, 1 - 2 * SA), (target >> 1) + 1);
  const int ahi = imin(last, 2 * (nst - SA) - 1);
  const int na = ahi >= alo ? odd_upto(ahi) - odd_upto(alo - 1) : 0;
  const int nf = count_in(imax(0, target - kFront + 1), imin(KP, nk) - 1);
  return nbl * (nb + nf) + na2 * na;
}

// The counts far from both ends of the k loop (a deep k loop), for odd and
// even s.
constexpr int kDeep = 1 << 12;
BEAM_HD constexpr int steady(int SA, int SB, int KP, int L, int nbl, int na2, int parity) {
  return younger(SA, SB, KP, nbl, na2, kDeep, 200 + parity, last_of(200 + parity, L));
}

// Smallest s0 from which every sub-step s >= s0 of a deep loop waits with the
// steady count of its parity (checked up to s0 + 24; the schedule repeats
// every two sub-steps once the prologue is behind).
BEAM_HD constexpr int steady_from(int SA, int SB, int KP, int L, int nbl, int na2) {
  const int st[2] = {steady(SA, SB, KP, L, nbl, na2, 0), steady(SA, SB, KP, L, nbl, na2, 1)};
  for (int s0 = 1; s0 < 64; ++s0) {
    bool ok = true;
    for (int s = s0; s < s0 + 24 && ok; ++s)
      ok = younger(SA, SB, KP, nbl, na2, kDeep, s, last_of(s, L)) == st[s & 1];
    if (ok) return s0;
  }
  return 1 << 30;
}

// Smallest T such that every sub-step s >= steady_from with s + T < nk waits
// with the steady count, for every even nk up to 48 (past the head, the count
// depends on nk - s only).
BEAM_HD constexpr int steady_tail(int SA, int SB, int KP, int L, int nbl, int na2) {
  const int s0 = steady_from(SA, SB, KP, L, nbl, na2);
  const int st[2] = {steady(SA, SB, KP, L, nbl, na2, 0), steady(SA, SB, KP, L, nbl, na2, 1)};
  for (int T = 0; T < 64; ++T) {
    bool ok = true;
    for (int nk = 2; nk <= 48 && ok; nk += 2)
      for (int s = s0; s + T < nk && ok; ++s)
        ok = younger(SA, SB, KP, nbl, na2, nk, s, last_of(s, L)) == st[s & 1];
    if (ok) return T;
  }
  return 1 << 30;
}

// The counts the kernel waits with (never more than younger(), i.e. never
// less waiting): loops shorter than deep_min() drain all loads (a rare,
// small K); otherwise a sub-step s >= 1 with s + steady_tail() < nk takes the
// steady count of its parity (for schedules with head_ok(): after the
// prologue the count never drops below it), and the last ones tail_count(),
// the count of a deep loop at the same distance d = nk - s from its end.
// Where a wave may hold either of two A load counts, the kernel takes the
// larger steady_tail() and deep_min() of the two.
BEAM_HD constexpr int tail_count(int SA, int SB, int KP, int L, int nbl, int na2, int d) {
  return younger(SA, SB, KP, nbl, na2, kDeep, kDeep - d, last_of(kDeep - d, L));
}
BEAM_HD constexpr int deep_min(int SA, int SB, int KP, int L, int nbl, int na2) {
  // past the prologue's loads and long enough for the tail pattern
  return 2 * (SB + 2 * SA + KP + L + steady_tail(SA, SB, KP, L, nbl, na2) + 4);
}
// Whether the steady counts are safe at the head of a deep loop (from
// sub-step 1 on), and the schedule issues every load before its wait; the
// kernel only runs schedules for which both hold.
BEAM_HD constexpr bool head_ok(int SA, int SB, int KP, int L, int nbl, int na2) {
  if (SB < L + 2 || 2 * SA < L + 3) return false;  // B(s) / A(s/2) issued by the wait for s
  const int s0 = steady_from(SA, SB, KP, L, nbl, na2);
  for (int s = 1; s < s0; ++s)
    if (younger(SA, SB, KP, nbl, na2, kDeep, s, last_of(s, L)) < steady(SA, SB, KP, L, nbl, na2, s & 1))
      return false;
  return true;
}

// Largest count of any wait (loops of up to 48 sub-steps; deeper ones repeat
// the counts of their last 48).
BEAM_HD constexpr int max_count(int SA, int SB, int KP, int L, int nbl, int na2) {
  int m = 0;
  for (int nk = 2; nk <= 48; nk += 2)
    for (int s = 0; s < nk; ++s) {
      const int c = younger(SA, SB, KP, nbl, na2, nk, s, last_of(s, L));
      m = c > m ? c : m;
    }
  return m;
}

// The above for one (SA, SB, KP, L, nbl, na2), evaluated once per distinct set.
template <int SA, int SB, int KP, int L, int NBL, int NA2>
struct Steady {
  static constexpr bool ok = head_ok(SA, SB, KP, L, NBL, NA2);
  static constexpr int deep = deep_min(SA, SB, KP, L, NBL, NA2);
  static constexpr int max = max_count(SA, SB, KP, L, NBL, NA2);
  static constexpr int from = steady_from(SA, SB, KP, L, NBL, NA2);
  static constexpr int tail = steady_tail(SA, SB, KP, L, NBL, NA2);
  static constexpr int odd = steady(SA, SB, KP, L, NBL, NA2, 1);
  static constexpr int even = steady(SA, SB, KP, L, NBL, NA2, 0);
};

}  // namespace half_ring
}  // namespace beam
