// Order in which the grouped GEMM's persistent walk visits its work items.
// Plain C++ (no HIP types), so that a host program can check it.
#pragma once

#include <stdint.h>

#ifndef BEAM_HD
#if defined(__HIPCC__)
#define BEAM_HD __host__ __device__
#else
#define BEAM_HD
#endif
#endif

namespace beam {

// Item q -> (m-tile, n-tile).  Plain order: q = tile * nt_n + ntile, so the
// n-tiles of an m-tile are consecutive.  Blocked order (first != null): an
// expert's items (its M m-tiles x nt_n n-tiles, at the same positions as in
// the plain order) run n-group by n-group, each group of kGroupN n-tiles
// m-tile by m-tile, so 32 consecutive items of a hot expert are 8 m-tiles x
// 4 n-tiles: the weights of 4 n-tiles and the rows of 8 m-tiles instead of
// the weights of 32.
#ifndef BEAM_GROUP_N
#define BEAM_GROUP_N 4
#endif
constexpr int kGroupN = BEAM_GROUP_N;
BEAM_HD inline void item_of(int q, int nt_n, const int32_t* first, const int32_t* count, int& tile,
                            int& ntile) {
  const int t0 = q / nt_n;  // a tile of the same expert
  if (!first) {
    tile = t0;
    ntile = q - t0 * nt_n;
    return;
  }
  const int f = first[t0], M = count[t0];
  const int l = q - f * nt_n;  // item within the expert
  const int full = nt_n / kGroupN * kGroupN;
  int g0, gs, r;
  if (l < full * M) {
    const int g = l / (kGroupN * M);
    g0 = g * kGroupN;
    gs = kGroupN;
    r = l - g * kGroupN * M;
  } else {  // the last, partial group
    g0 = full;
    gs = nt_n - full;
    r = l - full * M;
  }
  const int m = r / gs;
  tile = f + m;
  ntile = g0 + (r - m * gs);
}

}  // namespace beam
