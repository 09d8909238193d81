// Workgroup -> output-tile mapping for the large GEMMs on MI355X.
//
// The hardware deals consecutive workgroup ids round-robin to the 8 XCDs, each
// with its own L2.  tile_of() gives XCD x (= id % 8) a contiguous run of a
// grouped tile order, so the ~32 workgroups resident on one XCD at a time
// cover a compact block of tiles (4 M-tiles by ~8 N-tiles) and share their
// operand rows in that XCD's L2.
#pragma once

#include <hip/hip_runtime.h>

namespace qnf4 {

constexpr int kXcds = 8;
constexpr int kGroupM = 4;

inline unsigned tile_grid(int tiles_m, int tiles_n) {
  const int T = tiles_m * tiles_n;
  return (unsigned)(kXcds * ((T + kXcds - 1) / kXcds));
}

// Returns false for the padding workgroups beyond the last tile.
__device__ __forceinline__ bool tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int per = (T + kXcds - 1) / kXcds;
  const int t = (bid % kXcds) * per + bid / kXcds;
  if (t >= T) return false;
  const int group = t / (kGroupM * tiles_n);
  const int first = group * kGroupM;
  const int gm = min(kGroupM, tiles_m - first);
  const int in = t - group * kGroupM * tiles_n;
  tm = first + in % gm;
  tn = in / gm;
  return true;
}

}  // namespace qnf4
