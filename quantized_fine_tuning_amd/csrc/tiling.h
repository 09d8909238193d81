// Workgroup -> output-tile mapping for the large GEMMs on MI355X.
//
// The hardware deals consecutive workgroup ids round-robin to the 8 XCDs, each
// with its own L2.  tile_of() gives XCD x (= id % 8) a contiguous run of a
// grouped tile order (GM M-tiles per group), so the ~32 workgroups resident
// on one XCD at a time cover a compact block of tiles (GM M-tiles by 32 / GM
// N-tiles) and share their operand rows in that XCD's L2.  The block that
// an XCD's L2 fills per reduction step is GM·a + (32 / GM)·b for a bytes of
// activation per M-tile and b bytes of codes per N-tile: with 256 x 256
// tiles (a = 32 KB, b = 8 KB) GM = 4 (192 KB), with the forward's 512 x 128
// tiles (a = 64 KB, b = 4 KB) GM = 2 (192 KB where GM = 4 fills 288 KB;
// measured 1.3 % faster).
//
// When the output has too few tiles to occupy the chip (few tokens), the
// reduction is split: unit u = (split, tile), split-major, each unit one
// workgroup that reduces over its own range of steps and writes an fp32
// partial tile; a second kernel sums the partials in split order.
#pragma once

#include <hip/hip_runtime.h>

namespace qnf4 {

constexpr int kXcds = 8;
constexpr int kGroupM = 4;

constexpr int kGemmCus = 256;  // one GEMM workgroup per compute unit

inline unsigned tile_grid(int tiles_m, int tiles_n, int splits = 1) {
  const int T = tiles_m * tiles_n * splits;
  return (unsigned)(kXcds * ((T + kXcds - 1) / kXcds));
}

// Number of reduction splits for a GEMM of `tiles` output tiles and `steps`
// reduction steps: 1 while the tiles fill at least 3/4 of the compute units,
// else as many as fit one round of workgroups, with at least 8 steps each,
// fewer while the fp32 partials (splits x rows x cols x 4 bytes) exceed
// `cap` bytes.
inline int gemm_splits(int64_t tiles, int64_t steps, int64_t rows, int64_t cols, size_t cap) {
  if (tiles <= 0 || 4 * tiles >= 3 * kGemmCus) return 1;
  int64_t s = kGemmCus / tiles;
  s = s < steps / 8 ? s : steps / 8;
  while (s > 1 && (size_t)s * (size_t)rows * (size_t)cols * 4u > cap) --s;
  return s > 1 ? (int)s : 1;
}

// Steps [first, last) of split `sp` out of `splits` over `steps` steps.
__host__ __device__ inline int split_first(int sp, int splits, int steps) {
  return (int)(((int64_t)sp * steps) / splits);
}

// Returns false for the padding workgroups beyond the last unit.
template <int GM = kGroupM>
__device__ __forceinline__ bool tile_of(int bid, int tiles_m, int tiles_n, int splits, int& tm, int& tn,
                                        int& sp) {
  const int T = tiles_m * tiles_n;
  const int U = T * splits;
  const int per = (U + kXcds - 1) / kXcds;
  const int u = (bid % kXcds) * per + bid / kXcds;
  if (u >= U) return false;
  sp = u / T;
  const int t = u - sp * T;
  const int group = t / (GM * tiles_n);
  const int first = group * GM;
  const int gm = min(GM, tiles_m - first);
  const int in = t - group * GM * tiles_n;
  tm = first + in % gm;
  tn = in / gm;
  return true;
}

}  // namespace qnf4
