// Host-side construction of the NF4 levels and decision thresholds.
//
// P4 §三 (English derivation and Chinese text): the 16 levels sit at
// quantiles of the standard normal so that each level carries the same
// probability mass, an adjustment around zero keeps an exact zero, and the
// block maximum normalises to ±1.  Reading used (the literal midpoint formula
// on the page is infinite at both ends and has no zero): level 7 is 0; the 8
// positive levels are Φ⁻¹(1/2 + j·(p_end − 1/2)/8)/z for j = 1..8 and the 7
// negative levels −Φ⁻¹(1/2 + j·(p_end − 1/2)/7)/z for j = 1..7, with
// p_end = 31/32 and z = Φ⁻¹(p_end), so the ends are exactly ±1.
//
// Φ⁻¹ is found here by bisection on Φ(x) = erfc(−x/√2)/2 to full double
// precision; each level is then rounded to the nearest fp32.
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "host.h"

namespace qnf4 {
namespace {

double phi(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double phi_inv(double p) {
  double lo = -12.0, hi = 12.0;
  for (int i = 0; i < 400; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (phi(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

Codebook build() {
  Codebook cb;
  const double p_end = 31.0 / 32.0;
  const double step = p_end - 0.5;
  const double z = phi_inv(p_end);
  double q[16];
  q[7] = 0.0;
  for (int j = 1; j <= 8; ++j) q[7 + j] = phi_inv(0.5 + j * step / 8.0) / z;
  for (int j = 1; j <= 7; ++j) q[7 - j] = -phi_inv(0.5 + j * step / 7.0) / z;
  for (int i = 0; i < 16; ++i) cb.q[i] = (float)q[i];
  for (int j = 0; j < 15; ++j) {
    // exact in double: two fp32 values in [-1, 1]
    const double m = ((double)cb.q[j] + (double)cb.q[j + 1]) * 0.5;
    float t = (float)m;
    if ((double)t > m) t = std::nextafter(t, -INFINITY);
    cb.t[j] = t;
  }
  return cb;
}

// The quantize kernels find a code through a table of cells: |x| in
// [2^-5, 1] is cut into cells by its exponent and top 3 mantissa bits (bits
// 20..30 of the fp32 pattern), and each cell may hold at most one threshold
// (code = thresholds below the cell + (x > the one inside)); |x| < 2^-5 must
// hold none.  Returns false if the thresholds break that.
bool cells_hold_one_threshold(const Codebook& cb) {
  int count[2][512] = {};
  for (int j = 0; j < 15; ++j) {
    const float t = cb.t[j];
    if (!(std::fabs(t) > 0x1p-5f) || !(std::fabs(t) < 1.0f)) return false;
    uint32_t u;
    std::memcpy(&u, &t, 4);
    // cells are [lo, hi) for x >= 0 and (-hi, -lo] for x < 0: either way
    // the cell of t is given by the bits of |t|
    const uint32_t cell = (u & 0x7fffffffu) >> 20;
    if (++count[u >> 31][cell & 511] > 1) return false;
  }
  return true;
}

}  // namespace

const Codebook& codebook() {
  static Codebook cb;
  static std::once_flag once;
  std::call_once(once, [] {
    cb = build();
    if (!cells_hold_one_threshold(cb)) {
      std::fprintf(stderr, "qlora_nf4: NF4 thresholds break the quantizer's one-threshold-per-cell table\n");
      std::abort();
    }
  });
  return cb;
}

}  // namespace qnf4
