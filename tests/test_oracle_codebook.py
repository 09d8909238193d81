"""Pins of the oracle's NF4 codebook and nearest-code search (CPU only).

The codebook follows P4 §三 (levels at standard-normal quantiles, equal
probability mass per level, exact zero) under the reading documented in
``oracle.nf4.codebook_f64``.  The pins check it against the normal CDF taken
from ``math.erfc`` (independent of the inverse used by the oracle) and the
structural facts the pages fix; the nearest-code search is checked against an
exact rational brute force.
"""

import math
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4
from tests._exact import f32_bits


def phi(x: float) -> float:
    """Standard normal CDF from the complementary error function."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def phi_inv_bisect(p: float) -> float:
    lo, hi = -12.0, 12.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_structure_pages_fix():
    # north star / P4 §三: 16 sorted values in [-1, 1] that include 0
    q = nf4.codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    assert q[0] == -1.0 and q[15] == 1.0 and q[7] == 0.0
    assert np.all(np.abs(q) <= 1.0)
    assert int(np.sum(q < 0)) == 7 and int(np.sum(q > 0)) == 8


def test_quantiles_against_erfc():
    # each non-zero level times z = Φ⁻¹(31/32) sits at an evenly spaced
    # probability on its side; Φ comes from math.erfc, not from the inverse.
    q = nf4.codebook_f64()
    z = phi_inv_bisect(31 / 32)
    assert abs(z - nf4._normal_quantile(31 / 32)) < 1e-12
    step = 31 / 32 - 0.5
    for j in range(1, 9):
        assert abs(phi(q[7 + j] * z) - (0.5 + j * step / 8)) < 1e-12
    for j in range(1, 8):
        assert abs(phi(-q[7 - j] * z) - (0.5 + j * step / 7)) < 1e-12


def test_equal_probability_mass_per_side():
    # P4 §三 中文: every level covers the same probability mass
    q = nf4.codebook_f64()
    z = phi_inv_bisect(31 / 32)
    cdf = [phi(v * z) for v in q]
    pos = np.diff(cdf[7:])
    neg = np.diff(cdf[:8])
    assert np.allclose(pos, pos[0], atol=1e-12, rtol=0)
    assert np.allclose(neg, neg[0], atol=1e-12, rtol=0)
    assert abs(pos.sum() - (31 / 32 - 0.5)) < 1e-12


def test_fp32_rounding_of_levels():
    # every fp32 level is the nearest fp32 of its fp64 value
    q64 = nf4.codebook_f64()
    q32 = nf4.codebook()
    for a, b in zip(q64, q32):
        b = float(b)
        up = float(np.nextafter(np.float32(b), np.float32(2)))
        dn = float(np.nextafter(np.float32(b), np.float32(-2)))
        assert abs(a - b) <= abs(a - up) and abs(a - b) <= abs(a - dn)


# An independent computation of the same reading (fp32 bit patterns of the
# levels and of the round-down midpoints), made separately from this oracle.
# It is a regression cross-check, not a value printed on the pages.
INDEPENDENT_LEVEL_BITS = [
    0xbf800000, 0xbf3188d6, 0xbf05c6b0, 0xbec92605, 0xbe90d881, 0xbe3c28e3,
    0xbdb96cbb, 0x00000000, 0x3da210d6, 0x3e23e03b, 0x3e7aa402, 0x3eac17c0,
    0x3ee08015, 0x3f0f5d29, 0x3f38654d, 0x3f800000]
INDEPENDENT_THRESHOLD_BITS = [
    0xbf58c46b, 0xbf1ba7c3, 0xbeea59b3, 0xbeacff43, 0xbe6eecf3, 0xbe0c6fa1,
    0xbd396cbb, 0x3d2210d6, 0x3df4e8a6, 0x3e4f421e, 0x3e94b4e0, 0x3ec64bea,
    0x3eff9d33, 0x3f23e13b, 0x3f5c32a6]


def test_levels_match_independent_computation():
    q = nf4.codebook()
    assert [f32_bits(v) for v in q] == INDEPENDENT_LEVEL_BITS
    t = nf4.thresholds(q)
    assert [f32_bits(v) for v in t] == INDEPENDENT_THRESHOLD_BITS


def test_golden_codebook_file():
    from tests.golden import make_codebook
    assert make_codebook.read_table() == make_codebook.table_lines()


# ---------------------------------------------------------------------------
# nearest code
# ---------------------------------------------------------------------------

def brute_nearest(x: float, q) -> int:
    """Exact argmin over all 16 levels with rationals; first minimiser."""
    xf = Fraction(float(x))
    best, best_d = None, None
    for j, v in enumerate(q):
        d = abs(xf - Fraction(float(v)))
        if best_d is None or d < best_d:
            best, best_d = j, d
    return best


def crafted_points(q):
    """Every midpoint (when representable), its fp32 neighbours, the
    round-down thresholds and their neighbours, the levels themselves."""
    pts = []
    m = nf4.midpoints(q)
    t = nf4.thresholds(q)
    for mj, tj in zip(m, t):
        for base in (np.float32(mj), tj):
            pts.append(base)
            pts.append(np.nextafter(base, np.float32(2)))
            pts.append(np.nextafter(base, np.float32(-2)))
    pts.extend(list(q))
    pts.extend([np.float32(-0.0), np.float32(1e-45), np.float32(-1e-45)])
    return np.array(pts, dtype=np.float32)


def test_nearest_code_brute_force_crafted():
    q = nf4.codebook()
    x = crafted_points(q)
    got = nf4.nearest_code(x, q)
    for xi, gi in zip(x, got):
        assert int(gi) == brute_nearest(xi, q), float(xi)


def test_ties_reachable_and_go_low():
    # 7 of the 15 midpoints are exactly representable in fp32: those are ties,
    # which go to the lower index.
    q = nf4.codebook()
    m = nf4.midpoints(q)
    exact = [j for j, mj in enumerate(m) if float(np.float32(mj)) == mj]
    assert len(exact) == 7
    for j in exact:
        assert int(nf4.nearest_code(np.array([m[j]], np.float32), q)[0]) == j


def test_nearest_code_brute_force_random():
    rng = random.Random(7)
    q = nf4.codebook()
    x = np.array([rng.uniform(-1, 1) for _ in range(3000)], dtype=np.float32)
    got = nf4.nearest_code(x, q)
    for xi, gi in zip(x, got):
        assert int(gi) == brute_nearest(xi, q)


def test_threshold_formulation_agrees():
    q = nf4.codebook()
    t = nf4.thresholds(q)
    rng = np.random.default_rng(3)
    x = np.concatenate([crafted_points(q), rng.uniform(-1, 1, 20000).astype(np.float32)])
    by_count = np.sum(x[:, None] > t[None, :], axis=1)
    assert np.array_equal(by_count, nf4.nearest_code(x, q))


def test_code_monotone_in_x():
    q = nf4.codebook()
    x = np.sort(np.random.default_rng(5).uniform(-1, 1, 50000).astype(np.float32))
    c = nf4.nearest_code(x, q).astype(int)
    assert np.all(np.diff(c) >= 0)
    assert nf4.nearest_code(np.array([-1.0, 1.0], np.float32), q).tolist() == [0, 15]
