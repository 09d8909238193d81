"""Pins of the oracle's E4M3 encoding and double quantization (P4 §二 / §三:
the fp32 block constants are quantized to an 8-bit float with a second-level
block of 256; the e4m3, mean-centred reading is documented in
``oracle.nf4.double_quant``).  CPU only."""

import math
from fractions import Fraction

import numpy as np

from oracle import nf4, footprint
from tests._exact import to_f32


# ---------------------------------------------------------------------------
# E4M3 format facts (OCP FP8 E4M3: bias 7, 3 mantissa bits)
# ---------------------------------------------------------------------------

def test_e4m3_decode_format_facts():
    d = nf4.e4m3_decode_scalar
    assert d(0x00) == 0.0 and math.copysign(1, d(0x80)) == -1.0
    assert d(0x01) == 2.0 ** -9
    assert d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6
    assert d(0x38) == 1.0
    assert d(0x40) == 2.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    t = nf4.e4m3_table()
    pos = t[:0x7F].astype(np.float64)
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def brute_e4m3(y: float) -> int:
    """Nearest finite E4M3 by exhaustive rational comparison; ties to the even
    code (even mantissa); |y| >= 448 saturates; the sign bit follows y."""
    a = abs(Fraction(float(y)))
    best, best_d = None, None
    for code in range(0x7F):
        v = Fraction(nf4.e4m3_decode_scalar(code))
        dd = abs(a - v)
        if best_d is None or dd < best_d or (dd == best_d and code % 2 == 0):
            best, best_d = code, dd
    if a >= 448:
        best = 0x7E
    if math.copysign(1.0, float(y)) < 0:
        best |= 0x80
    return best


def sweep_points():
    pts = []
    for e in range(-12, 10):
        for k in range(0, 256):  # 8 sub-mantissa bits per binade: all midpoints
            v = np.float32((1 + k / 256) * 2.0 ** e)
            pts += [v, np.nextafter(v, np.float32(1e9)), np.nextafter(v, np.float32(0))]
    pts += [np.float32(v) for v in (0.0, 448.0, 464.0, 479.9, 480.0, 1e6, 2.0 ** -10,
                                    3 * 2.0 ** -11, 2.0 ** -11, 1e-30, 1e-45)]
    a = np.array(pts, dtype=np.float32)
    return np.concatenate([a, -a])


def test_e4m3_encode_vs_brute_force_sweep():
    y = sweep_points()
    got = nf4.e4m3_encode(y)
    ys = list(y)
    for i in range(0, len(ys), 3):  # every midpoint, and its down neighbour
        assert int(got[i]) == brute_e4m3(ys[i]), float(ys[i])
    for i in range(2, len(ys), 9):
        assert int(got[i]) == brute_e4m3(ys[i]), float(ys[i])


def test_e4m3_saturation_and_signed_zero():
    enc = nf4.e4m3_encode
    y = np.array([448, 464, 1e6, -1e6, -0.0, -1e-30, 1e-30, 2.0 ** -10, 3 * 2.0 ** -10],
                 dtype=np.float32)
    # 2^-10 is the midpoint of 0 and 2^-9: tie to even -> 0x00;
    # 3*2^-10 is the midpoint of 2^-9 (0x01) and 2^-8 (0x02): tie to even -> 0x02
    assert enc(y).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x00, 0x02]


# ---------------------------------------------------------------------------
# mean, group scales, codes
# ---------------------------------------------------------------------------

def test_tree_sum_order():
    # adjacent pairs level by level: (1 + 2^53) + (1 - 2^53) = 2^53 - (2^53 - 1) = 1
    # (a left-to-right sum gives 0, the exact sum is 2)
    assert nf4.tree_sum_f64(np.array([1.0, 2.0 ** 53, 1.0, -(2.0 ** 53)])) == 1.0
    # odd length, zero padded: ((2^53 + 1) + (1 + 0)); 2^53 + 1 is a tie that
    # rounds to the even 2^53, and so does the final 2^53 + 1
    assert nf4.tree_sum_f64(np.array([2.0 ** 53, 1.0, 1.0])) == 2.0 ** 53
    # (1 + 1) + (2^53 + 0) is exact
    assert nf4.tree_sum_f64(np.array([1.0, 1.0, 2.0 ** 53])) == 2.0 ** 53 + 2.0
    assert nf4.tree_sum_f64(np.array([3.5])) == 3.5


def exact_mean_f32(c):
    s = sum(Fraction(float(v)) for v in c)
    return to_f32(s / len(c))


def test_mean_matches_exact_mean():
    rng = np.random.default_rng(21)
    for n in (1, 3, 256, 1000, 4096):
        c = np.abs(rng.standard_normal(n) * 0.05).astype(np.float32)
        _, _, mu = nf4.double_quant(c)
        assert mu == exact_mean_f32(c)


def synthetic_constants(n=4096, seed=22):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n // 64, 64 * 64)) * 0.02).astype(np.float32)
    return nf4.block_absmax(w)


def test_group_extreme_encodes_to_448():
    c = synthetic_constants()
    e, s, mu = nf4.double_quant(c)
    d = (c - mu).astype(np.float32)
    for g in range(s.shape[0]):
        dg = d[256 * g:256 * g + 256]
        i = int(np.argmax(np.abs(dg)))
        assert e[256 * g + i] in (0x7E, 0xFE)
        assert s[g] == to_f32(Fraction(float(np.abs(dg[i]))) / 448)


def test_reconstruction_error_invariant():
    c = synthetic_constants(seed=23)
    e, s, mu = nf4.double_quant(c)
    d = (c - mu).astype(np.float64)
    g = np.arange(c.shape[0]) // 256
    rec = nf4.e4m3_table()[e].astype(np.float64) * s[g]
    bound = np.maximum(2.0 ** -4 * np.abs(d), 2.0 ** -10 * s[g]) * (1 + 2.0 ** -20) + 1e-30
    assert np.all(np.abs(rec - d) <= bound)


def test_zero_scale_group():
    c = np.full(512, 0.25, dtype=np.float32)
    c[256:] = 0.5
    e, s, mu = nf4.double_quant(c)
    # mean 0.375: d = ±0.125 in both groups -> codes ±448 (not zero-scale)
    assert mu == np.float32(0.375)
    assert set(e[:256].tolist()) == {0xFE} and set(e[256:].tolist()) == {0x7E}
    c2 = np.full(300, 0.125, dtype=np.float32)
    e2, s2, mu2 = nf4.double_quant(c2)
    assert mu2 == np.float32(0.125) and np.all(s2 == 0) and np.all(e2 == 0)
    assert np.all(nf4.decode_constants(e2, s2, mu2) == np.float32(0.125))


def test_decode_two_roundings_by_hand():
    # c' = fl32(fl32(dec(e) * s) + mu)
    e = np.array([0x38, 0xB8, 0x01], np.uint8)  # 1.0, -1.0, 2^-9
    s = np.array([np.float32(0.1)], np.float32)
    mu = np.float32(0.3)
    got = nf4.decode_constants(e, s, mu)
    for k, dv in enumerate([1.0, -1.0, 2.0 ** -9]):
        prod = to_f32(Fraction(dv) * Fraction(float(s[0])))
        ref = to_f32(Fraction(float(prod)) + Fraction(float(mu)))
        assert got[k] == ref


def test_footprint_from_sizes():
    # bits per parameter of the four arrays: 4 + 8/64 + 32/(64*256) + 32/(N*K)
    for n, k in ((4096, 4096), (11008, 4096), (8192, 22016)):
        nb = n * k // 64
        assert nb % 256 == 0
        expect = 4 + 8 / 64 + 32 / (64 * 256) + 32 / (n * k)
        assert abs(footprint.bits_per_param(n, k) - expect) < 1e-12
