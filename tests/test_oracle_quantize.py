"""Pins of the oracle's blockwise absmax, normalisation, codes and packing
(P4 §三 English derivation: W^norm = W / max|W_block| with B = 64, then the
nearest level).  CPU only."""

from fractions import Fraction

import numpy as np

from oracle import nf4
from tests._exact import to_f32
from tests.test_oracle_codebook import brute_nearest


def test_absmax_is_exact_max_per_block():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    c = nf4.block_absmax(w)
    flat = w.reshape(-1)
    for b in range(c.shape[0]):
        assert c[b] == max(abs(float(v)) for v in flat[64 * b:64 * b + 64])


def test_division_is_correctly_rounded_fp32():
    # x = fl32(w / c): compare numpy's float32 division with exact rationals
    rng = np.random.default_rng(12)
    w = (rng.standard_normal(64 * 40) * 0.02).astype(np.float32).reshape(-1, 64)
    w[3] *= np.float32(1e-38)  # subnormal block
    c = nf4.block_absmax(w)
    x = np.divide(w, c[:, None])
    for b in range(w.shape[0]):
        for i in range(0, 64, 7):
            ref = to_f32(Fraction(float(w[b, i])) / Fraction(float(c[b])))
            assert x[b, i] == ref


def test_codes_equal_brute_force_of_exact_quotient():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal(64 * 12) * 0.02).astype(np.float32)
    w[5] *= 10  # an outlier
    codes, c = nf4.quantize_codes(w)
    q = nf4.codebook()
    for i in range(0, w.shape[0], 3):
        cb = c[i // 64]
        x = to_f32(Fraction(float(w[i])) / Fraction(float(cb)))
        assert int(codes[i]) == brute_nearest(x, q)


def test_crafted_block_with_unit_scale():
    # a block holding 1.0 has c = 1, so x = w exactly: midpoints and their
    # neighbours land on the exact tie rule
    q = nf4.codebook()
    m = nf4.midpoints(q)
    vals = [1.0]
    for mj in m:
        f = np.float32(mj)
        vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    vals = np.array(vals[:64] + [0.0] * (64 - len(vals[:64])), dtype=np.float32)
    codes, c = nf4.quantize_codes(vals)
    assert c[0] == 1.0
    for v, code in zip(vals, codes):
        assert int(code) == brute_nearest(v, q)


def test_zero_block_and_signed_zero():
    w = np.zeros(128, dtype=np.float32)
    w[64:] = -0.0
    codes, c = nf4.quantize_codes(w)
    assert np.all(codes == 7) and np.all(c == 0)


def test_block_max_maps_to_end_codes():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    codes, c = nf4.quantize_codes(w)
    codes = codes.reshape(16, 64)
    for b in range(16):
        i = int(np.argmax(np.abs(w[b])))
        assert codes[b, i] == (15 if w[b, i] > 0 else 0)


def test_pack_order_and_roundtrip():
    # element i -> byte i // 2, low nibble if i even, high nibble if odd
    assert nf4.pack_nibbles(np.array([1, 2, 3, 4], np.uint8)).tolist() == [0x21, 0x43]
    assert nf4.pack_nibbles(np.array([15, 0], np.uint8)).tolist() == [0x0F]
    rng = np.random.default_rng(15)
    c = rng.integers(0, 16, 4096).astype(np.uint8)
    p = nf4.pack_nibbles(c)
    assert p.shape == (2048,)
    assert np.array_equal(nf4.unpack_nibbles(p), c)


def test_quantize_codes_do_not_depend_on_double_quant():
    # the weights are normalised with the raw absmax, so codes depend on c only
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    out = nf4.quantize(w)
    codes, _ = nf4.quantize_codes(w)
    assert np.array_equal(out["codes"], nf4.pack_nibbles(codes))
