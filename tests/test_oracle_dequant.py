"""Pins of the oracle's bf16 rounding and dequantization (P1 §七: the 4-bit
weight is dequantized block by block to BF16 before the matmul; P4 §四 ①:
Ŵ = Dequant(W^NF4)·c).  CPU only."""

import math
from fractions import Fraction

import numpy as np

from oracle import nf4
from tests._exact import to_f32, to_bf16_value


def test_bf16_rounding_vs_exact():
    rng = np.random.default_rng(31)
    x = np.concatenate([
        (rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000)).astype(np.float32),
        # exact ties: bf16 value plus half an ulp
        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([1e-40, -1e-40, 0.0, -0.0], np.float32)])
    b = nf4.bf16_bits(x)
    for xi, bi in zip(x, b):
        v = nf4.bf16_to_f32(np.array([bi], np.uint16))[0]
        ref = to_bf16_value(Fraction(float(xi)))
        assert float(v) == ref, float(xi)
        assert math.copysign(1, float(v)) == math.copysign(1, float(xi))


def make_quantized(n=8, k=512, seed=32):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, 5, replace=False)] *= 10
    return w, nf4.quantize(w)


def test_dequant_chain_exact():
    w, qt = make_quantized()
    out = nf4.dequantize(qt["codes"], qt["absmax_e4m3"], qt["dq_scale"], qt["dq_mean"])
    q = nf4.codebook()
    codes = nf4.unpack_nibbles(qt["codes"])
    dec = nf4.e4m3_table()
    for i in range(0, codes.shape[0], 13):
        b = i // 64
        g = b // 256
        prod = to_f32(Fraction(float(dec[qt["absmax_e4m3"][b]])) * Fraction(float(qt["dq_scale"][g])))
        cp = to_f32(Fraction(float(prod)) + Fraction(float(qt["dq_mean"])))
        wv = to_f32(Fraction(float(q[codes[i]])) * Fraction(float(cp)))
        ref = to_bf16_value(Fraction(float(wv)))
        got = float(nf4.bf16_to_f32(out[i:i + 1])[0])
        assert got == ref


def test_block_max_and_zero_code():
    w, qt = make_quantized(seed=33)
    out = nf4.dequantize(qt["codes"], qt["absmax_e4m3"], qt["dq_scale"], qt["dq_mean"])
    vals = nf4.bf16_to_f32(out).reshape(-1, 64)
    cp = nf4.decode_constants(qt["absmax_e4m3"], qt["dq_scale"], qt["dq_mean"])
    wb = w.reshape(-1, 64)
    codes = nf4.unpack_nibbles(qt["codes"]).reshape(-1, 64)
    for b in range(wb.shape[0]):
        i = int(np.argmax(np.abs(wb[b])))
        sign = 1 if wb[b, i] > 0 else -1
        ref = nf4.bf16_to_f32(nf4.bf16_bits(np.array([sign * cp[b]], np.float32)))[0]
        assert vals[b, i] == ref
        z = codes[b] == 7
        assert np.all(vals[b][z] == 0)
        assert np.all(np.signbit(vals[b][z]) == np.signbit(cp[b]))


def test_negative_scale_gives_negative_zero():
    # code 7 (level +0) times a negative c' is -0 in IEEE arithmetic
    packed = np.array([0x77] * 32, np.uint8)
    e = np.array([0xFE], np.uint8)      # -448
    s = np.array([1.0], np.float32)
    mu = np.float32(0.0)
    out = nf4.dequantize(packed, e, s, mu)
    assert np.all(out == 0x8000)


def int4_absmax_error(w):
    wb = w.reshape(-1, 64).astype(np.float64)
    c = np.max(np.abs(wb), axis=1, keepdims=True)
    qv = np.round(wb / c * 7) / 7 * c
    return np.linalg.norm(qv - wb) / np.linalg.norm(wb)


def test_nf4_beats_uniform_int4_on_gaussian_weights():
    # P2 §4.1 and P4 §四 ②: on normally distributed weights NF4 keeps more
    # information than uniform 4-bit integers (lower reconstruction error).
    rng = np.random.default_rng(34)
    w = (rng.standard_normal((512, 1024)) * 0.02).astype(np.float32)
    qt = nf4.quantize(w)
    out = nf4.dequantize(qt["codes"], qt["absmax_e4m3"], qt["dq_scale"], qt["dq_mean"])
    wh = nf4.bf16_to_f32(out).astype(np.float64)
    err_nf4 = np.linalg.norm(wh - w.reshape(-1)) / np.linalg.norm(w)
    err_int4 = int4_absmax_error(w)
    assert 0.09 < err_nf4 < 0.12
    assert err_nf4 < err_int4
