"""Pins of the oracle's fp16 compute format (oracle/nf4.py: f16_bits and the
fp16 dequantization) on the CPU: hand-worked roundings, the block maximum,
and agreement with the bf16 dequantization of the same fp32 products."""

import numpy as np
import pytest

from oracle import linalg, nf4

F32 = np.float32


@pytest.mark.parametrize("x, want", [
    (1.0 + 2.0 ** -11, 1.0),                   # tie, even below
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),   # tie, even above
    (-(1.0 + 3 * 2.0 ** -11), -(1.0 + 2.0 ** -9)),
    (2.0 ** -24 * 0.75, 2.0 ** -24),           # subnormal spacing 2^-24
    (2.0 ** -24 * 0.5, 0.0),                   # tie to even (zero)
    (65504.0, 65504.0),
    (65519.0, 65504.0),
    (65520.0, float("inf")),                   # the tie past the largest value
])
def test_f16_rounding(x, want):
    assert float(nf4.f16_to_f32(nf4.f16_bits(np.array([x], F32)))[0]) == want


def fp16_and_bf16(seed, N=32, K=256):
    w = (np.random.default_rng(seed).standard_normal((N, K)) * 0.02).astype(F32)
    qz = nf4.quantize(w)
    args = (qz["codes"], qz["absmax_e4m3"], qz["dq_scale"], qz["dq_mean"])
    return qz, nf4.dequantize(*args, fmt16="f16"), nf4.dequantize(*args)


def test_block_maximum_dequantizes_to_the_rounded_constant():
    qz, h, _ = fp16_and_bf16(1)
    cp = nf4.decode_constants(qz["absmax_e4m3"], qz["dq_scale"], qz["dq_mean"])
    codes = nf4.unpack_nibbles(qz["codes"]).reshape(-1, 64)
    h = h.reshape(-1, 64)
    for b in range(codes.shape[0]):
        top = np.nonzero(codes[b] == 15)[0]
        if top.size:
            assert h[b, top[0]] == nf4.f16_bits(np.array([cp[b]], F32))[0]


def test_fp16_and_bf16_round_the_same_products():
    # both are one rounding of fl32(q·c'): for normal fp16 values, bf16 of the
    # fp16 value equals the bf16 value unless the fp16 value sits exactly
    # halfway between two bf16 values (a double-rounding tie: its 3 extra
    # bits are 100, about 1 value in 16); fp16 is within 2^-8 + 2^-11
    # (relative) of bf16
    _, h, b = fp16_and_bf16(2)
    hf = nf4.f16_to_f32(h).astype(np.float64)
    bf = nf4.bf16_to_f32(b).astype(np.float64)
    normal = np.abs(hf) >= 2.0 ** -14
    tie = (hf.astype(F32).view(np.uint32) & 0xFFFF) == 0x8000
    again = nf4.bf16_bits(hf.astype(F32))
    assert np.array_equal(again[normal & ~tie], b[normal & ~tie])
    assert 0.02 < np.mean(tie[normal]) < 0.2  # (the products take few distinct values per block)
    assert np.all(np.abs(hf - bf)[normal] <= (2.0 ** -8 + 2.0 ** -11) * np.abs(bf)[normal])
    assert linalg.rel_fro(hf, bf) < 2e-3
