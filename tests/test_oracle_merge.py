"""Pins of the oracle's LoRA merge (oracle/merge.py) on the CPU: B = 0 gives
the dequantized weight back, the merged weight carries the forward pass's
function, the single roundings against hand-worked values, and re-quantizing
the dequantized weight returns its codes."""

import numpy as np
import pytest

from oracle import linalg, merge, nf4

F32 = np.float32


def small_layer(seed, N=48, K=128, r=8):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    q = nf4.quantize(W)
    W_hat = nf4.dequantize(q["codes"], q["absmax_e4m3"], q["dq_scale"], q["dq_mean"]).reshape(N, K)
    A = nf4.bf16_bits((rng.standard_normal((r, K)) * 0.02).astype(F32))
    B = nf4.bf16_bits((rng.standard_normal((N, r)) * 0.01).astype(F32))
    return q, W_hat, A, B


def test_zero_b_gives_the_dequantized_weight():
    q, W_hat, A, _ = small_layer(1)
    B0 = np.zeros((W_hat.shape[0], A.shape[0]), np.uint16)
    assert np.array_equal(merge.merge(W_hat, A, B0, 16.0, 8, "bf16"), W_hat)
    # bf16 values of this size are exact in fp16
    f16 = nf4.bf16_to_f32(W_hat).astype(np.float16).view(np.uint16)
    assert np.array_equal(merge.merge(W_hat, A, B0, 16.0, 8, "f16"), f16)


def test_merged_weight_carries_the_forward_function():
    # X·(Ŵ + s·B·A)ᵀ equals the forward oracle's X·Ŵᵀ + s·(X·Aᵀ)·Bᵀ: catches a
    # transposed or swapped product and a wrong or missing scale
    _, W_hat, A, B = small_layer(2)
    alpha, r = 16.0, 8
    X = nf4.bf16_bits(np.random.default_rng(3).standard_normal((5, W_hat.shape[1])).astype(F32))
    Xf = linalg.bf16_to_f64(X)
    Y_ref, _ = linalg.linear_fwd(Xf, linalg.bf16_to_f64(W_hat), linalg.bf16_to_f64(A),
                                 linalg.bf16_to_f64(B), alpha, r)
    Y = Xf @ merge.merged_exact(W_hat, A, B, alpha, r).T
    assert np.max(np.abs(Y - Y_ref)) <= 1e-12 * np.max(np.abs(Y_ref))


def test_scale_is_the_fp32_quotient():
    assert merge.lora_scale(16.0, 64) == 0.25
    assert merge.lora_scale(1.0, 3) == float(F32(1.0) / F32(3.0))
    assert merge.lora_scale(1.0, 3) != 1.0 / 3.0


@pytest.mark.parametrize("x, want", [
    (1.0 + 2.0 ** -8, 1.0),                            # tie, even neighbour below
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),            # tie, even neighbour above
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),   # just above the tie
    (-(1.0 + 2.0 ** -8 + 2.0 ** -30), -(1.0 + 2.0 ** -7)),
    (2.0 ** -133 * 10.5, 2.0 ** -133 * 10),           # subnormal spacing 2^-133, tie
    (2.0 ** -133 * 10.75, 2.0 ** -133 * 11),
    (2.0 ** -133 * 2.5, 2.0 ** -132),                  # subnormal tie to even
    (0.0, 0.0),
])
def test_bf16_single_rounding(x, want):
    got = nf4.bf16_to_f32(merge.round_bf16_bits(np.array([x])))[0]
    assert float(got) == want


def test_bf16_single_rounding_differs_from_rounding_through_fp32():
    # 1 + 2^-8 + 2^-30 rounds up once; through fp32 it first becomes the tie
    # 1 + 2^-8 and then rounds down to 1: why the device result is compared
    # within one unit in the last place
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert nf4.bf16_to_f32(merge.round_bf16_bits(x))[0] == 1.0 + 2.0 ** -7
    assert nf4.bf16_to_f32(nf4.bf16_bits(x.astype(F32)))[0] == 1.0


@pytest.mark.parametrize("x, want", [
    (1.0 + 2.0 ** -11, 1.0),
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),
    (1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 2.0 ** -10),
    (65504.0, 65504.0),
    (2.0 ** -24 * 0.75, 2.0 ** -24),                   # fp16 subnormal
])
def test_f16_single_rounding(x, want):
    got = merge.round_f16_bits(np.array([x])).view(np.float16)[0]
    assert float(got) == want


def test_requantizing_the_dequantized_weight_returns_its_codes():
    # Ŵ's block maximum is ±RNE_bf16(c'), so every ratio Ŵ/max stays within
    # 2^-7 (relative) of its level, far inside the level spacing (>= 0.079):
    # NF4 applied to its own output gives the same codes
    q, W_hat, _, _ = small_layer(4, N=64, K=256)
    rq = merge.requantize(W_hat)
    assert np.array_equal(rq["codes"], q["codes"])


def test_requantized_merge_error_is_of_the_nf4_size():
    # a merged weight re-quantized: the error relative to the merged weight is
    # that of NF4 on Gaussian-like data (about 0.1 of the Frobenius norm)
    _, W_hat, A, B = small_layer(5, N=64, K=256, r=16)
    Wm = merge.merge(W_hat, A, B, 32.0, 16, "bf16")
    rq = merge.requantize(Wm)
    back = nf4.dequantize(rq["codes"], rq["absmax_e4m3"], rq["dq_scale"], rq["dq_mean"])
    err = linalg.rel_fro(nf4.bf16_to_f32(back).reshape(Wm.shape), nf4.bf16_to_f32(Wm))
    assert 0.05 < err < 0.15
