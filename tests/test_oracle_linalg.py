"""Pins of the fp64 forward / backward references (P1 §七 dataflow figure;
P3 公式导读 3 wide + narrow path; P1 简化版 and P2 §4.4: gradients flow through
the dequantized frozen weight into LoRA only).  CPU only."""

import numpy as np

from oracle import linalg


def tiny(seed=41, M=5, K=64, N=7, r=3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.02
    A = rng.standard_normal((r, K)) * 0.02
    B = rng.standard_normal((N, r)) * 0.01
    dY = rng.standard_normal((M, N))
    return X, W, A, B, dY


def test_forward_against_fsum_triple_loop():
    X, W, A, B, _ = tiny()
    alpha, r = 6.0, 3
    Y, T = linalg.linear_fwd(X, W, A, B, alpha, r)
    T_ref = linalg.matmul_fsum(X, A.T)
    Y_ref = linalg.matmul_fsum(X, W.T) + (alpha / r) * linalg.matmul_fsum(T_ref, B.T)
    assert np.allclose(T, T_ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(Y, Y_ref, rtol=1e-13, atol=1e-15)


def loss(X, W, A, B, dY, alpha, r):
    Y, _ = linalg.linear_fwd(X, W, A, B, alpha, r)
    return float(np.sum(Y * dY))


def test_backward_by_central_differences():
    # L = <Y, dY> is linear in each of X, A, B separately, so the central
    # difference along any direction equals the directional derivative up to
    # rounding.
    X, W, A, B, dY = tiny(seed=42)
    alpha, r = 6.0, 3
    dX, dA, dB = linalg.linear_bwd(X, dY, W, A, B, alpha, r)
    rng = np.random.default_rng(43)
    h = 1e-3
    for name, grad in (("X", dX), ("A", dA), ("B", dB)):
        args = {"X": X, "A": A, "B": B}
        V = rng.standard_normal(args[name].shape)
        plus = dict(args)
        minus = dict(args)
        plus[name] = args[name] + h * V
        minus[name] = args[name] - h * V
        fd = (loss(plus["X"], W, plus["A"], plus["B"], dY, alpha, r)
              - loss(minus["X"], W, minus["A"], minus["B"], dY, alpha, r)) / (2 * h)
        an = float(np.sum(grad * V))
        assert abs(fd - an) <= 1e-9 * max(1.0, abs(an)), name


def test_special_cases():
    X, W, A, B, dY = tiny(seed=44)
    r = 3
    Y0, _ = linalg.linear_fwd(X, W, A, np.zeros_like(B), 6.0, r)
    assert np.array_equal(Y0, X @ W.T)
    Ya, _ = linalg.linear_fwd(X, W, A, B, 0.0, r)
    assert np.array_equal(Ya, X @ W.T)
    # linear in alpha
    Y1, _ = linalg.linear_fwd(X, W, A, B, 1.0, r)
    Y3, _ = linalg.linear_fwd(X, W, A, B, 3.0, r)
    assert np.allclose(Y3 - Ya, 3 * (Y1 - Ya), rtol=1e-12, atol=1e-14)
    dX, dA, dB = linalg.linear_bwd(X, dY, W, A, np.zeros_like(B), 6.0, r)
    assert np.all(dA == 0) and np.array_equal(dX, dY @ W)
    _, _, dB0 = linalg.linear_bwd(X, dY, W, np.zeros_like(A), B, 6.0, r)
    assert np.all(dB0 == 0)


def test_identity_input_returns_weight():
    _, W, A, B, _ = tiny(seed=45, K=64, N=64)
    X = np.eye(64)
    Y, _ = linalg.linear_fwd(X, W, A, np.zeros_like(B), 2.0, 3)
    assert np.array_equal(Y, W.T)
    dX, _, _ = linalg.linear_bwd(np.ones((64, 64)), np.eye(64), W, A, np.zeros_like(B), 2.0, 3)
    assert np.array_equal(dX, W)


def test_rel_fro():
    a = np.array([3.0, 4.0])
    assert linalg.rel_fro(a, a) == 0.0
    assert abs(linalg.rel_fro(a * 1.001, a) - 1e-3) < 1e-12
