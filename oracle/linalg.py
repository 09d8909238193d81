"""fp64 references of the QLoRA linear layer.  Oracle (test infrastructure
only; see ``oracle/__init__``).

Shapes: X [M, K], W and Ŵ [N, K] (out_features x in_features, row-major),
A [r, K], B [N, r], Y and dY [M, N], s = alpha / r.

P1 §七 (dataflow figure): the frozen 4-bit weight is dequantized to BF16 and
multiplied with the BF16 activation; the trainable LoRA path is added to the
output.  P3 公式导读 3: the input goes through a wide (frozen backbone) path and
a narrow (LoRA) path and the two are summed.  P1 简化版 / P2 §4.4: the gradient
passes through the dequantized frozen weight into the LoRA parameters only; the
4-bit codes receive no update (there is no dW here at all).
"""

from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(b16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.asarray(b16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def linear_fwd(X, W_hat, A, B, alpha: float, r: int):
    """Y = X·Ŵᵀ + (α/r)·(X·Aᵀ)·Bᵀ in fp64.  Returns (Y, T) with T = X·Aᵀ."""
    X = np.asarray(X, dtype=np.float64)
    W_hat = np.asarray(W_hat, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = float(alpha) / float(r)
    T = X @ A.T
    Y = X @ W_hat.T + s * (T @ B.T)
    return Y, T


def linear_bwd(X, dY, W_hat, A, B, alpha: float, r: int):
    """Gradients of L = <Y, dY> for the layer above, in fp64.

    U = dY·B;  dX = dY·Ŵ + s·U·A;  dA = s·Uᵀ·X;  dB = s·dYᵀ·(X·Aᵀ).
    Returns (dX, dA, dB).  T is recomputed here, never taken from elsewhere.
    """
    dX = linear_dx(dY, W_hat, A, B, alpha, r)
    dA, dB = lora_grads(X, dY, A, B, alpha, r)
    return dX, dA, dB


def linear_dx(dY, W_hat, A, B, alpha: float, r: int):
    """dX = dY·Ŵ + s·(dY·B)·A in fp64.  Columns of dX depend only on the same
    columns of Ŵ and A."""
    dY = np.asarray(dY, dtype=np.float64)
    W_hat = np.asarray(W_hat, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = float(alpha) / float(r)
    return dY @ W_hat + s * ((dY @ B) @ A)


def lora_grads(X, dY, A, B, alpha: float, r: int):
    """dA = s·(dY·B)ᵀ·X and dB = s·dYᵀ·(X·Aᵀ) in fp64 (they do not involve Ŵ)."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = float(alpha) / float(r)
    U = dY @ B
    T = X @ A.T
    return s * (U.T @ X), s * (dY.T @ T)


def matmul_fsum(a, b):
    """a @ b by a triple loop with exactly rounded sums (math.fsum).  For tiny
    shapes only: it is the fp64-exact-sum definition of a matrix product."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m, k = a.shape
    k2, n = b.shape
    assert k == k2
    out = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            out[i, j] = math.fsum(a[i, t] * b[t, j] for t in range(k))
    return out


def rel_fro(got, ref) -> float:
    """||got - ref||_F / ||ref||_F (0 if both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0:
        return 0.0 if num == 0 else math.inf
    return float(num / den)
