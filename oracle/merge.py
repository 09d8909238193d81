"""Merging the LoRA adapter into the dequantized weight: the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * P5 (follow-up 1): at inference the NF4 weight has to be dequantized before
    the product; for speed the fine-tuned model can be converted once to FP16,
    merging the LoRA weights into the dequantized weight, at the cost of the
    memory saving.
  * P1 §五 (limitations): merging and re-quantizing can bring quantization
    error back.
  * P1 §七 (dataflow figure): the layer computes Y = X·Ŵᵀ + s·(X·Aᵀ)·Bᵀ, which
    is X·(Ŵ + s·B·A)ᵀ, so the merged weight is Ŵ + s·B·A.

Reading (the pages give no arithmetic for the merge):
  * Ŵ is the bf16 dequantized weight, exactly as the forward pass multiplies
    it (oracle.nf4.dequantize), A [r, K] and B [N, r] are bf16, and
    s = fl32(alpha / r), the scale the library uses.
  * The merged value is the exact sum Ŵ + s·Σ_j B[n][j]·A[j][k] (formed in
    fp64 here) rounded once, to nearest with ties to even, into the 16-bit
    output format: bf16 (the training path's compute format) or fp16 (the
    format P5 names for the merged model).
  * Re-quantization is the NF4 + double quantization of oracle.nf4, applied to
    the bf16 merged weight.

Pins (tests/test_oracle_merge.py): B = 0 gives Ŵ back exactly; the merged
weight reproduces the forward oracle's output (X·W_mᵀ against
oracle.linalg.linear_fwd); the single-rounding functions against hand-worked
ties and a double-rounding case; re-quantizing Ŵ itself returns the same
codes.
"""

from __future__ import annotations

import numpy as np

from . import nf4
from .linalg import bf16_to_f64

F32 = np.float32


def lora_scale(alpha: float, r: int) -> float:
    """s = fl32(alpha / r), as an exact fp64 value."""
    return float(F32(F32(alpha) / F32(r)))


def merged_exact(W_hat_bits, A_bits, B_bits, alpha: float, r: int) -> np.ndarray:
    """Ŵ + s·B·A in fp64 ([N, K]).  The products of two bf16 values are exact
    in fp64 and r <= 256 of them add with at most fp64 rounding."""
    W = bf16_to_f64(W_hat_bits)
    A = bf16_to_f64(A_bits)
    B = bf16_to_f64(B_bits)
    if A.shape[0] != r or B.shape[1] != r or W.shape != (B.shape[0], A.shape[1]):
        raise ValueError("shapes: W_hat [N, K], A [r, K], B [N, r]")
    return W + lora_scale(alpha, r) * (B @ A)


def round_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 with one rounding to nearest, ties to even (finite values
    within the bf16 range).  bf16 keeps 8 significant bits; below 2^-126 its
    spacing is fixed at 2^-133."""
    x = np.asarray(x64, dtype=np.float64)
    _, e = np.frexp(x)  # x = m·2^e, 0.5 <= |m| < 1
    ulp_exp = np.maximum(e - 8, -133)
    ulp = np.ldexp(np.ones_like(x), ulp_exp)
    v = np.rint(x / ulp) * ulp  # np.rint: ties to even; both steps exact
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > 3.3895313892515355e38):
        raise OverflowError("value outside the bf16 range")
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def round_f16_bits(x64: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 with one rounding to nearest, ties to even (numpy's direct
    double-to-half conversion); values past the fp16 range become infinities."""
    with np.errstate(over="ignore"):
        return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)


def merge(W_hat_bits, A_bits, B_bits, alpha: float, r: int, out: str = "bf16") -> np.ndarray:
    """The merged weight W_m = Ŵ + s·B·A as 16-bit patterns (uint16 [N, K]),
    ``out`` = "bf16" or "f16"."""
    x = merged_exact(W_hat_bits, A_bits, B_bits, alpha, r)
    if out == "bf16":
        return round_bf16_bits(x)
    if out == "f16":
        return round_f16_bits(x)
    raise ValueError(out)


def requantize(merged_bf16_bits: np.ndarray):
    """NF4 + double quantization of a bf16 merged weight [N, K] (P1 §五: the
    step that can bring the error back).  Same dict as oracle.nf4.quantize."""
    return nf4.quantize(nf4.bf16_to_f32(np.asarray(merged_bf16_bits)))
