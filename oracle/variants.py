"""Other 4- and 8-bit formats of the frozen weight, for comparison with NF4 +
double quantization: the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * P4 §三 (English derivation): NF4 normalises each 64-block by its absmax
    and picks the nearest of 16 levels; double quantization (P4 §二) then
    re-quantizes the fp32 block constants.  Turning it off leaves the fp32
    constants: 0.5 bit per parameter of overhead (P4 §三: 32/64).
  * P2 §4.1 and P4 (trade-off ②): ordinary 4-bit integer quantization cuts
    the range into uniform steps; NF4's normal-quantile levels lose less on
    Gaussian-like weights.
  * P3 (公式导读 2, the INT8 worked example): absmax integer quantization:
    alpha = 127 / max|x|, q = round(x·alpha), x' = q / alpha.

Readings (all three keep one fp32 absmax c per 64-block, no double
quantization):
  * "nf4"  -- NF4 with DQ off: the codes of oracle.nf4 (x = fl32(w / c),
    nearest level, ties to the lower index), dequantized with the exact fp32
    c: w' = RNE_bf16(fl32(q[code]·c)).
  * "int4" -- absmax INT4, P3's scheme at 4 bits: alpha = fl32(7 / c),
    p = fl32(w·alpha), k = round(p) with halves away from zero (P3's
    rounding), k in [-7, 7] (15 levels), stored as the nibble k + 8 (packed
    like NF4 codes).  Level of code k + 8: L = fl32(k / 7); w' =
    RNE_bf16(fl32(L·c)).
  * "int8" -- absmax INT8 (P3): alpha = fl32(127 / c), the same rounding,
    k in [-127, 127], one byte per weight (two's complement); level
    L = fl32(k / 127), w' = RNE_bf16(fl32(L·c)).
  A block of zeros (c = 0) stores the zero code (nf4: 7, int4: 8, int8: 0).

Pins (tests/test_oracle_variants.py): P3's INT8 worked numbers; closed forms
(blocks on the integer grid come back exactly); the rounding of halves; the
NF4 codes equal oracle.nf4's; error bounds of half a step; the pages' claim
that NF4 reconstructs Gaussian weights better than uniform INT4.
"""

from __future__ import annotations

import numpy as np

from . import nf4

F32 = np.float32
BLOCK = 64
FORMATS = ("nf4", "int4", "int8")
QMAX = {"int4": 7, "int8": 127}


def levels(fmt: str) -> np.ndarray:
    """fp32 level of every code: 16 for nf4 and int4 (int4 code 0 unused,
    level 0), 256 for int8 (indexed by the byte, two's complement)."""
    if fmt == "nf4":
        return nf4.codebook()
    if fmt == "int4":
        k = np.arange(16) - 8
        return np.where(k >= -7, (k.astype(F32) / F32(7)).astype(F32), F32(0)).astype(F32)
    if fmt == "int8":
        k = np.arange(256).astype(np.uint8).view(np.int8).astype(F32)
        return np.where(k >= -127, (k / F32(127)).astype(F32), F32(0)).astype(F32)
    raise ValueError(fmt)


def _round_half_away(p: np.ndarray) -> np.ndarray:
    """round(p) with halves away from zero, p fp32; the result as int32."""
    a = np.floor(np.abs(p).astype(np.float64) + 0.5)
    return (np.sign(p) * a).astype(np.int32)


def quantize(w32: np.ndarray, fmt: str):
    """w32: [N, K] fp32 (K % 64 == 0).  Returns (codes, absmax): codes packed
    nibbles uint8[N*K/2] (nf4, int4) or int8 bytes uint8[N*K] (int8), absmax
    fp32[N*K/64]."""
    w = np.asarray(w32, dtype=F32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("weight must be [N, K] with K % 64 == 0")
    blocks = w.reshape(-1, BLOCK)
    c = nf4.block_absmax(w)
    if fmt == "nf4":
        codes, c2 = nf4.quantize_codes(w)
        assert np.array_equal(c2.view(np.uint32), c.view(np.uint32))
        return nf4.pack_nibbles(codes), c
    qmax = QMAX[fmt]
    with np.errstate(divide="ignore", invalid="ignore"):
        alpha = (F32(qmax) / c).astype(F32)  # inf for a zero block
        p = (blocks * alpha[:, None]).astype(F32)
    p = np.where(c[:, None] > 0, p, F32(0))
    k = np.clip(_round_half_away(p), -qmax, qmax)
    if fmt == "int4":
        return nf4.pack_nibbles((k + 8).astype(np.uint8).reshape(-1)), c
    return k.astype(np.int8).view(np.uint8).reshape(-1), c


def unpack(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Code of every weight (uint8, flattened row-major)."""
    if fmt == "int8":
        return np.asarray(codes, dtype=np.uint8).reshape(-1)
    return nf4.unpack_nibbles(codes)


def dequantize(codes: np.ndarray, absmax: np.ndarray, fmt: str) -> np.ndarray:
    """w' = RNE_bf16(fl32(L[code]·c)); returns uint16 bf16 bits, flattened."""
    L = levels(fmt)
    cd = unpack(codes, fmt).reshape(-1, BLOCK)
    w = (L[cd] * np.asarray(absmax, dtype=F32)[:, None]).astype(F32)
    return nf4.bf16_bits(w).reshape(-1)


def storage_bits_per_weight(fmt: str) -> float:
    """Code bits plus the fp32 absmax spread over its 64-block."""
    return (8.0 if fmt == "int8" else 4.0) + 32.0 / BLOCK


def gemv_ref(X_bits: np.ndarray, W_hat_bits: np.ndarray) -> np.ndarray:
    """Y = X·Ŵᵀ in fp64 from bf16 bit patterns X [M, K] and Ŵ [N, K]."""
    from .linalg import bf16_to_f64

    return bf16_to_f64(X_bits) @ bf16_to_f64(W_hat_bits).T
