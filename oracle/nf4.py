"""NF4 storage format: codebook, blockwise quantization, double quantization,
dequantization.  Oracle (test infrastructure only; see ``oracle/__init__``).

Arithmetic conventions (the pages fix none of them; they are chosen so that two
independent implementations produce identical bytes):
  * fp32 values are IEEE binary32 with round-to-nearest-even; numpy float32
    arithmetic is used for every fp32 operation, one rounding per operation,
    no fused multiply-add, no flush-to-zero;
  * bf16 is the upper half of binary32, rounded to nearest, ties to even;
  * the 8-bit float of double quantization is OCP FP8 E4M3 (bias 7, 3 mantissa
    bits, largest finite 448, subnormals down to 2^-9, S.1111.111 is NaN, no
    infinities).
"""

from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

# P4 §三 (English derivation, eq. for W^norm): weights are normalised in blocks
# of B = 64 consecutive elements by the block's largest magnitude.
BLOCK = 64
# P4 §三 (English derivation, double quantization): the first-level constants
# are themselves quantized to an 8-bit float with a second-level block of 256.
DQ_BLOCK = 256
# Largest finite OCP E4M3 magnitude.
E4M3_MAX = 448.0
# Index of the exact zero in the codebook (7 negative levels below it).
ZERO_CODE = 7
# Probability at which both halves of the codebook end (reading of P4 §三, see
# ``codebook_f64``).
P_END = 31.0 / 32.0


# ----------------------------------------------------------------------------
# Codebook  (P4 §三 English derivation: NF4 levels at standard-normal
# quantiles; P4 §三 中文: each level carries the same probability mass; exact
# zero kept by an adjustment around zero)
# ----------------------------------------------------------------------------

def _normal_quantile(p: float) -> float:
    """Φ⁻¹(p) for the standard normal, in fp64 (the Q_X of P4 §三)."""
    return NormalDist(0.0, 1.0).inv_cdf(p)


def codebook_f64() -> list[float]:
    """The 16 NF4 levels in fp64, ascending.

    P4 §三 places the 16 levels at quantiles of the standard normal so that each
    level covers the same probability mass, and states that an adjustment
    around zero keeps an exact zero.  The literal midpoint formula printed there
    is infinite at both ends and has no zero, so it needs a reading.  Reading
    used here (the plainest one that gives 16 finite, sorted values in [-1, 1]
    including 0):

      * one exact zero at index 7;
      * 8 positive and 7 negative levels (the only near-symmetric split of 15
        non-zero levels; the extra level goes to the positive side);
      * each side sits at quantiles of evenly spaced probabilities running from
        1/2 (exclusive; that is the zero) up to p_end = 31/32, the centre of the
        top bin when [0, 1] is cut into 2^4 equal-mass bins;
      * both sides are divided by z = Φ⁻¹(p_end), so the ends are exactly -1
        and +1 (the block maximum, normalised to ±1, is represented exactly).
    """
    z = _normal_quantile(P_END)
    step = P_END - 0.5
    pos = [_normal_quantile(0.5 + j * step / 8.0) / z for j in range(1, 9)]
    neg = [-_normal_quantile(0.5 + j * step / 7.0) / z for j in range(1, 8)]
    return sorted(neg) + [0.0] + pos


def codebook() -> np.ndarray:
    """The NF4 levels as float32 (each fp64 level rounded to nearest even)."""
    return np.array(codebook_f64(), dtype=np.float64).astype(np.float32)


def midpoints(q32: np.ndarray) -> np.ndarray:
    """Exact midpoints (q[j] + q[j+1]) / 2 in fp64 (exact: the levels are fp32
    in [-1, 1] with small exponent gaps, so the sum needs < 53 bits)."""
    q = q32.astype(np.float64)
    return (q[:-1] + q[1:]) / 2.0


def thresholds(q32: np.ndarray) -> np.ndarray:
    """t_j = the largest fp32 value <= midpoint j, for j = 0..14.

    For an fp32 x:  x > t_j  <=>  x > m_j  (if m_j is representable t_j = m_j;
    otherwise no fp32 lies strictly between t_j and m_j).  So the nearest code
    with ties to the lower index is  #{j : x > t_j}.  Used by the pins as an
    independent formulation of the argmin in ``nearest_code``.
    """
    m = midpoints(q32)
    t = m.astype(np.float32)
    over = t.astype(np.float64) > m
    t[over] = np.nextafter(t[over], np.float32(-np.inf))
    return t


# ----------------------------------------------------------------------------
# Blockwise quantization  (P4 §三 English derivation: W^norm = W / max|W_block|,
# W^NF4 = argmin_q |W^norm - q|)
# ----------------------------------------------------------------------------

def block_absmax(w32: np.ndarray) -> np.ndarray:
    """c_b = max |w| over each block of 64 consecutive elements of the
    row-major flattened weight (fp32, exact)."""
    w = np.ascontiguousarray(w32, dtype=np.float32).reshape(-1, BLOCK)
    return np.max(np.abs(w), axis=1)


def nearest_code(x32: np.ndarray, q32: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """argmin_j |x - q_j|, the first minimiser (ties go to the lower index).

    The distances are taken in fp64.  Wherever two candidates are close to a
    tie, x lies near a midpoint of two levels, so x and the levels have nearby
    exponents and both differences are exact in fp64; the comparison is then
    exact.  np.argmin returns the first minimiser.
    """
    x = np.asarray(x32, dtype=np.float32).reshape(-1).astype(np.float64)
    q = q32.astype(np.float64)
    out = np.empty(x.shape[0], dtype=np.uint8)
    for s in range(0, x.shape[0], chunk):
        d = np.abs(x[s:s + chunk, None] - q[None, :])
        out[s:s + chunk] = np.argmin(d, axis=1).astype(np.uint8)
    return out


def quantize_codes(w32: np.ndarray, q32: np.ndarray | None = None):
    """Blockwise NF4 codes of a weight.

    Returns (codes uint8 one per element, row-major flattened; c fp32 [nb]).
    x = fl32(w / c_b) is one correctly rounded fp32 division.  A block whose
    absmax is 0 gets the zero code everywhere.  No mean is subtracted from the
    weights (P4 §三 English derivation and the 64-element absmax block; the
    mean-centring belongs to double quantization).
    """
    if q32 is None:
        q32 = codebook()
    w = np.ascontiguousarray(w32, dtype=np.float32).reshape(-1, BLOCK)
    c = block_absmax(w)
    codes = np.full(w.shape, ZERO_CODE, dtype=np.uint8)
    nz = c != 0
    if np.any(nz):
        x = np.divide(w[nz], c[nz][:, None])  # float32 / float32 -> float32
        codes[nz] = nearest_code(x, q32).reshape(-1, BLOCK)
    return codes.reshape(-1), c


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte (P3 table of bytes per weight: 4-bit is 0.5 B).
    Flattened element i goes to byte i // 2: low nibble if i is even, high
    nibble if i is odd."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.shape[0] * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------
# OCP FP8 E4M3
# ----------------------------------------------------------------------------

def e4m3_decode_scalar(b: int) -> float:
    """Value of one E4M3 byte from the format's definition."""
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """float32 value of every byte 0..255 (all exact in fp32)."""
    return np.array([e4m3_decode_scalar(b) for b in range(256)], dtype=np.float32)


def e4m3_encode(y32: np.ndarray) -> np.ndarray:
    """Round fp32 values to E4M3: nearest finite value, ties to the even
    mantissa, magnitudes at or beyond 448 saturate to 448, never NaN.  The sign
    bit is the sign of y (so -0 and negative values that round to zero give
    0x80)."""
    y = np.asarray(y32, dtype=np.float32).reshape(-1)
    mags = e4m3_table()[:0x7F].astype(np.float64)  # codes 0x00..0x7E, ascending
    a = np.abs(y.astype(np.float64))
    out = np.empty(y.shape[0], dtype=np.uint8)
    sat = a >= E4M3_MAX
    out[sat] = 0x7E
    idx = np.nonzero(~sat)[0]
    if idx.size:
        av = a[idx]
        i = np.searchsorted(mags, av, side="right") - 1  # mags[i] <= a < mags[i+1]
        lo = mags[i]
        hi = mags[i + 1]
        two_a = 2.0 * av          # exact
        mid2 = lo + hi            # exact (two E4M3 values)
        pick_hi = (two_a > mid2) | ((two_a == mid2) & ((i & 1) == 1))
        out[idx] = np.where(pick_hi, i + 1, i).astype(np.uint8)
    neg = np.signbit(y)
    out[neg] |= 0x80
    return out


# ----------------------------------------------------------------------------
# Double quantization  (P4 §二 / §三: first-level fp32 constants -> 8-bit float,
# second-level block 256; the mean-centred e4m3 form with one fp32 scale per 256
# constants is the reading adopted for the "8-bit FP" of the pages)
# ----------------------------------------------------------------------------

def tree_sum_f64(v: np.ndarray) -> float:
    """Balanced binary-tree sum in fp64: zero-pad to the next power of two and
    add adjacent pairs level by level until one value remains."""
    x = np.asarray(v, dtype=np.float64).reshape(-1)
    n = 1
    while n < x.shape[0]:
        n *= 2
    if n != x.shape[0]:
        x = np.concatenate([x, np.zeros(n - x.shape[0])])
    while x.shape[0] > 1:
        x = x[0::2] + x[1::2]
    return float(x[0]) if x.shape[0] else 0.0


def double_quant(c32: np.ndarray):
    """Quantize the block constants.

    Returns (e uint8[nb], s float32[ng], mu float32):
      mu  = fl32(S / nb) with S the fp64 tree sum of all constants of the
            tensor (one mean per tensor keeps the footprint of P4 §三 at
            8/64 + 32/(64*256) bits per parameter);
      d_b = fl32(c_b - mu);
      s_g = fl32(max|d| over group g / 448), group g = constants [256g, 256g+256);
      e_b = E4M3(fl32(d_b / s_g)), or 0x00 for every constant of a group whose
            scale is 0.
    """
    c = np.asarray(c32, dtype=np.float32).reshape(-1)
    nb = c.shape[0]
    S = tree_sum_f64(c.astype(np.float64))
    mu = np.float32(S / float(nb))
    d = (c - mu).astype(np.float32)
    ng = (nb + DQ_BLOCK - 1) // DQ_BLOCK
    e = np.zeros(nb, dtype=np.uint8)
    s = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        dg = d[g * DQ_BLOCK:(g + 1) * DQ_BLOCK]
        m = np.max(np.abs(dg))
        sg = np.float32(m) / np.float32(E4M3_MAX)
        s[g] = sg
        if sg == 0:
            continue
        y = (dg / sg).astype(np.float32)
        e[g * DQ_BLOCK:(g + 1) * DQ_BLOCK] = e4m3_encode(y)
    return e, s, np.float32(mu)


def decode_constants(e: np.ndarray, s: np.ndarray, mu) -> np.ndarray:
    """c'_b = fl32(fl32(dec(e_b) * s_g) + mu), two roundings, no clamp."""
    e = np.asarray(e, dtype=np.uint8).reshape(-1)
    g = np.arange(e.shape[0]) // DQ_BLOCK
    prod = (e4m3_table()[e] * np.asarray(s, dtype=np.float32)[g]).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


# ----------------------------------------------------------------------------
# bf16 and dequantization  (P1 §七: the frozen 4-bit weight is dequantized block
# by block to BF16 just before the matmul; P4 §四 English ①: Ŵ = Dequant(W^NF4)·c)
# ----------------------------------------------------------------------------

def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit
    patterns.  Finite inputs only."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b16: np.ndarray) -> np.ndarray:
    return (np.asarray(b16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to IEEE binary16 (nearest, ties to even, subnormals kept,
    overflow to infinity); returns the uint16 bit patterns.  (numpy's
    float-to-half conversion, one rounding.)"""
    with np.errstate(over="ignore"):
        return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(b16: np.ndarray) -> np.ndarray:
    return np.asarray(b16, dtype=np.uint16).view(np.float16).astype(np.float32)


def round16(x32: np.ndarray, fmt16: str) -> np.ndarray:
    """fp32 -> 16-bit bit patterns in the compute format ("bf16" or "f16")."""
    if fmt16 == "bf16":
        return bf16_bits(x32)
    if fmt16 == "f16":
        return f16_bits(x32)
    raise ValueError(fmt16)


def dequantize(packed: np.ndarray, e: np.ndarray, s: np.ndarray, mu,
               q32: np.ndarray | None = None, fmt16: str = "bf16") -> np.ndarray:
    """ŵ_i = RNE16(fl32(q[code_i] * c'_b)) with RNE16 the rounding into the
    compute format (bf16 by default; fp16 for the fp16 compute path, P1 §四
    and §七 naming FP16 beside BF16); returns uint16 bit patterns, flattened
    row-major.  Signed zeros follow IEEE (code 7 with c' < 0 gives -0)."""
    codes = unpack_nibbles(packed).reshape(-1, BLOCK)
    return dequantize_blocks(codes, np.arange(codes.shape[0]), e, s, mu, q32, fmt16).reshape(-1)


def dequantize_blocks(codes: np.ndarray, block_ids: np.ndarray, e: np.ndarray, s: np.ndarray,
                      mu, q32: np.ndarray | None = None, fmt16: str = "bf16") -> np.ndarray:
    """The same dequantization for a subset of blocks: ``codes`` holds the
    unpacked codes of the listed blocks ([len(block_ids), 64]); ``e``, ``s`` and
    ``mu`` are the whole tensor's constants.  Returns uint16 bit patterns of
    the compute format [len(block_ids), 64].  (Blocks dequantize
    independently of each other.)"""
    if q32 is None:
        q32 = codebook()
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, BLOCK)
    cp = decode_constants(e, s, mu)[np.asarray(block_ids)]
    w32 = (q32[codes] * cp[:, None]).astype(np.float32)
    return round16(w32, fmt16)


def quantize(w32: np.ndarray):
    """Full NF4 + double quantization of one weight tensor [N, K] (K % 64 == 0).

    Returns a dict with packed codes (uint8[N*K/2]), e4m3 constants (uint8[nb]),
    group scales (float32[ng]), mean (float32), and the raw fp32 absmax c.
    """
    w = np.asarray(w32, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("weight must be [N, K] with K % 64 == 0")
    codes, c = quantize_codes(w)
    e, s, mu = double_quant(c)
    return {"codes": pack_nibbles(codes), "absmax_e4m3": e, "dq_scale": s,
            "dq_mean": mu, "absmax": c, "shape": w.shape}
