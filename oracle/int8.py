"""Absmax INT8 quantization (P3 公式导读 2 "INT8 量化" and its four steps).
Oracle (test infrastructure only; see ``oracle/__init__``).

P3 walks the absmax convention on a small vector: find the largest magnitude,
pick the scale alpha that maps it to 127, multiply and round to store, divide
by alpha to restore.  NF4 uses the same absmax convention per 64-block (P4 §三),
which is why the worked numbers serve as a pin of the convention.
"""

from __future__ import annotations

import math

import numpy as np

QMAX = 127


def absmax_scale(x) -> float:
    """alpha = 127 / max|x| in fp64."""
    a = max(abs(float(v)) for v in np.asarray(x, dtype=np.float64).reshape(-1))
    return QMAX / a


def _round_half_away(v: float) -> int:
    return int(math.floor(abs(v) + 0.5)) * (1 if v >= 0 else -1)


def quantize(x):
    """q = round(x * alpha), halves away from zero (the ordinary rounding the
    page's example uses).  Returns (int list, alpha)."""
    alpha = absmax_scale(x)
    q = [_round_half_away(float(v) * alpha) for v in np.asarray(x, dtype=np.float64).reshape(-1)]
    return q, alpha


def dequantize(q, alpha: float):
    """x' = q / alpha."""
    return [float(v) / alpha for v in q]
