"""The quantizer's code table (quantize.hip), restated on the CPU with the
oracle's thresholds.

The kernel finds a code as base + (x > t*) from a table of cells: |x| in
[2^-5, 1] is cut by its fp32 exponent and top 3 mantissa bits (bits 20..30),
each sign's cells store the count of thresholds below the cell and the one
threshold inside it; |x| < 2^-5 has the zero code 7.  That is exact only if no
cell holds two thresholds and every threshold has |t| > 2^-5 (the library
checks this when it builds its thresholds).  The tests check the property for
the oracle's thresholds (which equal the library's bit for bit, see
test_abi) and that the table rule gives the oracle's nearest code on every
cell edge, on and next to every threshold, and on a sweep of x in [-1, 1].
"""

import numpy as np

from oracle import nf4

CELL_BIAS = (122 << 3) - 1  # bits 20..30 of 2^-5, minus one
CELLS = 42


def f32(u):
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def bits(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def table(t):
    """(t*, base) per cell: cells 0..41 for x >= 0, then 42..83 for x < 0."""
    tab = []
    for c in range(2 * CELLS):
        neg, i = divmod(c, CELLS)
        if i == 0:
            tab.append((np.float32(np.inf), 7))
            continue
        lo, hi = f32((CELL_BIAS + i) << 20), f32((CELL_BIAS + i + 1) << 20)
        base, tstar = 0, np.float32(np.inf)
        for tj in t:
            if not neg:
                if tj < lo:
                    base += 1
                elif tj < hi:
                    tstar = tj
            else:
                if tj <= -hi:
                    base += 1
                elif tj <= -lo:
                    tstar = tj
        tab.append((tstar, base))
    return tab


def table_code(tab, x):
    u = bits(x)
    mag = max(((u & 0x7FFFFFFF) >> 20) - CELL_BIAS, 0)
    tstar, base = tab[mag + (u >> 31) * CELLS]
    return base + (1 if np.float32(x) > tstar else 0)


def test_thresholds_fall_one_per_cell():
    t = nf4.thresholds(nf4.codebook())
    assert all(abs(float(v)) > 2.0 ** -5 for v in t)
    cells = {}
    for v in t:
        u = bits(v)
        key = (u >> 31, (u & 0x7FFFFFFF) >> 20)
        assert key not in cells, f"thresholds {cells.get(key)} and {v} share a cell"
        cells[key] = v


def test_table_rule_equals_the_nearest_code():
    t = nf4.thresholds(nf4.codebook())
    tab = table(t)
    xs = [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0)]
    for v in t:
        for d in range(-3, 4):
            xs.append(np.nextafter(np.float32(v), np.float32(np.inf if d > 0 else -np.inf)) if d else v)
            y = np.float32(v)
            for _ in range(abs(d)):
                y = np.nextafter(y, np.float32(np.inf if d > 0 else -np.inf))
            xs.append(y)
    for i in range(2 * CELLS):
        for s in (1, -1):
            e = f32((CELL_BIAS + (i % CELLS) + 1) << 20) if i % CELLS else np.float32(2.0 ** -5)
            for y in (e, np.nextafter(e, np.float32(0)), np.nextafter(e, np.float32(2))):
                if abs(float(y)) <= 1.0:
                    xs.append(np.float32(s * y))
    rng = np.random.default_rng(4)
    xs.extend(rng.uniform(-1, 1, 20000).astype(np.float32))
    xs = np.array(xs, dtype=np.float32)
    ref = nf4.nearest_code(xs, nf4.codebook())
    got = np.array([table_code(tab, x) for x in xs])
    assert np.array_equal(got, ref)
