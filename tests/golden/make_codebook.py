"""Writes ``nf4_codebook.txt``: the oracle's fp32 NF4 levels and round-down
midpoints as bit patterns.  Calls only ``oracle``.  Run from the repository
root:  python -m tests.golden.make_codebook
"""

from pathlib import Path

HERE = Path(__file__).resolve().parent
OUT = HERE / "nf4_codebook.txt"

HEADER = [
    "# NF4 levels (fp32) and the largest fp32 at or below each midpoint.",
    "# Written by tests/golden/make_codebook.py from oracle.nf4 (a regression",
    "# table of the oracle's reading of P4 §三, not a value printed on the pages).",
    "# columns: index level_bits level_value threshold_bits",
]


def table_lines():
    import numpy as np
    from oracle import nf4

    q = nf4.codebook()
    t = nf4.thresholds(q)
    qb = q.view(np.uint32)
    tb = t.view(np.uint32)
    lines = []
    for i in range(16):
        thr = f"0x{int(tb[i]):08x}" if i < 15 else "-"
        lines.append(f"{i} 0x{int(qb[i]):08x} {float(q[i]):.9f} {thr}")
    return lines


def read_table():
    return [ln for ln in OUT.read_text(encoding="utf-8").splitlines()
            if ln.strip() and not ln.startswith("#")]


if __name__ == "__main__":
    OUT.write_text("\n".join(HEADER + table_lines()) + "\n", encoding="utf-8")
    print(f"wrote {OUT}")
