"""Storage arithmetic of NF4 + double quantization.  Oracle (test
infrastructure only; see ``oracle/__init__``).

P4 §二 / §三 (English derivation, double quantization): fp32 constants every 64
parameters cost 32/64 = 0.5 bit per parameter; with the constants quantized to
8 bits and one fp32 second-level constant per 256 of them the cost is
8/64 + 32/(64*256) bits per parameter.
"""

from __future__ import annotations

BLOCK = 64
DQ_BLOCK = 256


def constant_bits_per_param(double_quant: bool, block: int = BLOCK,
                            dq_block: int = DQ_BLOCK) -> float:
    if double_quant:
        return 8.0 / block + 32.0 / (block * dq_block)
    return 32.0 / block


def dq_saving_bits_per_param() -> float:
    return constant_bits_per_param(False) - constant_bits_per_param(True)


def dq_saving_bytes(n_params: float) -> float:
    return n_params * dq_saving_bits_per_param() / 8.0


def tensor_bytes(n_rows: int, n_cols: int) -> dict:
    """Bytes of the four arrays of one NF4 + DQ tensor [n_rows, n_cols]."""
    numel = n_rows * n_cols
    nb = numel // BLOCK
    ng = (nb + DQ_BLOCK - 1) // DQ_BLOCK
    return {"codes": numel // 2, "absmax_e4m3": nb, "dq_scale": 4 * ng, "dq_mean": 4}


def bits_per_param(n_rows: int, n_cols: int) -> float:
    b = tensor_bytes(n_rows, n_cols)
    return 8.0 * sum(b.values()) / (n_rows * n_cols)


def weight_bytes(n_params: float, bits: float) -> float:
    return n_params * bits / 8.0
