"""The oracle against numbers the pages print (fixtures under tests/golden/,
each with its citation).  CPU only."""

import numpy as np

from oracle import footprint, int8
from tests.golden._fixture import load


def test_int8_absmax_worked_example():
    g = load("int8_absmax_example.txt")
    x = [float(v) for v in g["input"].split()]
    q, alpha = int8.quantize(x)
    assert max(abs(v) for v in x) == float(g["absmax"])
    assert abs(alpha - float(g["alpha_approx"])) < float(g["alpha_tolerance"])
    assert round(alpha) == int(g["alpha_rounded"])
    assert q[0] == int(g["code_of_1.2"])
    assert q[2] == int(g["code_of_peak"])
    back = int8.dequantize([q[0]], alpha)[0]
    assert abs(back - float(g["restored_of_28"])) < float(g["restored_tolerance"])
    # derived, not printed: -0.5 -> round(-11.76) = -12
    assert q[1] == -12


def test_footprint_arithmetic():
    g = load("footprint.txt")
    assert int(g["block"]) == footprint.BLOCK and int(g["dq_block"]) == footprint.DQ_BLOCK
    assert footprint.constant_bits_per_param(False) == float(g["bits_without_dq"])
    assert abs(footprint.constant_bits_per_param(True) - float(g["bits_with_dq"])) \
        < float(g["bits_with_dq_tolerance"])
    assert footprint.constant_bits_per_param(True) == 8 / 64 + 32 / (64 * 256)
    assert abs(footprint.dq_saving_bits_per_param() - float(g["saving_bits"])) \
        < float(g["saving_bits_tolerance"])
    saved = footprint.dq_saving_bytes(float(g["model_params"]))
    assert abs(saved - float(g["saving_bytes"])) < float(g["saving_bytes_tolerance"])


def test_memory_arithmetic():
    g = load("memory.txt")
    assert footprint.weight_bytes(float(g["params_7b"]), 16) == float(g["bf16_bytes_7b"])
    assert footprint.weight_bytes(float(g["params_7b"]), 4) == float(g["int4_bytes_7b"])
    assert footprint.weight_bytes(float(g["params_65b"]), 16) == float(g["bf16_bytes_65b"])
    for key, bits in (("bytes_fp32", 32), ("bytes_fp16", 16), ("bytes_int8", 8), ("bytes_int4", 4)):
        assert footprint.weight_bytes(1, bits) == float(g[key])
    assert 32 / 4 == float(g["ratio_32_to_4"])


def test_nf4_dq_weights_fit_the_pages_claims():
    # NF4 + DQ storage of the 65B model is far below the 130 GB of 16-bit
    # weights (P2 §二) and fits the single 48 GB card of P2 §五 with room for
    # activations and adapters.
    bits = 4 + footprint.constant_bits_per_param(True)
    assert footprint.weight_bytes(65e9, bits) < 48e9
    assert abs(footprint.weight_bytes(65e9, bits) / 1e9 - 33.5) < 0.1
