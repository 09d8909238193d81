"""GPU parity of quantization, double quantization and dequantization against
the oracle: bit-exact codes, E4M3 constants, group scales, mean and
dequantized bf16 weights.  Every call goes through the C ABI."""

import numpy as np
import pytest

from oracle import nf4
from tests import gpu_util as G
from workloads import Inputs, random_f32, to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def check_full(W32: np.ndarray, W_dev):
    qt = G.gpu_quantize(W_dev)
    ref = nf4.quantize(W32)
    assert np.array_equal(G.host(qt.codes), ref["codes"]), "codes"
    assert np.array_equal(G.host(qt.absmax_e4m3), ref["absmax_e4m3"]), "e4m3 constants"
    assert np.array_equal(G.host(qt.dq_scale).view(np.uint32), ref["dq_scale"].view(np.uint32)), "scales"
    assert G.host(qt.dq_mean).view(np.uint32)[0] == np.float32(ref["dq_mean"]).view(np.uint32), "mean"
    w_hat = G.host_bf16(G.gpu_dequantize(qt)).reshape(-1)
    assert np.array_equal(w_hat, G.oracle_w_hat(ref)), "dequantized weight"
    return qt


def test_tiny_layer_fp32():
    w = Inputs(1)
    W = w.weight(0)
    print("tiny 256x256 fp32", flush=True)
    check_full(W, G.dev_f32(W))


def test_qproj_4096_fp32_with_outliers():
    w = Inputs(2)
    W = w.weight(0)
    print("q_proj 4096x4096 fp32", flush=True)
    check_full(W, G.dev_f32(W))


def test_bf16_input_attention_shape():
    w = Inputs(4)
    Wb = w.weight(0)  # bf16 bits, 4096x4096
    print("7b q 4096x4096 bf16", flush=True)
    check_full(bf16_bits_to_f32(Wb), G.dev_bf16(Wb))


@pytest.mark.parametrize("n,k", [(8, 64), (8, 320), (24, 192), (4096, 4160)])
def test_ragged_group_and_tree_shapes(n, k):
    # nb = 8 (one partial group), 40, 72 and 266240 (1040 chunks: two levels of
    # the pairwise mean)
    W = random_f32((n, k), seed=1000 + n + k, scale=0.02)
    print(f"shape {n}x{k}", flush=True)
    check_full(W, G.dev_f32(W))


def test_edge_values():
    rng = np.random.default_rng(77)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    W[0, :] = 0.0                        # zero blocks
    W[1, :64] = -0.0
    W[2, :] *= np.float32(1e-39)         # subnormal weights
    W[3, :64] = np.float32(1.0)          # constant block
    W[4, :] = np.abs(W[4, :])            # one-signed blocks
    W[5, 7] = np.float32(3.0)            # isolated outlier
    q = nf4.codebook()
    m = nf4.midpoints(q)
    W[6, :15] = [np.float32(v) for v in m]  # x exactly at midpoints (block max 1.0 below)
    W[6, 15] = 1.0
    print("edge values", flush=True)
    check_full(W, G.dev_f32(W))


def test_quotients_at_thresholds():
    # x = fl32(w / m) lands on or next to every decision threshold, for block
    # maxima spread over binades (including just below powers of two and
    # tiny ones): the codes depend on the quotient being correctly rounded
    q = nf4.codebook()
    t = nf4.thresholds(q).astype(np.float32)
    rng = np.random.default_rng(123)
    maxima = [np.float32(1.0), np.float32(np.nextafter(np.float32(2.0), np.float32(0))),
              np.float32(0.75), np.float32(3.0e-3), np.float32(np.nextafter(np.float32(0.5), np.float32(0))),
              np.float32(1e-30), np.float32(2.0 ** -120), np.float32(12345.678)]
    maxima += [np.float32(v) for v in rng.uniform(1e-3, 10.0, 24)]
    rows = []
    for m in maxima:
        for j in range(15):
            target = np.float32(t[j] * np.float64(m))
            blk = []
            for d in range(-2, 3):  # w = fl32(t_j * m) moved by -2..2 ulps
                v = target
                for _ in range(abs(d)):
                    v = np.nextafter(v, np.float32(np.inf if d > 0 else -np.inf))
                blk.append(v)
            blk = np.array(blk, dtype=np.float32)
            row = np.zeros(64, dtype=np.float32)
            row[0] = m  # the block maximum
            row[1:1 + len(blk)] = np.clip(blk, -m, m)
            rows.append(row)
    W = np.stack(rows).reshape(-1, 256)
    print(f"quotients at thresholds: {W.size // 64} blocks", flush=True)
    check_full(W, G.dev_f32(W))


def test_mlp_weight_sampled():
    # full-size 11008x4096 fp32 weight: mean, all constants and scales exact;
    # codes and dequantized values exact on 64 sampled weight rows
    w = Inputs(3)
    W = w.weight(0)
    print("7b gate 11008x4096 fp32", flush=True)
    qt = G.gpu_quantize(G.dev_f32(W))
    o = G.SampledOracle(W)
    assert G.host(qt.dq_mean).view(np.uint32)[0] == np.float32(o.mu).view(np.uint32)
    assert np.array_equal(G.host(qt.absmax_e4m3), o.e)
    assert np.array_equal(G.host(qt.dq_scale).view(np.uint32), o.s.view(np.uint32))
    rows = np.sort(np.random.default_rng(5).choice(W.shape[0], 64, replace=False))
    codes_gpu = G.host(qt.codes).reshape(W.shape[0], -1)[rows]
    codes_ref, _ = nf4.quantize_codes(W[rows])
    assert np.array_equal(codes_gpu.reshape(-1), nf4.pack_nibbles(codes_ref))
    w_hat = G.host_bf16(G.gpu_dequantize(qt)).reshape(W.shape)[rows]
    assert np.array_equal(w_hat, o._blocks(rows, 0, W.shape[1] // 64))


def test_large_tensor_tree_levels():
    # 16448x16384 (270 M weights): 16448 partial sums of 256 constants, more
    # than the encode kernel sums itself, so one tree level runs on its own
    # first; mean, all E4M3 constants and all group scales exact
    W = random_f32((16448, 16384), seed=4242, scale=0.02)
    print("16448x16384 fp32 (tree levels)", flush=True)
    qt = G.gpu_quantize(G.dev_f32(W))
    o = G.SampledOracle(W)
    assert G.host(qt.dq_mean).view(np.uint32)[0] == np.float32(o.mu).view(np.uint32)
    assert np.array_equal(G.host(qt.absmax_e4m3), o.e)
    assert np.array_equal(G.host(qt.dq_scale).view(np.uint32), o.s.view(np.uint32))


@pytest.mark.parametrize("n,k,seed", [(32000, 4096, 5061), (22016, 8192, 5037), (32000, 8192, 5042)])
def test_bulk_shapes_device_drawn(n, k, seed):
    # the bulk quantization shapes, drawn on the GPU as the bulk measurement
    # draws them (bf16 N(0, 0.02^2)); mean, all E4M3 constants and group
    # scales exact; codes and dequantized weights exact on 32 sampled rows
    from workloads import device_normal

    t = G.torch()
    print(f"bulk shape {n}x{k} bf16 seed {seed}", flush=True)
    Wd = device_normal(t, (n, k), seed, 0.02)
    qt = G.gpu_quantize(Wd)
    W = bf16_bits_to_f32(G.host(Wd.view(t.int16)).view(np.uint16))
    del Wd
    o = G.SampledOracle(W)
    assert G.host(qt.dq_mean).view(np.uint32)[0] == np.float32(o.mu).view(np.uint32)
    assert np.array_equal(G.host(qt.absmax_e4m3), o.e)
    assert np.array_equal(G.host(qt.dq_scale).view(np.uint32), o.s.view(np.uint32))
    rows = np.sort(np.random.default_rng(seed).choice(n, 32, replace=False))
    codes_gpu = G.host(qt.codes).reshape(n, -1)[rows]
    codes_ref, _ = nf4.quantize_codes(W[rows])
    assert np.array_equal(codes_gpu.reshape(-1), nf4.pack_nibbles(codes_ref))
    w_hat = G.host_bf16(G.gpu_dequantize(qt)).reshape(n, k)[rows]
    assert np.array_equal(w_hat, o._blocks(rows, 0, k // 64))


def test_deterministic():
    W = random_f32((1024, 1024), seed=9, scale=0.02)
    Wd = G.dev_f32(W)
    a = G.gpu_quantize(Wd)
    b = G.gpu_quantize(Wd)
    for name in ("codes", "absmax_e4m3", "dq_scale", "dq_mean"):
        assert np.array_equal(G.host(getattr(a, name)), G.host(getattr(b, name))), name
