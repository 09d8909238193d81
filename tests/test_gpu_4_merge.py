"""GPU parity of the LoRA merge (qlora_merge_lora) against the oracle
(oracle/merge.py): every element within one unit in the last place of the
16-bit output (the device sums in fp32, the oracle exactly, each then rounds
once), nearly all of them bit-exact; B = 0 gives the dequantized weight bit
for bit; the merged bf16 weight re-quantized on the device against the
oracle's re-quantization of the same merged weight.  Calls go through the C
ABI."""

import numpy as np
import pytest

import quantized_fine_tuning_amd as q
from oracle import merge, nf4
from tests import gpu_util as G
from workloads import Inputs

pytestmark = pytest.mark.gpu

# a rounding of the device's fp32 sum can differ from the exact sum's only
# near a rounding boundary of the output format
MAX_MISMATCH_FRACTION = {"bf16": 1e-3, "f16": 1e-2}


def torch():
    import torch as t
    return t


def gpu_merge(qt, Ad, Bd, r, alpha, out):
    t = torch()
    dt = t.bfloat16 if out == "bf16" else t.float16
    Wm = t.full((qt.n_rows, qt.n_cols), float("nan"), dtype=dt, device="cuda")
    q.qlora_merge_lora(qt, Ad, Bd, r, alpha, Wm)
    t.cuda.synchronize()
    return Wm.view(t.int16).cpu().numpy().view(np.uint16)


def compare(got, ref, out, what):
    """got, ref: uint16 bit patterns of finite values of one format."""
    assert got.shape == ref.shape
    gv = (nf4.bf16_to_f32(got).astype(np.float64) if out == "bf16"
          else got.view(np.float16).astype(np.float64))
    rv = (nf4.bf16_to_f32(ref).astype(np.float64) if out == "bf16"
          else ref.view(np.float16).astype(np.float64))
    assert np.all(np.isfinite(gv)), f"{what}: non-finite output"
    diff = got != ref
    n_diff = int(diff.sum())
    if n_diff:
        # neighbours in the format: same sign, bit patterns one apart (or
        # both zeros)
        g, rr = got[diff].astype(np.int64), ref[diff].astype(np.int64)
        same_sign = (g >> 15) == (rr >> 15)
        zeros = (gv[diff] == 0) & (rv[diff] == 0)
        assert np.all((same_sign & (np.abs(g - rr) == 1)) | zeros), \
            f"{what}: an element differs by more than one unit in the last place"
    frac = n_diff / got.size
    assert frac <= MAX_MISMATCH_FRACTION[out], f"{what}: {n_diff} of {got.size} elements one ulp off"
    print(f"  {what}: {n_diff} of {got.size} one ulp off", flush=True)


def oracle_layer(W32, A, B):
    ref = nf4.quantize(W32)
    W_hat = G.oracle_w_hat(ref).reshape(W32.shape)
    return ref, W_hat


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_tiny_layer(out):
    # the tiny 256 x 256 layer, r = 8, alpha = 16
    w = Inputs(1)
    W32, A, B = w.weight(0), w.lora_A(0), w.lora_B(0)
    r, alpha = w.w.rank, w.w.alpha
    print(f"merge tiny {W32.shape} r={r} {out}", flush=True)
    _, W_hat = oracle_layer(W32, A, B)
    qt = G.gpu_quantize(G.dev_f32(W32))
    got = gpu_merge(qt, G.dev_bf16(A), G.dev_bf16(B), r, alpha, out)
    compare(got, merge.merge(W_hat, A, B, alpha, r, out), out, "tiny")


@pytest.mark.parametrize("N, K, r, alpha", [
    (72, 320, 7, 3.5),      # rows past a 64-row tile, 5 blocks per row, rank below 32, odd rank
    (136, 192, 256, 64.0),  # the largest rank: 8 slices of 32
    (8, 64, 33, 1.0),       # one block per row, a rank just past a slice
])
@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_ragged_shapes(N, K, r, alpha, out):
    print(f"merge ragged N={N} K={K} r={r} {out}", flush=True)
    rng = np.random.default_rng(N * 1000 + r)
    W32 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = nf4.bf16_bits((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    B = nf4.bf16_bits((rng.standard_normal((N, r)) * 0.05).astype(np.float32))
    _, W_hat = oracle_layer(W32, A, B)
    qt = G.gpu_quantize(G.dev_f32(W32))
    got = gpu_merge(qt, G.dev_bf16(A), G.dev_bf16(B), r, alpha, out)
    compare(got, merge.merge(W_hat, A, B, alpha, r, out), out, f"{N}x{K} r={r}")


def test_zero_adapter_gives_the_dequantized_weight():
    rng = np.random.default_rng(11)
    N, K, r = 200, 448, 16
    W32 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = nf4.bf16_bits((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    qt = G.gpu_quantize(G.dev_f32(W32))
    B0 = np.zeros((N, r), np.uint16)
    got = gpu_merge(qt, G.dev_bf16(A), G.dev_bf16(B0), r, 32.0, "bf16")
    assert np.array_equal(got, G.host_bf16(G.gpu_dequantize(qt)))
    # re-quantizing it returns the codes (NF4 is idempotent on its own output)
    t = torch()
    Wm = t.from_numpy(got.view(np.int16)).view(t.bfloat16).cuda()
    qt2 = G.gpu_quantize(Wm)
    assert np.array_equal(G.host(qt2.codes), G.host(qt.codes))


def test_requantized_merge_matches_the_oracle():
    # the device-merged bf16 weight through the device quantizer, against the
    # oracle's re-quantization of the oracle's merged weight: the codes of
    # every block whose merged values agree bit for bit are equal (codes
    # depend on the block alone); the constants, which go through the
    # tensor-wide mean, are equal when every merged value agrees
    w = Inputs(1)
    W32, A, B = w.weight(0), w.lora_A(0), w.lora_B(0)
    r, alpha = w.w.rank, w.w.alpha
    _, W_hat = oracle_layer(W32, A, B)
    ref_m = merge.merge(W_hat, A, B, alpha, r, "bf16")
    qt = G.gpu_quantize(G.dev_f32(W32))
    got = gpu_merge(qt, G.dev_bf16(A), G.dev_bf16(B), r, alpha, "bf16")
    t = torch()
    qt2 = G.gpu_quantize(t.from_numpy(got.view(np.int16)).view(t.bfloat16).cuda())
    rq = merge.requantize(ref_m)
    same = np.all(got.reshape(-1, 64) == ref_m.reshape(-1, 64), axis=1)
    print(f"  {int(same.sum())} of {same.size} merged blocks identical", flush=True)
    assert same.mean() > 0.99
    codes = G.host(qt2.codes).reshape(-1, 32)
    assert np.array_equal(codes[same], rq["codes"].reshape(-1, 32)[same])
    if same.all():
        assert np.array_equal(G.host(qt2.absmax_e4m3), rq["absmax_e4m3"])
        assert np.array_equal(G.host(qt2.dq_scale).view(np.uint32), rq["dq_scale"].view(np.uint32))
        assert G.host(qt2.dq_mean).view(np.uint32)[0] == np.float32(rq["dq_mean"]).view(np.uint32)


@pytest.mark.parametrize("layer", [0, 2])
def test_mlp_7b_full_size_sampled_rows(layer):
    # the 7B MLP's gate (11008 x 4096) and down (4096 x 11008) weights at
    # r = 64, in the launch configuration the benchmark times; the oracle
    # merges 96 sampled rows
    w = Inputs(3)
    r, alpha = w.w.rank, w.w.alpha
    Wst, A, B = w.weight(layer), w.lora_A(layer), w.lora_B(layer)
    if w.w.weight_dtype == "bf16":
        W32, w_dev = (Wst.astype(np.uint32) << 16).view(np.float32), G.dev_bf16(Wst)
    else:
        W32, w_dev = Wst, G.dev_f32(Wst)
    N, K = W32.shape
    print(f"merge 7b MLP {N}x{K} r={r}", flush=True)
    qt = G.gpu_quantize(w_dev)
    del w_dev
    got = gpu_merge(qt, G.dev_bf16(A), G.dev_bf16(B), r, alpha, "bf16")
    rows = np.sort(np.random.default_rng(layer).choice(N, 96, replace=False))
    so = G.SampledOracle(W32)
    W_hat_rows = so._blocks(rows, 0, K // 64)
    ref = merge.merge(W_hat_rows, A, B[rows], alpha, r, "bf16")
    compare(got[rows], ref, "bf16", f"7b layer {layer} rows")
