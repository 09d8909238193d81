"""GPU parity of the fp16 compute format (qlora_linear_fwd_ex /
qlora_linear_bwd_ex with QLORA_F16, fp16 dequantization) against the oracle:
the dequantized fp16 weight bit-exact; Y, dX, dA and dB within the relative
Frobenius bars of the bf16 path (2e-3 for 16-bit outputs, 1e-4 for fp32
outputs) of the oracle's fp64 references built from the same fp16 inputs and
the oracle's fp16 Ŵ.  Inputs: the workloads' seeded draws, rounded to fp16."""

import numpy as np
import pytest

from oracle import linalg, nf4
from tests import gpu_util as G
from workloads import Inputs

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def to_f16(bf16_bits):
    """The workloads' bf16 values rounded into fp16 (exact where in range)."""
    return nf4.f16_bits(nf4.bf16_to_f32(bf16_bits))


def dev_f16(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(t.float16).cuda()


def f64(bits):
    return nf4.f16_to_f32(bits).astype(np.float64)


def w_hat_f16(qt_ref, shape):
    return f64(nf4.dequantize(qt_ref["codes"], qt_ref["absmax_e4m3"], qt_ref["dq_scale"], qt_ref["dq_mean"],
                              fmt16="f16")).reshape(shape)


def gpu_dequantize_f16(qt):
    import quantized_fine_tuning_amd as q
    t = torch()
    out = t.empty(qt.n_rows, qt.n_cols, dtype=t.float16, device="cuda")
    q.qlora_dequantize(qt, out)
    return out.view(t.int16).cpu().numpy().view(np.uint16).reshape(-1)


def run_layer(W32, X, A, B, dY, r, alpha, rows=None):
    """fwd and bwd in fp16 on the device against the oracle (fp16 inputs)."""
    t = torch()
    qt = G.gpu_quantize(G.dev_f32(W32))
    ref = nf4.quantize(W32)
    bits = nf4.dequantize(ref["codes"], ref["absmax_e4m3"], ref["dq_scale"], ref["dq_mean"], fmt16="f16")
    assert np.array_equal(gpu_dequantize_f16(qt), bits), "fp16 dequantized weight"
    W_hat = f64(bits).reshape(W32.shape)
    Xd, Ad, Bd, dYd = dev_f16(X), dev_f16(A), dev_f16(B), dev_f16(dY)
    Yh, T = G.gpu_forward(qt, Xd, Ad, Bd, r, alpha, t.float16)
    Yf, _ = G.gpu_forward(qt, Xd, Ad, Bd, r, alpha, t.float32, save_T=False)
    Y_ref, T_ref = linalg.linear_fwd(f64(X), W_hat, f64(A), f64(B), alpha, r)
    e1 = G.assert_close(G.out_f64(Yh), Y_ref, G.TOL_BF16, "Y fp16")
    e2 = G.assert_close(G.out_f64(Yf), Y_ref, G.TOL_F32, "Y fp32")
    G.assert_close(G.out_f64(T), T_ref, G.TOL_F32, "T")
    dXh, dA, dB = G.gpu_backward(qt, Xd, dYd, Ad, Bd, r, alpha, T, t.float16)
    dXf, dA2, dB2 = G.gpu_backward(qt, Xd, dYd, Ad, Bd, r, alpha, None, t.float32)
    dX_ref, dA_ref, dB_ref = linalg.linear_bwd(f64(X), f64(dY), W_hat, f64(A), f64(B), alpha, r)
    e3 = G.assert_close(G.out_f64(dXh), dX_ref, G.TOL_BF16, "dX fp16")
    e4 = G.assert_close(G.out_f64(dXf), dX_ref, G.TOL_F32, "dX fp32")
    e5 = G.assert_close(G.out_f64(dA), dA_ref, G.TOL_F32, "dA")
    e6 = G.assert_close(G.out_f64(dB), dB_ref, G.TOL_F32, "dB")
    G.assert_close(G.out_f64(dA2), dA_ref, G.TOL_F32, "dA (T recomputed)")
    G.assert_close(G.out_f64(dB2), dB_ref, G.TOL_F32, "dB (T recomputed)")
    print(f"  Y fp16 {e1:.2e} fp32 {e2:.2e}  dX fp16 {e3:.2e} fp32 {e4:.2e}  dA {e5:.2e}  dB {e6:.2e}",
          flush=True)


def test_tiny_layer_fp16():
    w = Inputs(1)
    W32 = w.weight(0)
    M = 32
    print("fp16 tiny layer", flush=True)
    run_layer(W32, to_f16(w.X(0, M)), to_f16(w.lora_A(0)), to_f16(w.lora_B(0)), to_f16(w.dY(0, M)),
              w.w.rank, w.w.alpha)


# the last two split the GEMMs' reductions (forward 4 and 8 splits, dX 2 and
# 4), the last with a ragged weight row count
@pytest.mark.parametrize("M, N, K, r", [(100, 200, 320, 7), (300, 264, 576, 40), (17, 72, 64, 96),
                                        (100, 1024, 2048, 16), (40, 2056, 4096, 8),
                                        (2100, 5400, 256, 8),  # 512 x 128 forward tiles
                                        (1024, 1000, 1024, 8)])  # the same with a split reduction
def test_ragged_shapes_fp16(M, N, K, r):
    print(f"fp16 ragged M={M} N={N} K={K} r={r}", flush=True)
    rng = np.random.default_rng(M + N + K + r)
    W32 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    h = lambda a: nf4.f16_bits(a.astype(np.float32))  # noqa: E731
    run_layer(W32, h(rng.standard_normal((M, K))), h(rng.standard_normal((r, K)) * 0.02),
              h(rng.standard_normal((N, r)) * 0.01), h(rng.standard_normal((M, N))), r, 2.0 * r)


@pytest.mark.parametrize("M", [1, 3])
def test_gemv_narrow_workgroups_fp16(M):
    # the narrow GEMV workgroups (257 row groups) in fp16: 4 waves at M = 1
    # (X within 8 KB), 8 at M = 3 (within 32 KB); ragged last row group and
    # block groups (K = 2368: 37 blocks)
    t = torch()
    N, K, r = 4104, 2368, 12
    print(f"fp16 narrow GEMV N={N} K={K} M={M}", flush=True)
    rng = np.random.default_rng(N + K + M)
    W32 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    h = lambda a: nf4.f16_bits(a.astype(np.float32))  # noqa: E731
    X, A, B = h(rng.standard_normal((M, K))), h(rng.standard_normal((r, K)) * 0.02), h(rng.standard_normal((N, r)) * 0.01)
    qt = G.gpu_quantize(G.dev_f32(W32))
    W_hat = w_hat_f16(nf4.quantize(W32), W32.shape)
    Yh, _ = G.gpu_forward(qt, dev_f16(X), dev_f16(A), dev_f16(B), r, 2.0 * r, t.float16)
    Yf, _ = G.gpu_forward(qt, dev_f16(X), dev_f16(A), dev_f16(B), r, 2.0 * r, t.float32)
    Y_ref, _ = linalg.linear_fwd(f64(X), W_hat, f64(A), f64(B), 2.0 * r, r)
    e2 = G.assert_close(G.out_f64(Yf), Y_ref, G.TOL_F32, "Y fp32")
    e1 = G.assert_close(G.out_f64(Yh), Y_ref, G.TOL_BF16, "Y fp16")
    print(f"  Y fp16 {e1:.2e} fp32 {e2:.2e}", flush=True)


@pytest.mark.parametrize("M", [1, 16])
def test_qproj_gemv_fp16(M):
    # the dequant-GEMV path (M <= 16) in fp16 on the 4096 x 4096 q_proj weight
    t = torch()
    w = Inputs(2)
    W32 = w.weight(0)
    r, alpha = w.w.rank, w.w.alpha
    print(f"fp16 q_proj GEMV M={M}", flush=True)
    qt = G.gpu_quantize(G.dev_f32(W32))
    ref = nf4.quantize(W32)
    W_hat = w_hat_f16(ref, W32.shape)
    X, A, B = to_f16(w.X(0, M)), to_f16(w.lora_A(0)), to_f16(w.lora_B(0))
    Yh, _ = G.gpu_forward(qt, dev_f16(X), dev_f16(A), dev_f16(B), r, alpha, t.float16)
    Yf, _ = G.gpu_forward(qt, dev_f16(X), dev_f16(A), dev_f16(B), r, alpha, t.float32)
    Y_ref, _ = linalg.linear_fwd(f64(X), W_hat, f64(A), f64(B), alpha, r)
    e2 = G.assert_close(G.out_f64(Yf), Y_ref, G.TOL_F32, "Y fp32")
    e1 = G.assert_close(G.out_f64(Yh), Y_ref, G.TOL_BF16, "Y fp16")
    print(f"  Y fp16 {e1:.2e} fp32 {e2:.2e}", flush=True)


def test_mlp_7b_down_full_size_sampled_fp16():
    # the 7B MLP's down projection (4096 x 11008) at M = 4096 in fp16, in the
    # launch configuration the benchmark times; the oracle on sampled rows
    t = torch()
    w = Inputs(3)
    li = 2
    W32 = w.weight(li)
    N, K = W32.shape
    M, r, alpha = 4096, w.w.rank, w.w.alpha
    print(f"fp16 7b down {N}x{K} M={M}", flush=True)
    qt = G.gpu_quantize(G.dev_f32(W32))
    X, A, B, dY = to_f16(w.X(li, M)), to_f16(w.lora_A(li)), to_f16(w.lora_B(li)), to_f16(w.dY(li, M))
    Xd, Ad, Bd, dYd = dev_f16(X), dev_f16(A), dev_f16(B), dev_f16(dY)
    Yh, T = G.gpu_forward(qt, Xd, Ad, Bd, r, alpha, t.float16)
    dXh, dA, dB = G.gpu_backward(qt, Xd, dYd, Ad, Bd, r, alpha, T, t.float16)
    so = G.SampledOracle(W32)
    rng = np.random.default_rng(5)
    tok = np.sort(rng.choice(M, 32, replace=False))
    wrows = np.sort(rng.choice(N, 128, replace=False))
    kpr = K // 64

    def w_hat(rows, kb0, kb1):
        # Ŵ[rows, 64 kb0 : 64 kb1] in fp16: the same fp32 products rounded
        # into binary16 (blocks dequantize independently; the mean and group
        # scales are the whole tensor's)
        codes, _ = nf4.quantize_codes(W32[rows][:, 64 * kb0:64 * kb1])
        ids = (rows[:, None] * kpr + np.arange(kb0, kb1)[None, :]).reshape(-1)
        return f64(nf4.dequantize_blocks(codes.reshape(-1, 64), ids, so.e, so.s, so.mu, fmt16="f16")).reshape(
            len(rows), 64 * (kb1 - kb0))

    Y_ref, _ = linalg.linear_fwd(f64(X[tok]), w_hat(wrows, 0, kpr), f64(A), f64(B[wrows]), alpha, r)
    e1 = G.assert_close(G.out_f64(Yh)[np.ix_(tok, wrows)], Y_ref, G.TOL_BF16, "Y fp16")
    kb = 37
    cols = np.arange(64 * kb, 64 * kb + 64)
    dX_ref = linalg.linear_dx(f64(dY[tok]), w_hat(np.arange(N), kb, kb + 1), f64(A)[:, cols], f64(B), alpha, r)
    e4 = G.assert_close(G.out_f64(dXh)[np.ix_(tok, cols)], dX_ref, G.TOL_BF16, "dX fp16")
    dA_ref, dB_ref = linalg.lora_grads(f64(X), f64(dY), f64(A), f64(B), alpha, r)
    e2 = G.assert_close(G.out_f64(dA), dA_ref, G.TOL_F32, "dA")
    e3 = G.assert_close(G.out_f64(dB), dB_ref, G.TOL_F32, "dB")
    print(f"  Y fp16 {e1:.2e}  dX fp16 {e4:.2e}  dA {e2:.2e}  dB {e3:.2e}", flush=True)
