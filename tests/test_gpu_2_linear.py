"""GPU parity of the QLoRA linear forward and backward against the oracle's
fp64 references on the same seeded inputs (relative Frobenius error <= 2e-3
for bf16 outputs, 1e-4 for fp32 outputs), plus bit-exact identity cases that
pin the in-tile dequantization.  Every call goes through the C ABI."""

import numpy as np
import pytest

from oracle import linalg, nf4
from tests import gpu_util as G
from workloads import Inputs, random_bf16, random_f32

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


class Layer:
    """One layer's inputs on host and device plus the oracle's Ŵ."""

    def __init__(self, W32, X, A, B, dY=None, w_dev=None):
        self.W32, self.X, self.A, self.B, self.dY = W32, X, A, B, dY
        self.qt = G.gpu_quantize(w_dev if w_dev is not None else G.dev_f32(W32))
        self.ref = nf4.quantize(W32)
        self.W_hat = G.bf16_f64(G.oracle_w_hat(self.ref)).reshape(W32.shape)
        self.Xd, self.Ad, self.Bd = G.dev_bf16(X), G.dev_bf16(A), G.dev_bf16(B)
        self.dYd = G.dev_bf16(dY) if dY is not None else None

    @classmethod
    def from_workload(cls, idx, layer, M):
        w = Inputs(idx)
        Wst = w.weight(layer)
        dY = w.dY(layer, M) if w.w.backward else None
        if w.w.weight_dtype == "bf16":
            W32 = (Wst.astype(np.uint32) << 16).view(np.float32)
            return cls(W32, w.X(layer, M), w.lora_A(layer), w.lora_B(layer), dY, G.dev_bf16(Wst))
        return cls(Wst, w.X(layer, M), w.lora_A(layer), w.lora_B(layer), dY)


def run_fwd(L, r, alpha, rows=None):
    t = torch()
    Yb, T = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, r, alpha, t.bfloat16)
    Yf, _ = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, r, alpha, t.float32, save_T=False)
    Xs = G.bf16_f64(L.X) if rows is None else G.bf16_f64(L.X[rows])
    Y_ref, T_ref = linalg.linear_fwd(Xs, L.W_hat, G.bf16_f64(L.A), G.bf16_f64(L.B), alpha, r)
    yb, yf, tt = G.out_f64(Yb), G.out_f64(Yf), G.out_f64(T)
    if rows is not None:
        yb, yf, tt = yb[rows], yf[rows], tt[rows]
    eb = G.assert_close(yb, Y_ref, G.TOL_BF16, "Y bf16")
    ef = G.assert_close(yf, Y_ref, G.TOL_F32, "Y fp32")
    et = G.assert_close(tt, T_ref, G.TOL_F32, "T")
    print(f"  Y bf16 {eb:.2e}  Y fp32 {ef:.2e}  T {et:.2e}", flush=True)
    return T


def run_bwd(L, r, alpha, T_saved, rows=None):
    t = torch()
    dXb, dA, dB = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, r, alpha, T_saved, t.bfloat16)
    dXf, dA2, dB2 = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, r, alpha, None, t.float32)
    X = G.bf16_f64(L.X)
    dY = G.bf16_f64(L.dY)
    A, B = G.bf16_f64(L.A), G.bf16_f64(L.B)
    if rows is None:
        dX_ref, dA_ref, dB_ref = linalg.linear_bwd(X, dY, L.W_hat, A, B, alpha, r)
        gx_b, gx_f = G.out_f64(dXb), G.out_f64(dXf)
    else:
        dX_ref, _, _ = linalg.linear_bwd(X[rows], dY[rows], L.W_hat, A, B, alpha, r)
        dA_ref, dB_ref = linalg.lora_grads(X, dY, A, B, alpha, r)
        gx_b, gx_f = G.out_f64(dXb)[rows], G.out_f64(dXf)[rows]
    e1 = G.assert_close(gx_b, dX_ref, G.TOL_BF16, "dX bf16")
    e2 = G.assert_close(gx_f, dX_ref, G.TOL_F32, "dX fp32")
    e3 = G.assert_close(G.out_f64(dA), dA_ref, G.TOL_F32, "dA")
    e4 = G.assert_close(G.out_f64(dB), dB_ref, G.TOL_F32, "dB")
    G.assert_close(G.out_f64(dA2), dA_ref, G.TOL_F32, "dA (T recomputed)")
    G.assert_close(G.out_f64(dB2), dB_ref, G.TOL_F32, "dB (T recomputed)")
    print(f"  dX bf16 {e1:.2e}  dX fp32 {e2:.2e}  dA {e3:.2e}  dB {e4:.2e}", flush=True)


def test_tiny_layer_fwd_bwd():
    w = Inputs(1)
    print("tiny 256x256 M=32 r=8", flush=True)
    L = Layer.from_workload(1, 0, 32)
    T = run_fwd(L, w.w.rank, w.w.alpha)
    run_bwd(L, w.w.rank, w.w.alpha, T)


def test_identity_input_gives_weight_bit_exact():
    # X = I and B = 0: every output is one exact product, so Y = Ŵᵀ bit for bit
    t = torch()
    w = Inputs(1)
    W = w.weight(0)
    eye = np.eye(256, dtype=np.float32)
    from workloads import to_bf16_bits
    L = Layer(W, to_bf16_bits(eye), w.lora_A(0), np.zeros((256, 8), np.uint16),
              dY=to_bf16_bits(eye))
    Y, _ = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, 8, 16.0, t.bfloat16)
    w_hat_bits = G.oracle_w_hat(L.ref).reshape(256, 256)
    assert np.array_equal(G.host_bf16(Y), w_hat_bits.T)
    # dY = I and B = 0: dX = Ŵ bit for bit
    dX, dA, dB = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, 8, 16.0, None, t.bfloat16)
    assert np.array_equal(G.host_bf16(dX), w_hat_bits)
    assert np.all(G.host(dA) == 0)


@pytest.mark.parametrize("M,r", [(1, 12), (3, 12), (1, 128), (1, 256)])
def test_gemv_narrow_workgroups(M, r):
    # more 16-row groups than compute units (N = 4104: 257 groups): 4-wave
    # workgroups with X within 8 KB and r <= 128 (M = 1), else 8-wave ones
    # with X within 32 KB (M = 3, and r = 256, whose B rows need 512
    # threads to stage); K = 2368 is 37 blocks, 10 block groups per row (the
    # last of one block), so the waves sum two or three each
    N, K = 4104, 2368
    print(f"narrow GEMV N={N} K={K} M={M} r={r}", flush=True)
    W = random_f32((N, K), seed=41 + M, scale=0.02)
    L = Layer(W, random_bf16((M, K), seed=42 + M), random_bf16((r, K), seed=43, scale=0.02),
              random_bf16((N, r), seed=44, scale=0.01))
    run_fwd(L, r, 2.0 * r)


@pytest.mark.parametrize("rows", [6, 1])
def test_gemv_narrow_identity_bit_exact(rows):
    # one-hot rows of X and B = 0 through the 8-wave workgroups (6 rows per
    # call) and the 4-wave ones (one row per call): every output is one
    # exact product, Y[m][n] = Ŵ[n][k_m]
    t = torch()
    N, K = 4104, 2368
    W = random_f32((N, K), seed=45, scale=0.02)
    ks = [0, 63, 64, 1000, 2303, 2367]
    from workloads import to_bf16_bits
    X = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    L = Layer(W, to_bf16_bits(X), random_bf16((4, K), seed=46, scale=0.02), np.zeros((N, 4), np.uint16))
    w_hat_bits = G.oracle_w_hat(L.ref).reshape(N, K)
    for i0 in range(0, len(ks), rows):
        Y, _ = G.gpu_forward(L.qt, L.Xd[i0:i0 + rows], L.Ad, L.Bd, 4, 8.0, t.bfloat16)
        assert np.array_equal(G.host_bf16(Y), w_hat_bits[:, ks[i0:i0 + rows]].T)


def test_qproj_gemv_m1_m16():
    w = Inputs(2)
    for M in (1, 3, 4, 5, 16):  # X staged 2 pieces a thread up to M = 4, 8 above
        print(f"q_proj 4096x4096 M={M} r=16", flush=True)
        L = Layer.from_workload(2, 0, M)
        run_fwd(L, w.w.rank, w.w.alpha)


@pytest.mark.parametrize("M,N,K,r", [
    (33, 200, 192, 5),     # ragged M, N, odd rank
    (17, 256, 256, 8),     # just above the GEMV threshold
    (5, 136, 320, 3),      # GEMV with ragged N
    (300, 520, 640, 256),  # maximum rank
    (64, 64, 64, 1),
    (3, 136, 320, 3),      # small-M GEMV, 5 blocks per row (a ragged block group)
    (1, 200, 192, 5),
    (4, 24, 64, 1),
    (2100, 5400, 256, 8),  # 512 x 128 forward tiles, ragged in both directions
    (1024, 1000, 1024, 8),  # 512 x 128 forward tiles with a 2-way split reduction
    (1536, 200, 192, 5),   # 512 x 128 forward tiles, rank padded to 32 (one LoRA step)
    (2048, 520, 320, 40),  # 512 x 128 forward tiles, rank padded to 64 (two LoRA steps)
    (5, 136, 8192, 16),    # GEMV, T from 16 slices of 512 (65B q_proj width)
    (2, 264, 22016, 8),    # GEMV, T from 22 slices of 1024, summed in the epilogue
])
def test_ragged_shapes(M, N, K, r):
    print(f"ragged M={M} N={N} K={K} r={r}", flush=True)
    W = random_f32((N, K), seed=M * 7 + N, scale=0.02)
    L = Layer(W, random_bf16((M, K), seed=N + 1), random_bf16((r, K), seed=N + 2, scale=0.02),
              random_bf16((N, r), seed=N + 3, scale=0.01), dY=random_bf16((M, N), seed=N + 4))
    T = run_fwd(L, r, 2.0 * r)
    run_bwd(L, r, 2.0 * r, T)


def test_zero_tokens():
    t = torch()
    W = random_f32((64, 128), seed=3, scale=0.02)
    L = Layer(W, np.zeros((0, 128), np.uint16), random_bf16((4, 128), seed=4),
              random_bf16((64, 4), seed=5), dY=np.zeros((0, 64), np.uint16))
    dX, dA, dB = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, 4, 8.0, None, t.bfloat16)
    assert dX.numel() == 0
    assert np.all(G.host(dA) == 0) and np.all(G.host(dB) == 0)
    Y, _ = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, 4, 8.0, t.bfloat16)
    assert Y.numel() == 0


class BigLayer:
    """A full-size layer on the device; the oracle works on samples of it."""

    def __init__(self, idx, layer, M):
        w = Inputs(idx)
        self.r, self.alpha = w.w.rank, w.w.alpha
        Wst = w.weight(layer)
        if w.w.weight_dtype == "bf16":
            self.W32 = (Wst.astype(np.uint32) << 16).view(np.float32)
            w_dev = G.dev_bf16(Wst)
        else:
            self.W32 = Wst
            w_dev = G.dev_f32(Wst)
        self.qt = G.gpu_quantize(w_dev)
        del w_dev
        self.X, self.A, self.B, self.dY = w.X(layer, M), w.lora_A(layer), w.lora_B(layer), w.dY(layer, M)
        self.Xd, self.Ad, self.Bd, self.dYd = (G.dev_bf16(a) for a in (self.X, self.A, self.B, self.dY))
        self.oracle = G.SampledOracle(self.W32)


def run_big(L, seed, n_tok=32, n_rows=256):
    """Y on sampled (token, weight-row) pairs, dX on sampled (token, 64-column
    stripe) pairs, dA and dB in full; bf16 and fp32 outputs.  The samples
    cover every output tile of both GEMMs: at least one token in every
    256-token tile, one weight row in every 256-row tile (Y) and one 64-column
    stripe in every 256-column tile (dX)."""
    t = torch()
    rng = np.random.default_rng(seed)
    M = L.X.shape[0]
    N, K = L.W32.shape
    r, alpha = L.r, L.alpha

    def cover(n, tile, extra):
        per_tile = [int(rng.integers(i, min(i + tile, n))) for i in range(0, n, tile)]
        more = rng.choice(n, min(extra, n), replace=False)
        return np.unique(np.concatenate([per_tile, more]))

    tok = cover(M, 256, n_tok)
    wrows = cover(N, 256, n_rows)
    stripes = np.array([int(rng.integers(4 * i, min(4 * i + 4, K // 64))) for i in range((K // 64 + 3) // 4)])
    Yb, T = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, r, alpha, t.bfloat16)
    Yf, _ = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, r, alpha, t.float32, save_T=False)
    X, A, B, dY = (G.bf16_f64(a) for a in (L.X, L.A, L.B, L.dY))
    Y_ref, _ = linalg.linear_fwd(X[tok], L.oracle.rows(wrows), A, B[wrows], alpha, r)
    e1 = G.assert_close(G.out_f64(Yb)[np.ix_(tok, wrows)], Y_ref, G.TOL_BF16, "Y bf16")
    e2 = G.assert_close(G.out_f64(Yf)[np.ix_(tok, wrows)], Y_ref, G.TOL_F32, "Y fp32")
    dXb, dA, dB = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, r, alpha, T, t.bfloat16)
    dXf, _, _ = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, r, alpha, None, t.float32)
    cols = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in stripes])
    w_cols = np.concatenate([L.oracle.cols(b, b + 1) for b in stripes], axis=1)
    dX_ref = linalg.linear_dx(dY[tok], w_cols, A[:, cols], B, alpha, r)
    e3 = G.assert_close(G.out_f64(dXb)[np.ix_(tok, cols)], dX_ref, G.TOL_BF16, "dX bf16")
    e4 = G.assert_close(G.out_f64(dXf)[np.ix_(tok, cols)], dX_ref, G.TOL_F32, "dX fp32")
    dA_ref, dB_ref = linalg.lora_grads(X, dY, A, B, alpha, r)
    e5 = G.assert_close(G.out_f64(dA), dA_ref, G.TOL_F32, "dA")
    e6 = G.assert_close(G.out_f64(dB), dB_ref, G.TOL_F32, "dB")
    print(f"  Y bf16 {e1:.2e} fp32 {e2:.2e}  dX bf16 {e3:.2e} fp32 {e4:.2e}  "
          f"dA {e5:.2e}  dB {e6:.2e}", flush=True)


@pytest.mark.parametrize("idx,layer,M", [(4, 0, 8192), (4, 6, 8192), (5, 0, 2048), (5, 4, 2048)])
def test_bf16_weight_layers_sampled(idx, layer, M):
    w = Inputs(idx)
    print(f"workload {idx} {w.w.layers[layer]} M={M}", flush=True)
    run_big(BigLayer(idx, layer, M), seed=100 + layer)


def test_forward_backward_deterministic():
    t = torch()
    L = Layer.from_workload(1, 0, 32)
    y1, T1 = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, 8, 16.0, t.bfloat16)
    y2, T2 = G.gpu_forward(L.qt, L.Xd, L.Ad, L.Bd, 8, 16.0, t.bfloat16)
    assert t.equal(y1, y2) and t.equal(T1, T2)
    g1 = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, 8, 16.0, T1, t.bfloat16)
    g2 = G.gpu_backward(L.qt, L.Xd, L.dYd, L.Ad, L.Bd, 8, 16.0, T1, t.bfloat16)
    for a, b in zip(g1, g2):
        assert t.equal(a, b)
