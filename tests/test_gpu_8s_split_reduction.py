"""Parity of the GEMMs' split reduction (few tokens: the output tiles alone
would leave most compute units idle, so each tile's reduction is split over
several workgroups whose fp32 partials a second kernel sums in split order).

1. Every element of Y, dX, dA and dB of the 7B MLP linears at token counts
   where the forward and/or the dX product split (gate 11008x4096: forward
   5 splits up to 256 tokens, 2 up to 512; dX 16 and 8; down 4096x11008:
   forward 16 and 8, dX 5 and 2), against the oracle's fp64
   result with the per-element rounding bound of the full-size test; M <= 16
   runs the dequant-GEMV forward and the split dX product.
2. One-hot pins with B = 0 at 256 tokens: every token row is one-hot at a
   column chosen so that, over the calls, every reduction index of every
   split is hit once; each output is one exact product, so Y (forward) and
   dX equal slices of the oracle's Ŵ bit for bit.

P1 "QLoRA 的原理是什么？" §七 (分清存储精度与计算精度): the 4-bit weight is
dequantized to BF16 before the matmul, whatever the launch shape.
"""

import numpy as np
import pytest

from tests import gpu_util as G
from tests.test_gpu_8_fullsize import canon_zero, compare_every_element, oracle_w_hat_bits
from workloads import Inputs

pytestmark = pytest.mark.gpu


# The GEMV's X staging: (0, 1) 8 KB, (2, 1) 22 KB, (2, 5) 110 KB staged (the
# adapter term's arrays then take X's place after the main loop), (2, 16)
# 352 KB not staged; (2, *) with 43 partial slices of T, summed after the
# main loop (at most 16 are summed from registers)
@pytest.mark.parametrize("layer,M", [(0, 1), (0, 17), (0, 130), (0, 300), (2, 1), (2, 5), (2, 16), (2, 64),
                                     (2, 100), (1, 256)])
def test_split_reduction_every_element(layer, M):
    compare_every_element(layer, M)


@pytest.mark.parametrize("layer", [0, 2])
def test_split_reduction_one_hot_pins(layer):
    import torch as t

    import quantized_fine_tuning_amd as q
    w = Inputs(3)
    name, N, K = w.w.layers[layer]
    r, alpha = w.w.rank, w.w.alpha
    M = 256
    print(f"split one-hot pins {name} {N}x{K} M={M}", flush=True)
    W32 = w.weight(layer)
    qt = G.gpu_quantize(G.dev_f32(W32))
    w_hat = canon_zero(oracle_w_hat_bits(W32))
    A = G.dev_bf16(w.lora_A(layer))
    B0 = t.zeros(N, r, dtype=t.bfloat16, device="cuda")
    sz = q.qlora_nf4_sizes(N, K, M, r)
    wsf, wsb = q.workspace(sz["fwd_ws_bytes"]), q.workspace(sz["bwd_ws_bytes"])
    # forward: call c, row m one-hot at k = c + (K / M) m (the K / M calls
    # cover every k once, spread over every split's range of K)
    calls = K // M
    Y = t.empty(M, N, dtype=t.bfloat16, device="cuda")
    bad = 0
    for c in range(calls):
        ks = c + calls * np.arange(M)
        X = t.zeros(M, K, dtype=t.bfloat16, device="cuda")
        X[t.arange(M, device="cuda"), t.from_numpy(ks).cuda()] = 1.0
        q.qlora_linear_fwd(qt, X, A, B0, r, alpha, Y, None, wsf)
        bad += int(np.count_nonzero(canon_zero(G.host_bf16(Y)) != w_hat[:, ks].T))
    print(f"  forward: {bad} of {calls * M * N} outputs differ", flush=True)
    assert bad == 0
    # dX: call c, row m one-hot at n = c + ceil(N / M) m (n < N), dX = Ŵ rows
    step = -(-N // M)
    dX = t.empty(M, K, dtype=t.bfloat16, device="cuda")
    dA = t.empty(r, K, dtype=t.float32, device="cuda")
    dB = t.empty(N, r, dtype=t.float32, device="cuda")
    Xb = t.zeros(M, K, dtype=t.bfloat16, device="cuda")
    bad = total = 0
    for c in range(step):
        ns = c + step * np.arange(M)
        ok = ns < N
        dY = t.zeros(M, N, dtype=t.bfloat16, device="cuda")
        rows = np.nonzero(ok)[0]
        dY[t.from_numpy(rows).cuda(), t.from_numpy(ns[ok]).cuda()] = 1.0
        q.qlora_linear_bwd(qt, Xb, dY, A, B0, r, alpha, None, dX, dA, dB, wsb)
        got = canon_zero(G.host_bf16(dX))
        bad += int(np.count_nonzero(got[rows] != w_hat[ns[ok]]))
        bad += int(np.count_nonzero(got[~ok] != 0))
        total += got.size
    print(f"  dX: {bad} of {total} outputs differ", flush=True)
    assert bad == 0
