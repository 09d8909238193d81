"""qlora_linear_fwd_noalloc (the forward for callers that cannot allocate:
its scratch is the library's static per-GPU array) against qlora_linear_fwd
with a caller workspace, through the C ABI: identical bytes of Y and T on
consecutive calls that shrink, so the second call reuses the array that the
first one left filled (GEMM path at the 7B gate shape, a smaller ragged GEMM,
then the M <= 16 GEMV path), with and without a saved T."""

import pytest

from tests import gpu_util as G
from workloads import Inputs

pytestmark = pytest.mark.gpu


def test_noalloc_forward_matches_the_workspace_forward():
    import torch as t

    import quantized_fine_tuning_amd as q
    w = Inputs(3)
    name, N, K = w.w.layers[0]
    r, alpha = w.w.rank, w.w.alpha
    qt = G.gpu_quantize(G.dev_f32(w.weight(0)))
    A, B = G.dev_bf16(w.lora_A(0)), G.dev_bf16(w.lora_B(0))
    for M, y_dtype, save_T in ((4096, t.bfloat16, True), (300, t.bfloat16, True), (5, t.float32, True),
                               (1, t.bfloat16, False), (130, t.float32, False)):
        print(f"noalloc forward {name} {N}x{K} M={M} y={y_dtype} T saved={save_T}", flush=True)
        X = G.dev_bf16(w.X(0, M))
        ws = q.workspace(q.qlora_nf4_sizes(N, K, M, r)["fwd_ws_bytes"])
        Y_ref = t.empty(M, N, dtype=y_dtype, device="cuda")
        T_ref = t.empty(M, r, dtype=t.float32, device="cuda") if save_T else None
        q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y_ref, T_ref, ws)
        Y = t.full((M, N), float("nan"), dtype=y_dtype, device="cuda")
        T = t.full((M, r), float("nan"), dtype=t.float32, device="cuda") if save_T else None
        q.qlora_linear_fwd_noalloc(qt, X, A, B, r, alpha, Y, T)
        t.cuda.synchronize()
        assert t.equal(Y.view(t.int16) if y_dtype == t.bfloat16 else Y.view(t.int32),
                       Y_ref.view(t.int16) if y_dtype == t.bfloat16 else Y_ref.view(t.int32))
        if save_T:
            assert t.equal(T.view(t.int32), T_ref.view(t.int32))


def test_noalloc_forward_with_fewer_splits_than_the_workspace_forward():
    """7B gate at 512 tokens: the workspace forward splits the GEMM's
    reduction in two (partials of 45 MB), the no-alloc forward keeps one
    split to fit its 32 MiB array.  The sums run in another order, so the
    fp32 outputs agree to fp32 rounding, not byte for byte; T (computed
    before the GEMM, the same way) is byte-identical."""
    import torch as t

    import quantized_fine_tuning_amd as q
    w = Inputs(3)
    name, N, K = w.w.layers[0]
    r, alpha = w.w.rank, w.w.alpha
    M = 512
    qt = G.gpu_quantize(G.dev_f32(w.weight(0)))
    A, B = G.dev_bf16(w.lora_A(0)), G.dev_bf16(w.lora_B(0))
    X = G.dev_bf16(w.X(0, M))
    print(f"noalloc forward {name} {N}x{K} M={M}: fewer splits", flush=True)
    assert q.qlora_nf4_sizes(N, K, M, r)["fwd_ws_bytes"] > 32 << 20
    ws = q.workspace(q.qlora_nf4_sizes(N, K, M, r)["fwd_ws_bytes"])
    Y_ref = t.empty(M, N, dtype=t.float32, device="cuda")
    T_ref = t.empty(M, r, dtype=t.float32, device="cuda")
    q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y_ref, T_ref, ws)
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    T = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    q.qlora_linear_fwd_noalloc(qt, X, A, B, r, alpha, Y, T)
    t.cuda.synchronize()
    assert t.equal(T.view(t.int32), T_ref.view(t.int32))
    assert bool(t.isfinite(Y).all())
    rel = float((Y.double() - Y_ref.double()).norm() / Y_ref.double().norm())
    print(f"  relative Frobenius difference {rel:.2e}", flush=True)
    assert rel <= 1e-5
