"""The library's calls under HIP graph capture: a forward + backward of the
GEMM path (M = 96) and a dequant-GEMV forward (M = 4) are captured into one
graph (torch.cuda.graph) and replayed several times, with eager work and
output clobbering in between; every replay must reproduce the eager results
bit for bit (every kernel reduces in a fixed order, and the calls enqueue
kernels only: no memset, copy or synchronisation)."""

import numpy as np
import pytest

import quantized_fine_tuning_amd as q
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_fwd_bwd_and_gemv_replay_bit_exact():
    import torch

    rng = np.random.default_rng(21)
    N, K, r, alpha = 192, 320, 16, 32.0
    W = G.dev_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).cuda()  # noqa: E731
    X, dY = bf(rng.standard_normal((96, K))), bf(rng.standard_normal((96, N)))
    Xs = bf(rng.standard_normal((4, K)))
    A, B = bf(rng.standard_normal((r, K)) * 0.02), bf(rng.standard_normal((N, r)) * 0.01)
    qt = G.gpu_quantize(W)
    sz = q.qlora_nf4_sizes(N, K, 96, r)
    wsf, wsb = q.workspace(sz["fwd_ws_bytes"]), q.workspace(sz["bwd_ws_bytes"])
    wsg = q.workspace(q.qlora_nf4_sizes(N, K, 4, r)["fwd_ws_bytes"])
    out = {
        "Y": torch.empty(96, N, dtype=torch.bfloat16, device="cuda"),
        "T": torch.empty(96, r, dtype=torch.float32, device="cuda"),
        "dX": torch.empty(96, K, dtype=torch.bfloat16, device="cuda"),
        "dA": torch.empty(r, K, dtype=torch.float32, device="cuda"),
        "dB": torch.empty(N, r, dtype=torch.float32, device="cuda"),
        "Ys": torch.empty(4, N, dtype=torch.float32, device="cuda"),
        "Ts": torch.empty(4, r, dtype=torch.float32, device="cuda"),
    }

    def step():
        q.qlora_linear_fwd(qt, X, A, B, r, alpha, out["Y"], out["T"], wsf)
        q.qlora_linear_bwd(qt, X, dY, A, B, r, alpha, out["T"], out["dX"], out["dA"], out["dB"], wsb)
        q.qlora_linear_fwd(qt, Xs, A, B, r, alpha, out["Ys"], out["Ts"], wsg)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}

    # capture (warm-up on the capture stream first, as torch recommends)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        print(f"graph replay {rep}", flush=True)
        for v in out.values():
            v.fill_(float("nan"))  # eager work between replays
        other = torch.empty(96, N, dtype=torch.bfloat16, device="cuda")
        q.qlora_linear_fwd(qt, X, B.new_zeros(r, K), B, r, alpha, other, None, wsf)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            bits = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(v.view(bits), eager[k].view(bits)), f"replay {rep}: {k} differs from the eager result"
