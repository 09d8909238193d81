"""Save and reload of a quantized weight: the four arrays of one NF4 + double
quantized tensor (codes, E4M3 constants, group scales, mean) written to a
safetensors file, read back into fresh device memory, give the same bytes and
a bit-identical forward output (P2 §四: the 4-bit base is stored once and
reused; nothing else is needed to rebuild Ŵ)."""

import pytest

from tests import gpu_util as G
from workloads import Inputs

pytestmark = pytest.mark.gpu


def test_quantized_weight_round_trips_through_a_file(tmp_path):
    import torch as t
    from safetensors.torch import load_file, save_file

    import quantized_fine_tuning_amd as q
    w = Inputs(3)
    _, N, K = w.w.layers[2]
    r, alpha, M = w.w.rank, w.w.alpha, 300
    qt = G.gpu_quantize(G.dev_f32(w.weight(2)))
    path = tmp_path / "down_nf4.safetensors"
    save_file({"codes": qt.codes.cpu(), "absmax_e4m3": qt.absmax_e4m3.cpu(), "dq_scale": qt.dq_scale.cpu(),
               "dq_mean": qt.dq_mean.cpu()}, str(path), metadata={"n_rows": str(N), "n_cols": str(K)})
    d = load_file(str(path))
    back = q.Nf4Tensor(N, K, *(d[k].cuda() for k in ("codes", "absmax_e4m3", "dq_scale", "dq_mean")))
    for name in ("codes", "absmax_e4m3", "dq_scale", "dq_mean"):
        a, b = getattr(qt, name), getattr(back, name)
        assert t.equal(a.view(t.uint8), b.view(t.uint8)), name
    X, A, B = G.dev_bf16(w.X(2, M)), G.dev_bf16(w.lora_A(2)), G.dev_bf16(w.lora_B(2))
    Y1, T1 = G.gpu_forward(qt, X, A, B, r, alpha, t.bfloat16)
    Y2, T2 = G.gpu_forward(back, X, A, B, r, alpha, t.bfloat16)
    assert t.equal(Y1.view(t.int16), Y2.view(t.int16)) and t.equal(T1, T2)
    assert t.equal(G.gpu_dequantize(qt).view(t.int16), G.gpu_dequantize(back).view(t.int16))
