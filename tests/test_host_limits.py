"""Host-side contracts of the C ABI and the binding, checked without a GPU:
workspace sizes that cover every smaller token count, the per-call limits of
the kernels' 32-bit buffer offsets, the static-scratch forward's size bound,
and the binding's shape and dtype checks (a mis-shaped tensor must raise
before any pointer reaches the library)."""

import ctypes
import re

import pytest
import torch

import quantized_fine_tuning_amd as q

FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def desc(n, k):
    return q.qlora_nf4_t(n, k, FAKE, FAKE, FAKE, FAKE)


def needed(call):
    """The exact workspace one call needs, read from the error the library
    gives for a zero-byte workspace (no HIP call is made)."""
    st = call()
    assert st == q.QLORA_ERR_WORKSPACE_TOO_SMALL, q.lib.qlora_last_error().decode()
    m = re.search(r"workspace 0 < (\d+) bytes", q.lib.qlora_last_error().decode())
    return int(m.group(1))


def fwd_need(N, K, M, r):
    d = desc(N, K)
    return needed(lambda: q.lib.qlora_linear_fwd(ctypes.byref(d), FAKE, M, FAKE, FAKE, r, 16.0, FAKE,
                                                 q.QLORA_BF16, None, FAKE, 0, None))


def bwd_need(N, K, M, r):
    d = desc(N, K)
    return needed(lambda: q.lib.qlora_linear_bwd(ctypes.byref(d), FAKE, FAKE, M, FAKE, FAKE, r, 16.0, None,
                                                 FAKE, q.QLORA_BF16, FAKE, FAKE, FAKE, 0, None))


@pytest.mark.parametrize("N,K,r,M_max", [(11008, 4096, 64, 2373), (4096, 4096, 16, 2373),
                                         (4096, 11008, 64, 1500), (520, 640, 256, 700)])
def test_sizes_cover_every_smaller_token_count(N, K, r, M_max):
    s = q.qlora_nf4_sizes(N, K, M_max, r)
    for M in list(range(17, M_max + 1, 7)) + [M_max]:
        assert fwd_need(N, K, M, r) <= s["fwd_ws_bytes"], M
    for M in list(range(1, M_max + 1, 11)) + [M_max]:
        assert bwd_need(N, K, M, r) <= s["bwd_ws_bytes"], M


@pytest.mark.parametrize("N,K,r", [(11008, 4096, 64), (4096, 11008, 64), (4096, 4096, 16)])
def test_sizes_cover_each_small_token_count(N, K, r):
    # sizes at M_max itself, for every M_max up to 300 (the GEMV forward, the
    # split reductions of both GEMMs)
    for M in range(1, 301):
        s = q.qlora_nf4_sizes(N, K, M, r)
        assert fwd_need(N, K, M, r) <= s["fwd_ws_bytes"], M
        assert bwd_need(N, K, M, r) <= s["bwd_ws_bytes"], M


def test_sizes_are_monotone_in_m_max():
    prev_f = prev_b = 0
    for M in range(0, 3000, 37):
        s = q.qlora_nf4_sizes(11008, 4096, M, 64)
        assert s["fwd_ws_bytes"] >= prev_f and s["bwd_ws_bytes"] >= prev_b
        prev_f, prev_b = s["fwd_ws_bytes"], s["bwd_ws_bytes"]


def test_large_token_counts_are_sized():
    # beyond 256 reduction tiles the size comes from the cmax <= 2 bound
    s = q.qlora_nf4_sizes(4096, 4096, 40000, 64)
    assert fwd_need(4096, 4096, 40000, 64) <= s["fwd_ws_bytes"]
    assert bwd_need(4096, 4096, 40000, 64) <= s["bwd_ws_bytes"]


@pytest.mark.parametrize("N,K,M,r", [
    (22016, 8192, 48800, 64),        # M * max(N, K) >= 2^30
    (4096, 11008, 97600, 64),
    (65536, 65536, 16, 8),           # N * K / 2 >= 2^31 code bytes
    (4096, 4096, (1 << 21) + 64, 256),  # transposed splits 2*Rp*Mp*2 >= 2^31
])
def test_linear_passes_reject_calls_beyond_32bit_offsets(N, K, M, r):
    d = desc(N, K)
    big = 1 << 40
    st = q.lib.qlora_linear_fwd(ctypes.byref(d), FAKE, M, FAKE, FAKE, r, 16.0, FAKE, q.QLORA_BF16, None,
                                FAKE, big, None)
    assert st == q.QLORA_ERR_INVALID_ARG and "limit" in q.lib.qlora_last_error().decode() or \
        "too large" in q.lib.qlora_last_error().decode()
    st = q.lib.qlora_linear_bwd(ctypes.byref(d), FAKE, FAKE, M, FAKE, FAKE, r, 16.0, None, FAKE,
                                q.QLORA_BF16, FAKE, FAKE, FAKE, big, None)
    assert st == q.QLORA_ERR_INVALID_ARG


def test_workload_shapes_are_within_the_limits():
    for N, K, M in ((11008, 4096, 8192), (4096, 11008, 8192), (22016, 8192, 2048), (8192, 22016, 2048)):
        d = desc(N, K)
        st = q.lib.qlora_linear_fwd(ctypes.byref(d), FAKE, M, FAKE, FAKE, 64, 16.0, FAKE, q.QLORA_BF16,
                                    None, FAKE, 0, None)
        assert st == q.QLORA_ERR_WORKSPACE_TOO_SMALL  # passed the limits, stopped at the workspace


def test_noalloc_forward_rejects_calls_beyond_its_scratch():
    f = q.lib.qlora_linear_fwd_noalloc
    # 65B gate at 48000 tokens needs more than the 32 MiB static scratch
    d = desc(22016, 8192)
    assert fwd_need(22016, 8192, 48000, 64) > 32 << 20
    st = f(ctypes.byref(d), FAKE, 48000, FAKE, FAKE, 64, 16.0, FAKE, q.QLORA_BF16, None, None)
    assert st == q.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch holds 33554432" in q.lib.qlora_last_error().decode()
    # argument errors come first, as in qlora_linear_fwd
    assert f(ctypes.byref(d), FAKE, 32, FAKE, FAKE, 0, 16.0, FAKE, q.QLORA_BF16, None, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert f(ctypes.byref(d), FAKE, 32, FAKE, FAKE, 8, 16.0, FAKE, q.QLORA_F16, None, None) == \
        q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert f(ctypes.byref(d), None, 32, FAKE, FAKE, 8, 16.0, FAKE, q.QLORA_BF16, None, None) == \
        q.QLORA_ERR_INVALID_ARG
    # every workload linear fits at its token count
    for N, K, M in ((11008, 4096, 8192), (4096, 11008, 8192), (22016, 8192, 2048), (8192, 22016, 2048),
                    (8192, 8192, 8192), (22016, 8192, 8192)):
        assert fwd_need(N, K, M, 64) <= 32 << 20, (N, K, M)
    # few tokens: the workspace forward splits the GEMM's reduction and needs
    # more than the array for its partials; the no-alloc forward takes fewer
    # splits and is not rejected (here it fails later, at the first HIP call,
    # since this host has no GPU)
    for N, K, M in ((22016, 8192, 256), (11008, 4096, 512), (22016, 8192, 17)):
        st = f(ctypes.byref(desc(N, K)), FAKE, M, FAKE, FAKE, 64, 16.0, FAKE, q.QLORA_BF16, None, None)
        assert st != q.QLORA_ERR_WORKSPACE_TOO_SMALL, (N, K, M)
    assert fwd_need(11008, 4096, 512, 64) > 32 << 20 and fwd_need(22016, 8192, 256, 64) > 32 << 20


# ---------------------------------------------------------------- binding


def cpu_nf4(N, K):
    s = q.qlora_nf4_sizes(N, K, 0, 1)
    return q.Nf4Tensor(N, K, torch.empty(s["codes_bytes"], dtype=torch.uint8),
                       torch.empty(s["absmax_bytes"], dtype=torch.uint8),
                       torch.empty(s["scale_bytes"] // 4, dtype=torch.float32),
                       torch.empty(1, dtype=torch.float32))


def bf(*shape):
    return torch.empty(*shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.empty(*shape, dtype=torch.float32)


def test_binding_forward_checks_shapes_and_dtypes():
    W = cpu_nf4(64, 128)
    ws = torch.empty(1 << 20, dtype=torch.uint8)
    good = dict(X=bf(32, 128), A=bf(8, 128), B=bf(64, 8), Y=bf(32, 64), T=f32(32, 8))
    bad_cases = [
        ("X", bf(32, 64), "X: shape"),
        ("A", bf(8, 64), "A: shape"),
        ("B", bf(8, 64), "B: shape"),
        ("Y", bf(32, 32), "Y: shape"),
        ("T", f32(32, 4), "T_save: shape"),
        ("A", f32(8, 128), "A: dtype"),
        ("Y", torch.empty(32, 64, dtype=torch.float16), "Y: dtype"),
    ]
    for key, val, msg in bad_cases:
        a = dict(good)
        a[key] = val
        with pytest.raises(ValueError, match=msg):
            q.qlora_linear_fwd(W, a["X"], a["A"], a["B"], 8, 16.0, a["Y"], a["T"], ws)
        with pytest.raises(ValueError, match=msg):
            q.qlora_linear_fwd_noalloc(W, a["X"], a["A"], a["B"], 8, 16.0, a["Y"], a["T"])
    # correct shapes reach the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        q.qlora_linear_fwd(W, good["X"], good["A"], good["B"], 8, 16.0, good["Y"], good["T"], ws)


def test_binding_backward_checks_shapes_and_dtypes():
    W = cpu_nf4(64, 128)
    ws = torch.empty(1 << 20, dtype=torch.uint8)
    good = dict(X=bf(32, 128), dY=bf(32, 64), A=bf(8, 128), B=bf(64, 8), T=f32(32, 8),
                dX=bf(32, 128), dA=f32(8, 128), dB=f32(64, 8))
    for key, val in (("dY", bf(32, 128)), ("dX", bf(32, 64)), ("dA", f32(128, 8)), ("dB", bf(64, 8)),
                     ("T", f32(8, 32)), ("X", bf(31, 128))):
        a = dict(good)
        a[key] = val
        with pytest.raises(ValueError):
            q.qlora_linear_bwd(W, a["X"], a["dY"], a["A"], a["B"], 8, 16.0, a["T"], a["dX"], a["dA"], a["dB"],
                               ws)


def test_binding_checks_the_quantized_arrays():
    W = cpu_nf4(64, 128)
    W.codes = torch.empty(64 * 128 // 2 - 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes"):
        q.qlora_dequantize(W, bf(64, 128))
    W = cpu_nf4(64, 128)
    W.dq_scale = torch.empty(1, dtype=torch.float64)
    with pytest.raises(ValueError, match="dq_scale"):
        q.qlora_dequantize(W, bf(64, 128))
    W = cpu_nf4(64, 128)
    with pytest.raises(ValueError, match="out: shape"):
        q.qlora_dequantize(W, bf(128, 64))
    with pytest.raises(ValueError, match="W: shape"):
        q.qlora_nf4_quantize(f32(64, 64), W, torch.empty(1024, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out: shape"):
        q.qlora_merge_lora(W, bf(8, 128), bf(64, 8), 8, 16.0, bf(64, 64))


def test_binding_checks_format_tensors():
    qt = q.QTensor(64, 128, "int8", torch.empty(64 * 128 // 2, dtype=torch.uint8),
                   torch.empty(128, dtype=torch.float32))
    with pytest.raises(ValueError, match="codes"):
        q.qlora_dequantize_format(qt, bf(64, 128))
    qt = q.QTensor.empty(64, 128, "nf4", device="cpu")
    with pytest.raises(ValueError, match="X: shape"):
        q.qlora_gemv_format(qt, bf(4, 64), f32(4, 64))
