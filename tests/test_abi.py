"""The C ABI library on the CPU: it loads, exports every declared entry point,
reports sizes, and rejects invalid arguments before making any HIP call (the
pointers below are fake; only validation paths run)."""

import ctypes
import re
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

import quantized_fine_tuning_amd as q
from oracle import footprint, nf4

ROOT = Path(__file__).resolve().parents[1]


def declared_functions():
    names = set()
    for h in (ROOT / "include").glob("*.h"):
        text = h.read_text()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"qlora_nf4_quantize", "qlora_dequantize", "qlora_linear_fwd",
            "qlora_linear_bwd"} <= set(names)
    for n in names:
        assert hasattr(q.lib, n), n
        assert n in q.EXPORTS


def test_library_codebook_equals_oracle_bit_for_bit():
    lib_q = np.array(q.qlora_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_q.view(np.uint32), nf4.codebook().view(np.uint32))


def test_sizes_match_storage_arithmetic():
    for n, k in ((256, 256), (4096, 4096), (11008, 4096), (8192, 22016)):
        s = q.qlora_nf4_sizes(n, k, 0, 16)
        ref = footprint.tensor_bytes(n, k)
        assert s["codes_bytes"] == ref["codes"]
        assert s["absmax_bytes"] == ref["absmax_e4m3"]
        assert s["scale_bytes"] == ref["dq_scale"]
        assert s["mean_bytes"] == ref["dq_mean"]
        bits = 8 * (s["codes_bytes"] + s["absmax_bytes"] + s["scale_bytes"] + s["mean_bytes"]) / (n * k)
        assert abs(bits - footprint.bits_per_param(n, k)) < 1e-12


def test_workspace_grows_with_tokens():
    a = q.qlora_nf4_sizes(4096, 4096, 16, 64)
    b = q.qlora_nf4_sizes(4096, 4096, 4096, 64)
    assert b["fwd_ws_bytes"] > a["fwd_ws_bytes"] and b["bwd_ws_bytes"] > a["bwd_ws_bytes"]
    assert q.qlora_nf4_sizes(256, 256, 0, 8)["quantize_ws_bytes"] >= 4 * 1024


FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def desc(n=256, k=256, codes=FAKE, e=FAKE, s=FAKE, mu=FAKE):
    return q.qlora_nf4_t(n, k, codes, e, s, mu)


def status(fn, *args):
    return fn(*args), q.lib.qlora_last_error().decode()


@pytest.mark.parametrize("n,k,r,m,expect", [
    (256, 0, 8, 0, q.QLORA_ERR_INVALID_ARG),
    (256, 96, 8, 0, q.QLORA_ERR_INVALID_ARG),      # K % 64
    (250, 256, 8, 0, q.QLORA_ERR_INVALID_ARG),     # N % 8
    (256, 256, 0, 0, q.QLORA_ERR_INVALID_ARG),     # r < 1
    (256, 256, 257, 0, q.QLORA_ERR_INVALID_ARG),   # r > 256
    (256, 256, 8, -1, q.QLORA_ERR_INVALID_ARG),    # M_max < 0
    (256, 256, 8, 0, q.QLORA_OK),
])
def test_sizes_validation(n, k, r, m, expect):
    out = q.qlora_sizes_t()
    st, msg = status(q.lib.qlora_nf4_sizes, n, k, m, r, ctypes.byref(out))
    assert st == expect, msg
    if st != q.QLORA_OK:
        assert msg


def test_quantize_validation():
    lib = q.lib
    d = desc()
    big = 1 << 30
    assert lib.qlora_nf4_quantize(FAKE, 7, 256, 256, ctypes.byref(d), FAKE, big, None) == \
        q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert lib.qlora_nf4_quantize(None, q.QLORA_F32, 256, 256, ctypes.byref(d), FAKE, big, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_nf4_quantize(FAKE + 4, q.QLORA_F32, 256, 256, ctypes.byref(d), FAKE, big,
                                  None) == q.QLORA_ERR_INVALID_ARG
    assert "aligned" in lib.qlora_last_error().decode()
    assert lib.qlora_nf4_quantize(FAKE, q.QLORA_F32, 256, 192, ctypes.byref(d), FAKE, big,
                                  None) == q.QLORA_ERR_INVALID_ARG   # descriptor shape
    bad = desc(codes=None)
    assert lib.qlora_nf4_quantize(FAKE, q.QLORA_F32, 256, 256, ctypes.byref(bad), FAKE, big,
                                  None) == q.QLORA_ERR_INVALID_ARG
    need = q.qlora_nf4_sizes(256, 256, 0, 1)["quantize_ws_bytes"]
    assert lib.qlora_nf4_quantize(FAKE, q.QLORA_F32, 256, 256, ctypes.byref(d), FAKE, need - 1,
                                  None) == q.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert lib.qlora_nf4_quantize(FAKE, q.QLORA_F32, 256, 256, None, FAKE, big, None) == \
        q.QLORA_ERR_INVALID_ARG


def test_dequantize_validation():
    lib = q.lib
    d = desc()
    assert lib.qlora_dequantize(ctypes.byref(d), FAKE, q.QLORA_F32, None) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert lib.qlora_dequantize(ctypes.byref(d), None, q.QLORA_BF16, None) == q.QLORA_ERR_INVALID_ARG
    bad = desc(k=100)
    assert lib.qlora_dequantize(ctypes.byref(bad), FAKE, q.QLORA_BF16, None) == q.QLORA_ERR_INVALID_ARG
    bad = desc(mu=FAKE + 8)
    assert lib.qlora_dequantize(ctypes.byref(bad), FAKE, q.QLORA_BF16, None) == q.QLORA_ERR_INVALID_ARG


def test_forward_validation():
    lib = q.lib
    d = desc()
    big = 1 << 30
    f = lib.qlora_linear_fwd
    ok_args = dict(X=FAKE, M=32, A=FAKE, B=FAKE, r=8, alpha=16.0, Y=FAKE, yd=q.QLORA_BF16,
                   T=None, ws=FAKE, wsb=big)

    def call(**kw):
        a = dict(ok_args)
        a.update(kw)
        return f(ctypes.byref(d), a["X"], a["M"], a["A"], a["B"], a["r"], a["alpha"], a["Y"],
                 a["yd"], a["T"], a["ws"], a["wsb"], None)

    assert call(r=0) == q.QLORA_ERR_INVALID_ARG
    assert call(r=300) == q.QLORA_ERR_INVALID_ARG
    assert call(M=-1) == q.QLORA_ERR_INVALID_ARG
    assert call(yd=5) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert call(X=None) == q.QLORA_ERR_INVALID_ARG
    assert call(A=FAKE + 2) == q.QLORA_ERR_INVALID_ARG
    assert call(T=FAKE + 4) == q.QLORA_ERR_INVALID_ARG
    assert call(wsb=0) == q.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert f(None, FAKE, 32, FAKE, FAKE, 8, 16.0, FAKE, 1, None, FAKE, big, None) == q.QLORA_ERR_INVALID_ARG


def test_backward_validation():
    lib = q.lib
    d = desc()
    big = 1 << 30
    b = lib.qlora_linear_bwd

    def call(X=FAKE, dY=FAKE, M=32, r=8, T=None, dX=FAKE, dxd=q.QLORA_BF16, dA=FAKE, dB=FAKE,
             ws=FAKE, wsb=big):
        return b(ctypes.byref(d), X, dY, M, FAKE, FAKE, r, 16.0, T, dX, dxd, dA, dB, ws, wsb, None)

    assert call(dA=None) == q.QLORA_ERR_INVALID_ARG
    assert call(dB=FAKE + 1) == q.QLORA_ERR_INVALID_ARG
    assert call(dY=None) == q.QLORA_ERR_INVALID_ARG
    assert call(dxd=3) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert call(r=-2) == q.QLORA_ERR_INVALID_ARG
    assert call(wsb=16) == q.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=None) == q.QLORA_ERR_INVALID_ARG


def test_adamw_validation():
    lib = q.lib
    T = q._binding.qlora_adamw_tensor_t

    def arr(*ts):
        a = (T * max(1, len(ts)))()
        for i, t in enumerate(ts):
            a[i] = t
        return a

    good = T(FAKE, FAKE, FAKE, FAKE, 1000)

    def call(ts=(good,), count=None, dt=q.QLORA_BF16, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0,
             step=1):
        a = arr(*ts)
        return lib.qlora_adamw_step(a, len(ts) if count is None else count, dt, lr, b1, b2, eps, wd,
                                    step, None)

    assert lib.qlora_adamw_step(None, 1, q.QLORA_BF16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert call(count=0) == q.QLORA_ERR_INVALID_ARG
    assert call(ts=(good,) * 9) == q.QLORA_ERR_INVALID_ARG
    assert call(dt=7) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert call(step=0) == q.QLORA_ERR_INVALID_ARG
    assert call(b1=1.0) == q.QLORA_ERR_INVALID_ARG
    assert call(b2=-0.1) == q.QLORA_ERR_INVALID_ARG
    assert call(eps=0.0) == q.QLORA_ERR_INVALID_ARG
    assert call(lr=-1.0) == q.QLORA_ERR_INVALID_ARG
    assert call(wd=float("inf")) == q.QLORA_ERR_INVALID_ARG
    assert call(ts=(T(FAKE, None, FAKE, FAKE, 10),)) == q.QLORA_ERR_INVALID_ARG
    assert call(ts=(T(FAKE, FAKE, FAKE + 4, FAKE, 10),)) == q.QLORA_ERR_INVALID_ARG
    assert "aligned" in lib.qlora_last_error().decode()
    assert call(ts=(good, T(FAKE, FAKE, FAKE, FAKE, -1))) == q.QLORA_ERR_INVALID_ARG
    # an empty tensor needs no pointers; all-empty enqueues nothing
    assert call(ts=(T(None, None, None, None, 0),)) == q.QLORA_OK


def test_compute_dtype_validation():
    lib = q.lib
    d = desc()
    big = 1 << 30

    def fwd(cd, yd):
        return lib.qlora_linear_fwd_ex(ctypes.byref(d), FAKE, 32, FAKE, FAKE, 8, 16.0, FAKE, yd, None, FAKE,
                                       big, cd, None)

    def bwd(cd, dxd):
        return lib.qlora_linear_bwd_ex(ctypes.byref(d), FAKE, FAKE, 32, FAKE, FAKE, 8, 16.0, None, FAKE, dxd,
                                       FAKE, FAKE, FAKE, big, cd, None)

    assert fwd(q.QLORA_F32, q.QLORA_F32) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert fwd(7, q.QLORA_F32) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert fwd(q.QLORA_F16, q.QLORA_BF16) == q.QLORA_ERR_UNSUPPORTED_DTYPE  # 16-bit output in the other format
    assert fwd(q.QLORA_BF16, q.QLORA_F16) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert bwd(q.QLORA_F32, q.QLORA_F32) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert bwd(q.QLORA_F16, q.QLORA_BF16) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    # the original entry points are the bf16 forms
    assert lib.qlora_linear_fwd(ctypes.byref(d), FAKE, 32, FAKE, FAKE, 8, 16.0, FAKE, q.QLORA_F16, None, FAKE,
                                big, None) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert lib.qlora_dequantize(ctypes.byref(d), FAKE, q.QLORA_F32, None) == q.QLORA_ERR_UNSUPPORTED_DTYPE


def test_merge_validation():
    lib = q.lib
    m = lib.qlora_merge_lora

    def call(d=None, A=FAKE, B=FAKE, r=8, out=FAKE, od=q.QLORA_BF16):
        d = desc() if d is None else d
        return m(ctypes.byref(d), A, B, r, 16.0, out, od, None)

    assert call(od=q.QLORA_F32) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert call(od=7) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert call(r=0) == q.QLORA_ERR_INVALID_ARG
    assert call(r=257) == q.QLORA_ERR_INVALID_ARG
    assert call(A=None) == q.QLORA_ERR_INVALID_ARG
    assert call(B=FAKE + 2) == q.QLORA_ERR_INVALID_ARG
    assert call(out=None) == q.QLORA_ERR_INVALID_ARG
    assert call(d=desc(k=100)) == q.QLORA_ERR_INVALID_ARG
    # 2^31 parameters is the limit of the 32-bit code offsets
    assert call(d=desc(n=1 << 16, k=1 << 16)) == q.QLORA_ERR_INVALID_ARG
    assert "too large" in lib.qlora_last_error().decode()
    assert m(None, FAKE, FAKE, 8, 16.0, FAKE, q.QLORA_BF16, None) == q.QLORA_ERR_INVALID_ARG


def test_format_validation():
    lib = q.lib
    QT = q.qlora_qtensor_t

    def qt(n=256, k=256, fmt=q._binding.QLORA_FMT_INT4, codes=FAKE, absmax=FAKE):
        return QT(n, k, fmt, codes, absmax)

    quant = lib.qlora_quantize_format
    assert quant(FAKE, q.QLORA_F16, 256, 256, ctypes.byref(qt()), None) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert quant(FAKE, q.QLORA_F32, 256, 100, ctypes.byref(qt(k=100)), None) == q.QLORA_ERR_INVALID_ARG
    assert quant(FAKE, q.QLORA_F32, 256, 256, ctypes.byref(qt(fmt=0)), None) == q.QLORA_ERR_INVALID_ARG
    assert quant(FAKE, q.QLORA_F32, 256, 256, ctypes.byref(qt(fmt=4)), None) == q.QLORA_ERR_INVALID_ARG
    assert quant(FAKE, q.QLORA_F32, 256, 256, ctypes.byref(qt(n=128)), None) == q.QLORA_ERR_INVALID_ARG
    assert quant(None, q.QLORA_F32, 256, 256, ctypes.byref(qt()), None) == q.QLORA_ERR_INVALID_ARG
    assert quant(FAKE, q.QLORA_F32, 256, 256, ctypes.byref(qt(absmax=FAKE + 4)), None) == q.QLORA_ERR_INVALID_ARG
    assert quant(FAKE, q.QLORA_F32, 256, 256, None, None) == q.QLORA_ERR_INVALID_ARG
    deq = lib.qlora_dequantize_format
    assert deq(ctypes.byref(qt()), FAKE, q.QLORA_F32, None) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert deq(ctypes.byref(qt()), None, q.QLORA_BF16, None) == q.QLORA_ERR_INVALID_ARG
    assert deq(ctypes.byref(qt(codes=None)), FAKE, q.QLORA_BF16, None) == q.QLORA_ERR_INVALID_ARG
    gemv = lib.qlora_gemv_format
    assert gemv(ctypes.byref(qt()), FAKE, 17, FAKE, q.QLORA_F32, None) == q.QLORA_ERR_INVALID_ARG
    assert gemv(ctypes.byref(qt()), FAKE, -1, FAKE, q.QLORA_F32, None) == q.QLORA_ERR_INVALID_ARG
    assert gemv(ctypes.byref(qt()), FAKE, 1, FAKE, q.QLORA_F16, None) == q.QLORA_ERR_UNSUPPORTED_DTYPE
    assert gemv(ctypes.byref(qt()), None, 1, FAKE, q.QLORA_F32, None) == q.QLORA_ERR_INVALID_ARG
    assert gemv(ctypes.byref(qt(fmt=9)), FAKE, 1, FAKE, q.QLORA_F32, None) == q.QLORA_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert q.lib.qlora_status_string(s).decode()
    assert q.lib.qlora_status_string(99).decode() == "unknown status"


def test_product_path_never_imports_the_oracle():
    code = ("import sys, quantized_fine_tuning_amd; "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules)")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
    for src in (ROOT / "quantized_fine_tuning_amd").rglob("*"):
        if src.suffix in (".py", ".hip", ".cpp", ".h"):
            assert "oracle" not in src.read_text(), src


def test_single_hip_runtime_whatever_the_import_order():
    # the library is handed torch's streams and device pointers, so both must
    # use one HIP runtime
    code = ("import quantized_fine_tuning_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = sorted(set(l.split()[-1] for l in maps if 'libamdhip64' in l))\n"
            "assert len(libs) == 1, libs\n")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
