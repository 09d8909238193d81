"""ctypes binding of libqlora_nf4.so (the C ABI in include/qlora_nf4.h).

Argument marshalling only: every function here checks that tensors are
contiguous and on the GPU, turns them into raw pointers and calls the C entry
point of the same name on torch's current stream.  All computation happens in
the library's HIP kernels.  There is no fallback: if the library is missing,
importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = Path(os.environ.get("QLORA_NF4_LIB", PKG / "libqlora_nf4.so"))

QLORA_OK = 0
QLORA_ERR_INVALID_ARG = 1
QLORA_ERR_UNSUPPORTED_DTYPE = 2
QLORA_ERR_WORKSPACE_TOO_SMALL = 3
QLORA_ERR_HIP = 4
QLORA_F32 = 0
QLORA_BF16 = 1
QLORA_F16 = 2

EXPORTS = ("qlora_nf4_sizes", "qlora_nf4_quantize", "qlora_dequantize", "qlora_linear_fwd",
           "qlora_linear_bwd", "qlora_nf4_codebook", "qlora_status_string", "qlora_last_error",
           "qlora_time_next_launch", "qlora_adamw_step", "qlora_merge_lora",
           "qlora_quantize_format", "qlora_dequantize_format", "qlora_gemv_format",
           "qlora_linear_fwd_ex", "qlora_linear_bwd_ex", "qlora_linear_fwd_noalloc",
           "qlora_bench_mfma_peak", "qlora_bench_copy", "qlora_bench_wall_clock_khz")

QLORA_KERNEL_NONE = 0
QLORA_KERNEL_FWD_GEMM = 1
QLORA_KERNEL_DX_GEMM = 2
QLORA_KERNEL_GEMV = 3
QLORA_KERNEL_QUANTIZE = 4
QLORA_KERNEL_ADAMW = 5
QLORA_KERNEL_MERGE = 6
QLORA_KERNEL_FORMAT_GEMV = 7
QLORA_FMT_NF4 = 1
QLORA_FMT_INT4 = 2
QLORA_FMT_INT8 = 3
FORMATS = {"nf4": QLORA_FMT_NF4, "int4": QLORA_FMT_INT4, "int8": QLORA_FMT_INT8}
QLORA_ADAMW_MAX_TENSORS = 8


class QloraError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"status {status}: {text}")
        self.status = status


class qlora_nf4_t(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("absmax_e4m3", ctypes.c_void_p),
                ("dq_scale", ctypes.c_void_p), ("dq_mean", ctypes.c_void_p)]


class qlora_sizes_t(ctypes.Structure):
    _fields_ = [("codes_bytes", ctypes.c_size_t), ("absmax_bytes", ctypes.c_size_t),
                ("scale_bytes", ctypes.c_size_t), ("mean_bytes", ctypes.c_size_t),
                ("quantize_ws_bytes", ctypes.c_size_t), ("fwd_ws_bytes", ctypes.c_size_t),
                ("bwd_ws_bytes", ctypes.c_size_t)]


class qlora_adamw_tensor_t(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("n", ctypes.c_int64)]


class qlora_qtensor_t(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64), ("format", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p)]


def _load():
    # The library must share torch's HIP runtime: it is handed torch's device
    # pointers, streams and events.  torch ships its own libamdhip64 with the
    # same soname, so loading torch first makes the dynamic loader bind this
    # library to that copy; loading this library first would map a second,
    # separate HIP runtime into the process.
    import torch  # noqa: F401

    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python quantized_fine_tuning_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(str(LIB_PATH))
    i64, i32, vp, sz, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER
    lib.qlora_nf4_sizes.argtypes = [i64, i64, i64, i32, P(qlora_sizes_t)]
    lib.qlora_nf4_quantize.argtypes = [vp, i32, i64, i64, P(qlora_nf4_t), vp, sz, vp]
    lib.qlora_dequantize.argtypes = [P(qlora_nf4_t), vp, i32, vp]
    lib.qlora_linear_fwd.argtypes = [P(qlora_nf4_t), vp, i64, vp, vp, i32, f32, vp, i32, vp, vp,
                                     sz, vp]
    lib.qlora_linear_bwd.argtypes = [P(qlora_nf4_t), vp, vp, i64, vp, vp, i32, f32, vp, vp, i32,
                                     vp, vp, vp, sz, vp]
    for name in ("qlora_nf4_sizes", "qlora_nf4_quantize", "qlora_dequantize",
                 "qlora_linear_fwd", "qlora_linear_bwd"):
        getattr(lib, name).restype = i32
    lib.qlora_nf4_codebook.argtypes = [P(ctypes.c_float)]
    lib.qlora_nf4_codebook.restype = None
    lib.qlora_status_string.argtypes = [i32]
    lib.qlora_status_string.restype = ctypes.c_char_p
    lib.qlora_last_error.argtypes = []
    lib.qlora_last_error.restype = ctypes.c_char_p
    lib.qlora_time_next_launch.argtypes = [i32, vp, vp]
    lib.qlora_time_next_launch.restype = i32
    lib.qlora_adamw_step.argtypes = [P(qlora_adamw_tensor_t), i32, i32, f32, f32, f32, f32, f32, i64, vp]
    lib.qlora_adamw_step.restype = i32
    lib.qlora_merge_lora.argtypes = [P(qlora_nf4_t), vp, vp, i32, f32, vp, i32, vp]
    lib.qlora_merge_lora.restype = i32
    lib.qlora_linear_fwd_ex.argtypes = [P(qlora_nf4_t), vp, i64, vp, vp, i32, f32, vp, i32, vp, vp,
                                        sz, i32, vp]
    lib.qlora_linear_bwd_ex.argtypes = [P(qlora_nf4_t), vp, vp, i64, vp, vp, i32, f32, vp, vp, i32,
                                        vp, vp, vp, sz, i32, vp]
    lib.qlora_linear_fwd_ex.restype = i32
    lib.qlora_linear_fwd_noalloc.argtypes = [P(qlora_nf4_t), vp, i64, vp, vp, i32, f32, vp, i32, vp, vp]
    lib.qlora_linear_fwd_noalloc.restype = i32
    lib.qlora_bench_mfma_peak.argtypes = [i64, vp, P(i64), vp]
    lib.qlora_bench_mfma_peak.restype = i32
    lib.qlora_bench_copy.argtypes = [vp, vp, i64, vp]
    lib.qlora_bench_copy.restype = i32
    lib.qlora_bench_wall_clock_khz.argtypes = [P(i32)]
    lib.qlora_bench_wall_clock_khz.restype = i32
    lib.qlora_linear_bwd_ex.restype = i32
    lib.qlora_quantize_format.argtypes = [vp, i32, i64, i64, P(qlora_qtensor_t), vp]
    lib.qlora_dequantize_format.argtypes = [P(qlora_qtensor_t), vp, i32, vp]
    lib.qlora_gemv_format.argtypes = [P(qlora_qtensor_t), vp, i64, vp, i32, vp]
    for name in ("qlora_quantize_format", "qlora_dequantize_format", "qlora_gemv_format"):
        getattr(lib, name).restype = i32
    return lib


lib = _load()


def _check(status: int):
    if status != QLORA_OK:
        raise QloraError(status, lib.qlora_last_error().decode())


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, name: str, shape, dtypes):
    """Host-side check of a tensor's shape and dtype before its pointer goes to
    the library (a wrong shape would otherwise become an out-of-bounds device
    access or silently reinterpreted data)."""
    if t is None:
        raise ValueError(f"{name} is None")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")


def _expect_numel(t, name: str, n: int, dtype):
    if t is None:
        raise ValueError(f"{name} is None")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.dim() != 1 or t.numel() < n:
        raise ValueError(f"{name}: needs a 1-d tensor of at least {n} elements, got shape {tuple(t.shape)}")


def _bytes(t, name: str) -> int:
    if t is None:
        raise ValueError(f"{name} is None")
    return t.numel() * t.element_size()


def _dtype(t, name: str) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return QLORA_F32
    if t.dtype == torch.bfloat16:
        return QLORA_BF16
    if t.dtype == torch.float16:
        return QLORA_F16  # (accepted by qlora_merge_lora's output only)
    raise ValueError(f"{name}: dtype {t.dtype} is not float32, bfloat16 or float16")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Nf4Tensor:
    """The four device arrays of one quantized weight [N, K] (torch tensors)."""

    def __init__(self, n_rows: int, n_cols: int, codes, absmax_e4m3, dq_scale, dq_mean):
        self.n_rows, self.n_cols = int(n_rows), int(n_cols)
        self.codes, self.absmax_e4m3 = codes, absmax_e4m3
        self.dq_scale, self.dq_mean = dq_scale, dq_mean

    @classmethod
    def empty(cls, n_rows: int, n_cols: int, device="cuda"):
        torch = _torch()
        s = qlora_nf4_sizes(n_rows, n_cols, 0, 1)
        u8 = torch.uint8
        return cls(n_rows, n_cols,
                   torch.empty(s["codes_bytes"], dtype=u8, device=device),
                   torch.empty(s["absmax_bytes"], dtype=u8, device=device),
                   torch.empty(s["scale_bytes"] // 4, dtype=torch.float32, device=device),
                   torch.empty(1, dtype=torch.float32, device=device))

    def c_struct(self) -> qlora_nf4_t:
        torch = _torch()
        nb = self.n_rows * self.n_cols // 64
        _expect_numel(self.codes, "codes", self.n_rows * self.n_cols // 2, torch.uint8)
        _expect_numel(self.absmax_e4m3, "absmax_e4m3", nb, torch.uint8)
        _expect_numel(self.dq_scale, "dq_scale", (nb + 255) // 256, torch.float32)
        _expect_numel(self.dq_mean, "dq_mean", 1, torch.float32)
        return qlora_nf4_t(self.n_rows, self.n_cols, _ptr(self.codes, "codes"),
                           _ptr(self.absmax_e4m3, "absmax_e4m3"), _ptr(self.dq_scale, "dq_scale"),
                           _ptr(self.dq_mean, "dq_mean"))


def workspace(nbytes: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def qlora_nf4_sizes(N: int, K: int, M_max: int, r: int) -> dict:
    out = qlora_sizes_t()
    _check(lib.qlora_nf4_sizes(N, K, M_max, r, ctypes.byref(out)))
    return {name: int(getattr(out, name)) for name, _ in qlora_sizes_t._fields_}


def qlora_nf4_codebook() -> list:
    buf = (ctypes.c_float * 16)()
    lib.qlora_nf4_codebook(buf)
    return list(buf)


def qlora_nf4_quantize(W, out: Nf4Tensor, ws, stream=None) -> None:
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    _expect(W, "W", (out.n_rows, out.n_cols), (torch.float32, torch.bfloat16))
    st = out.c_struct()
    _check(lib.qlora_nf4_quantize(_ptr(W, "W"), _dtype(W, "W"), N, K, ctypes.byref(st),
                                  _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def qlora_dequantize(q: Nf4Tensor, out, stream=None) -> None:
    torch = _torch()
    _expect(out, "out", (q.n_rows, q.n_cols), (torch.bfloat16, torch.float16))
    st = q.c_struct()
    _check(lib.qlora_dequantize(ctypes.byref(st), _ptr(out, "out"), _dtype(out, "out"),
                                _stream(stream)))


def qlora_linear_fwd(W: Nf4Tensor, X, A, B, r: int, alpha: float, Y, T_save, ws,
                     stream=None) -> None:
    """Forward in the compute format of X (bf16 or fp16: qlora_linear_fwd_ex)."""
    qlora_linear_fwd_ex(W, X, A, B, r, alpha, Y, T_save, ws, _dtype(X, "X"), stream)


def _compute_torch_dtype(compute_dtype: int):
    torch = _torch()
    if compute_dtype == QLORA_BF16:
        return torch.bfloat16
    if compute_dtype == QLORA_F16:
        return torch.float16
    raise ValueError(f"compute_dtype {compute_dtype}: QLORA_BF16 or QLORA_F16")


def _check_fwd(W: Nf4Tensor, X, A, B, r: int, Y, T_save, cdt):
    torch = _torch()
    if X is None or X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M = X.shape[0]
    N, K = W.n_rows, W.n_cols
    _expect(X, "X", (M, K), (cdt,))
    _expect(A, "A", (r, K), (cdt,))
    _expect(B, "B", (N, r), (cdt,))
    _expect(Y, "Y", (M, N), (torch.float32, cdt))
    if T_save is not None:
        _expect(T_save, "T_save", (M, r), (torch.float32,))
    return M


def qlora_linear_fwd_ex(W: Nf4Tensor, X, A, B, r: int, alpha: float, Y, T_save, ws, compute_dtype: int,
                        stream=None) -> None:
    M = _check_fwd(W, X, A, B, r, Y, T_save, _compute_torch_dtype(compute_dtype))
    st = W.c_struct()
    _check(lib.qlora_linear_fwd_ex(ctypes.byref(st), _ptr(X, "X"), M, _ptr(A, "A"), _ptr(B, "B"),
                                   r, float(alpha), _ptr(Y, "Y"), _dtype(Y, "Y"),
                                   _ptr(T_save, "T_save"), _ptr(ws, "ws"),
                                   _bytes(ws, "ws"), compute_dtype, _stream(stream)))


def qlora_linear_fwd_noalloc(W: Nf4Tensor, X, A, B, r: int, alpha: float, Y, T_save=None,
                             stream=None) -> None:
    """The bf16 forward with the library's static scratch instead of a
    workspace (for callers that cannot allocate).  Calls that overlap on one
    GPU race: order them."""
    M = _check_fwd(W, X, A, B, r, Y, T_save, _torch().bfloat16)
    st = W.c_struct()
    _check(lib.qlora_linear_fwd_noalloc(ctypes.byref(st), _ptr(X, "X"), M, _ptr(A, "A"), _ptr(B, "B"),
                                        r, float(alpha), _ptr(Y, "Y"), _dtype(Y, "Y"),
                                        _ptr(T_save, "T_save"), _stream(stream)))


def qlora_linear_bwd(W: Nf4Tensor, X, dY, A, B, r: int, alpha: float, T_saved, dX, dA, dB, ws,
                     stream=None) -> None:
    """Backward in the compute format of X (bf16 or fp16: qlora_linear_bwd_ex)."""
    qlora_linear_bwd_ex(W, X, dY, A, B, r, alpha, T_saved, dX, dA, dB, ws, _dtype(X, "X"), stream)


def qlora_linear_bwd_ex(W: Nf4Tensor, X, dY, A, B, r: int, alpha: float, T_saved, dX, dA, dB, ws,
                        compute_dtype: int, stream=None) -> None:
    torch = _torch()
    cdt = _compute_torch_dtype(compute_dtype)
    if X is None or X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M = X.shape[0]
    N, K = W.n_rows, W.n_cols
    _expect(X, "X", (M, K), (cdt,))
    _expect(dY, "dY", (M, N), (cdt,))
    _expect(A, "A", (r, K), (cdt,))
    _expect(B, "B", (N, r), (cdt,))
    if T_saved is not None:
        _expect(T_saved, "T_saved", (M, r), (torch.float32,))
    _expect(dX, "dX", (M, K), (torch.float32, cdt))
    _expect(dA, "dA", (r, K), (torch.float32,))
    _expect(dB, "dB", (N, r), (torch.float32,))
    st = W.c_struct()
    _check(lib.qlora_linear_bwd_ex(ctypes.byref(st), _ptr(X, "X"), _ptr(dY, "dY"), M, _ptr(A, "A"),
                                   _ptr(B, "B"), r, float(alpha), _ptr(T_saved, "T_saved"),
                                   _ptr(dX, "dX"), _dtype(dX, "dX"), _ptr(dA, "dA"), _ptr(dB, "dB"),
                                   _ptr(ws, "ws"), _bytes(ws, "ws"), compute_dtype,
                                   _stream(stream)))


def qlora_bench_mfma_peak(iters: int, sink, stream=None) -> int:
    """Launches the MFMA reference loop; returns its FLOP count.  sink: 2056
    float32 on the device; sink[2048:].view(int64) receives the shader and
    real-time clock counters of workgroup 0 (start, end, start, end)."""
    torch = _torch()
    _expect_numel(sink, "sink", 2056, torch.float32)
    flop = ctypes.c_int64(0)
    _check(lib.qlora_bench_mfma_peak(int(iters), _ptr(sink, "sink"), ctypes.byref(flop), _stream(stream)))
    return int(flop.value)


def qlora_bench_wall_clock_khz() -> int:
    """Rate of the device's real-time counter, kHz."""
    khz = ctypes.c_int32(0)
    _check(lib.qlora_bench_wall_clock_khz(ctypes.byref(khz)))
    return int(khz.value)


def qlora_bench_copy(src, dst, stream=None) -> None:
    """Streaming copy of src into dst (same number of bytes)."""
    if _bytes(src, "src") != _bytes(dst, "dst"):
        raise ValueError("src and dst sizes differ")
    _check(lib.qlora_bench_copy(_ptr(src, "src"), _ptr(dst, "dst"), _bytes(src, "src"), _stream(stream)))


def qlora_time_next_launch(kernel_id: int, start_event=None, stop_event=None) -> None:
    """Bracket the next launch of `kernel_id` with two torch.cuda.Event objects
    (each must have been recorded once so that its HIP event exists)."""
    s = ctypes.c_void_p(start_event.cuda_event) if start_event is not None else None
    e = ctypes.c_void_p(stop_event.cuda_event) if stop_event is not None else None
    _check(lib.qlora_time_next_launch(kernel_id, s, e))


def qlora_adamw_step(tensors, lr: float, beta1: float, beta2: float, eps: float,
                     weight_decay: float, step: int, stream=None) -> None:
    """One AdamW step on up to QLORA_ADAMW_MAX_TENSORS tensors in one launch.
    tensors: sequence of (param, grad, exp_avg, exp_avg_sq); every param is
    bf16 or every param is fp32; grad and the moments are fp32 of the same
    number of elements; all updated in place."""
    tensors = list(tensors)
    arr = (qlora_adamw_tensor_t * max(1, len(tensors)))()
    dt = None
    torch = _torch()
    for i, (p, g, m, v) in enumerate(tensors):
        d = _dtype(p, f"tensors[{i}].param")
        if d not in (QLORA_BF16, QLORA_F32):
            raise ValueError(f"tensors[{i}].param: bf16 or fp32")
        for t_, nm in ((g, "grad"), (m, "exp_avg"), (v, "exp_avg_sq")):
            if t_.dtype != torch.float32:
                raise ValueError(f"tensors[{i}].{nm}: dtype {t_.dtype}, expected float32")
        if dt is not None and d != dt:
            raise ValueError("every param must have the same dtype")
        dt = d
        n = p.numel()
        if not (g.numel() == m.numel() == v.numel() == n):
            raise ValueError(f"tensors[{i}]: element counts differ")
        arr[i] = qlora_adamw_tensor_t(_ptr(p, "param"), _ptr(g, "grad"), _ptr(m, "exp_avg"),
                                      _ptr(v, "exp_avg_sq"), n)
    _check(lib.qlora_adamw_step(arr, len(tensors), QLORA_BF16 if dt is None else dt, float(lr),
                                float(beta1), float(beta2), float(eps), float(weight_decay),
                                int(step), _stream(stream)))


def qlora_merge_lora(W: Nf4Tensor, A, B, r: int, alpha: float, out, stream=None) -> None:
    """out [N, K] (bf16 or fp16) = Ŵ + (alpha / r)·B·A, rounded once."""
    torch = _torch()
    _expect(A, "A", (r, W.n_cols), (torch.bfloat16,))
    _expect(B, "B", (W.n_rows, r), (torch.bfloat16,))
    _expect(out, "out", (W.n_rows, W.n_cols), (torch.bfloat16, torch.float16))
    st = W.c_struct()
    _check(lib.qlora_merge_lora(ctypes.byref(st), _ptr(A, "A"), _ptr(B, "B"), r, float(alpha),
                                _ptr(out, "out"), _dtype(out, "out"), _stream(stream)))


class QTensor:
    """A weight in one of the comparison formats ("nf4", "int4", "int8"):
    codes (uint8) and one fp32 absmax per 64-block, device tensors."""

    def __init__(self, n_rows: int, n_cols: int, fmt: str, codes, absmax):
        self.n_rows, self.n_cols, self.fmt = n_rows, n_cols, fmt
        self.codes, self.absmax = codes, absmax

    @classmethod
    def empty(cls, n_rows: int, n_cols: int, fmt: str, device="cuda"):
        torch = _torch()
        nbytes = n_rows * n_cols if fmt == "int8" else n_rows * n_cols // 2
        return cls(n_rows, n_cols, fmt, torch.empty(nbytes, dtype=torch.uint8, device=device),
                   torch.empty(n_rows * n_cols // 64, dtype=torch.float32, device=device))

    def c_struct(self) -> qlora_qtensor_t:
        torch = _torch()
        if self.fmt not in FORMATS:
            raise ValueError(f"format {self.fmt!r}: one of {sorted(FORMATS)}")
        nbytes = self.n_rows * self.n_cols * (2 if self.fmt == "int8" else 1) // 2
        _expect_numel(self.codes, "codes", nbytes, torch.uint8)
        _expect_numel(self.absmax, "absmax", self.n_rows * self.n_cols // 64, torch.float32)
        return qlora_qtensor_t(self.n_rows, self.n_cols, FORMATS[self.fmt], _ptr(self.codes, "codes"),
                               _ptr(self.absmax, "absmax"))


def qlora_quantize_format(W, out: QTensor, stream=None) -> None:
    torch = _torch()
    _expect(W, "W", (out.n_rows, out.n_cols), (torch.float32, torch.bfloat16))
    N, K = W.shape
    st = out.c_struct()
    _check(lib.qlora_quantize_format(_ptr(W, "W"), _dtype(W, "W"), N, K, ctypes.byref(st), _stream(stream)))


def qlora_dequantize_format(q: QTensor, out, stream=None) -> None:
    torch = _torch()
    _expect(out, "out", (q.n_rows, q.n_cols), (torch.bfloat16,))
    st = q.c_struct()
    _check(lib.qlora_dequantize_format(ctypes.byref(st), _ptr(out, "out"), _dtype(out, "out"), _stream(stream)))


def qlora_gemv_format(q: QTensor, X, Y, stream=None) -> None:
    torch = _torch()
    if X is None or X.dim() != 2:
        raise ValueError("X must be [M, K]")
    _expect(X, "X", (X.shape[0], q.n_cols), (torch.bfloat16,))
    _expect(Y, "Y", (X.shape[0], q.n_rows), (torch.float32, torch.bfloat16))
    st = q.c_struct()
    _check(lib.qlora_gemv_format(ctypes.byref(st), _ptr(X, "X"), X.shape[0], _ptr(Y, "Y"), _dtype(Y, "Y"),
                                 _stream(stream)))
