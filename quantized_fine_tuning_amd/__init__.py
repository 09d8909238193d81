"""NF4 QLoRA linear-layer hot path for MI355X (gfx950).

The computation lives in libqlora_nf4.so (hand-written HIP kernels behind the C
ABI of include/qlora_nf4.h); this package is a thin ctypes binding whose
functions carry the C entry points' names.  Importing it fails if the library
has not been built (``python quantized_fine_tuning_amd/build.py``).
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    QLORA_ADAMW_MAX_TENSORS,
    QLORA_BF16,
    QLORA_F16,
    QLORA_ERR_HIP,
    QLORA_ERR_INVALID_ARG,
    QLORA_ERR_UNSUPPORTED_DTYPE,
    QLORA_ERR_WORKSPACE_TOO_SMALL,
    QLORA_F32,
    QLORA_KERNEL_DX_GEMM,
    QLORA_KERNEL_FWD_GEMM,
    QLORA_KERNEL_GEMV,
    QLORA_KERNEL_NONE,
    QLORA_KERNEL_QUANTIZE,
    QLORA_KERNEL_ADAMW,
    QLORA_KERNEL_MERGE,
    QLORA_KERNEL_FORMAT_GEMV,
    QLORA_OK,
    Nf4Tensor,
    QTensor,
    QloraError,
    lib,
    qlora_adamw_step,
    qlora_dequantize,
    qlora_linear_bwd,
    qlora_linear_fwd,
    qlora_linear_fwd_ex,
    qlora_linear_fwd_noalloc,
    qlora_bench_mfma_peak,
    qlora_bench_copy,
    qlora_linear_bwd_ex,
    qlora_merge_lora,
    qlora_quantize_format,
    qlora_dequantize_format,
    qlora_gemv_format,
    qlora_qtensor_t,
    qlora_nf4_codebook,
    qlora_nf4_quantize,
    qlora_nf4_sizes,
    qlora_nf4_t,
    qlora_sizes_t,
    qlora_time_next_launch,
    workspace,
)
