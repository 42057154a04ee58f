"""q6_K x int8 prefill GEMM for MI355X (gfx950).

A thin ctypes binding of ``libq6k.so`` (C ABI in ``include/q6k.h`` and ``include/q4k.h``): every function here only
checks Python-side types, passes device pointers, sizes and the current HIP stream, and raises on
a non-zero status.  All arithmetic runs in the HIP kernels.  PyTorch is used for device memory
and streams only.  If the built library is missing, importing the binding raises.
"""
from ._lib import (  # noqa: F401
    q4k_act_sums,
    q4k_expand_weights,
    q4k_gemm,
    q4k_gemm_dots,
    q4k_gemm_workspace,
    q4k_launches,
    q4k_quantize_act,
    q4k_weight_bytes,
    LAYOUT_EXPANDED,
    LAYOUT_FOLDED,
    LAYOUT_PACKED,
    Q6KError,
    lib_path,
    q6k_act_bytes,
    q6k_expand_weights,
    q6k_gemm,
    q6k_gemm_chunkdots,
    q6k_gemm_noalloc,
    q6k_gemm_subdots,
    q6k_gemm_workspace,
    q6k_quantize_act,
    q6k_stats,
    q6k_strerror,
    q6k_swiglu_f32,
    q6k_swiglu_quantize_act,
    q6k_weight_bytes,
)
