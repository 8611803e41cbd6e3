"""HLWQ (Hadamard-Lloyd Weight Quantization) for MI355X: Python binding of libhlwq.

The package holds the HIP kernels and C ABI (``csrc/``, ``include/hlwq.h`` at
the repository root), the in-tree build (``build.py``) and this thin ctypes
binding.  Importing it loads nothing; the first call loads ``libhlwq.so`` and
fails loudly if it has not been built.
"""
from .binding import (  # noqa: F401
    HLWQError,
    MatDesc,
    declared_functions,
    hlwq_centroids,
    hlwq_dequantize,
    hlwq_dequantize_codes8,
    hlwq_dequantize_grouped,
    hlwq_dequantize_int4,
    hlwq_dequantize_int4_grouped,
    hlwq_kv_append,
    hlwq_kv_dequantize,
    hlwq_kv_quantize,
    hlwq_norm_count,
    hlwq_packed_bytes,
    hlwq_quantize,
    hlwq_quantize_codes8,
    hlwq_quantize_grouped,
    hlwq_search_table,
    hlwq_status_string,
    hlwq_tq3_dequantize,
    hlwq_tq3_dequantize_grouped,
    hlwq_tq3_quantize,
    hlwq_tq3_quantize_grouped,
    hlwq_tq3_signs,
    load_library,
    packed_shape,
)
