"""Packed Q1 (1-bit affine, group 128) decode kernels for MI355X (gfx950).

The compute lives in ``libq1.so`` (HIP kernels behind the C ABI declared in
``include/q1.h``); this package is the thin ctypes binding over it.
"""
from .q1 import (PackedQ1, Q1Error, load_library, q1_check_symmetric, q1_device_supported, q1_dequantize, q1_embed_rows, q1_ffn,
                 q1_ffn_workspace_bytes, q1_last_error, q1_pack_signs, q1_qmm, q1_qmm_noalloc, q1_qmm_workspace_bytes, q1_stream_read,
                 q1_set_max_packed_rows,
                 q1_version, EXPORTS, LIB_PATH)

__all__ = ["PackedQ1", "Q1Error", "load_library", "q1_check_symmetric", "q1_device_supported", "q1_dequantize", "q1_embed_rows", "q1_ffn",
           "q1_ffn_workspace_bytes", "q1_last_error", "q1_pack_signs", "q1_qmm", "q1_qmm_noalloc", "q1_qmm_workspace_bytes", "q1_stream_read", "q1_set_max_packed_rows",
           "q1_version", "EXPORTS", "LIB_PATH"]
