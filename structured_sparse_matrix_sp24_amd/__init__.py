"""MI355X (gfx950) 2:4 structured-sparse compression and sparse x dense GEMM.

The compute lives in libsp24.so (hand-written HIP kernels); see
include/sp24.h for the C ABI.  ``capi`` is a thin ctypes binding that mirrors
it; ``workloads`` builds seeded synthetic inputs.
"""
from .capi import (SP24_B_KN, SP24_B_NK, SP24_BF16, SP24_BF8_E5M2, SP24_F16, SP24_F32,  # noqa: F401
                   SP24_FP8_E4M3, SP24_I8, SP24_I32, SP24_LAYOUT_KBLOCK, SP24_LAYOUT_ROW, SP24_OK, Sp24Error,
                   compressed_shapes, decompress, gemm, kblock_width, prune_compress, sp24_calib_mfma,
                   sp24_calib_mfma_ex, sp24_calib_stream,
                   sp24_decompress, sp24_gemm, sp24_gemm_ex, sp24_gemm_workspace_bytes, sp24_meta_bytes,
                   sp24_prune_compress, sp24_status_string, sp24_validate_meta, sp24_values_bytes, sp24_version,
                   validate_meta)

__all__ = ["prune_compress", "gemm", "decompress", "validate_meta", "compressed_shapes", "kblock_width",
           "sp24_prune_compress", "sp24_decompress", "sp24_validate_meta", "sp24_gemm", "sp24_gemm_ex",
           "sp24_values_bytes", "sp24_meta_bytes", "sp24_gemm_workspace_bytes", "sp24_status_string",
           "sp24_version", "sp24_calib_stream", "sp24_calib_mfma", "sp24_calib_mfma_ex",
           "Sp24Error"]
