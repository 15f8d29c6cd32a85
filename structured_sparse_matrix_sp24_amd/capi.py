"""ctypes binding of libsp24 (argument marshalling only).

The functions named ``sp24_*`` mirror include/sp24.h one to one and take raw
device pointers (ints) plus a HIP stream handle.  ``prune_compress`` and
``gemm`` are torch conveniences: they allocate outputs with torch and pass
``torch.cuda.current_stream()``.  Every step of the computation runs in the
library's HIP kernels; if the library is missing this module raises -- there
is no other path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsp24.so")

SP24_F16, SP24_BF16, SP24_I8, SP24_FP8_E4M3, SP24_BF8_E5M2 = 1, 2, 3, 4, 5
SP24_F32, SP24_I32 = 6, 7  # output (C / D) types only
SP24_LAYOUT_ROW, SP24_LAYOUT_KBLOCK = 0, 1
SP24_B_KN, SP24_B_NK = 0, 1
SP24_OK = 0
_ESIZE = {SP24_F16: 2, SP24_BF16: 2, SP24_I8: 1, SP24_FP8_E4M3: 1, SP24_BF8_E5M2: 1}


class Sp24Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {sp24_status_string(status)} ({status})")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libsp24.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.sp24_values_bytes.argtypes = [I64, I64, I, I]
        L.sp24_values_bytes.restype = SZ
        L.sp24_meta_bytes.argtypes = [I64, I64, I, I]
        L.sp24_meta_bytes.restype = SZ
        L.sp24_gemm_workspace_bytes.argtypes = [I64, I64, I64, I, I]
        L.sp24_gemm_workspace_bytes.restype = SZ
        L.sp24_prune_compress.argtypes = [P, P, P, I64, I64, I, I, P]
        L.sp24_prune_compress.restype = I
        L.sp24_gemm.argtypes = [P, P, I, I, P, I, I, P, I64, I64, I64, F, F, P, SZ, P]
        L.sp24_gemm.restype = I
        L.sp24_gemm_ex.argtypes = [P, P, I, I, P, I, I, P, I, P, I64, I64, I64, F, F, P, SZ, P]
        L.sp24_gemm_ex.restype = I
        L.sp24_decompress.argtypes = [P, P, P, I64, I64, I, I, P]
        L.sp24_decompress.restype = I
        L.sp24_validate_meta.argtypes = [P, I64, I64, I, I, P, P]
        L.sp24_validate_meta.restype = I
        L.sp24_status_string.argtypes = [I]
        L.sp24_status_string.restype = ctypes.c_char_p
        L.sp24_version.argtypes = []
        L.sp24_version.restype = I
        L.sp24_calib_stream.argtypes = [P, ctypes.c_uint64, P, ctypes.c_uint64, P, I, I, P]
        L.sp24_calib_stream.restype = I
        U64 = ctypes.c_uint64
        L.sp24_calib_mfma.argtypes = [P, U64, P, U64, P, U64, I, I, I, I, P, P]
        L.sp24_calib_mfma.restype = I
        L.sp24_calib_mfma_ex.argtypes = [P, U64, P, U64, P, U64, I, I, I, I, I, P, U64, P, P]
        L.sp24_calib_mfma_ex.restype = I
        _lib = L
    return _lib


# ---- one-to-one C ABI mirrors ------------------------------------------------
def sp24_values_bytes(M: int, K: int, dtype: int, layout: int) -> int:
    return lib().sp24_values_bytes(M, K, dtype, layout)


def sp24_meta_bytes(M: int, K: int, dtype: int, layout: int) -> int:
    return lib().sp24_meta_bytes(M, K, dtype, layout)


def sp24_gemm_workspace_bytes(M: int, N: int, K: int, a_type: int, b_type: int) -> int:
    return lib().sp24_gemm_workspace_bytes(M, N, K, a_type, b_type)


def sp24_prune_compress(A: int, A_vals: int, meta: int, M: int, K: int, dtype: int, layout: int,
                        stream: int | None) -> int:
    return lib().sp24_prune_compress(A, A_vals, meta, M, K, dtype, layout, stream)


def sp24_gemm(A_vals: int, meta: int, a_type: int, layout: int, B: int, b_type: int, b_layout: int, C: int, M: int,
              N: int, K: int, alpha: float, beta: float, workspace: int | None, workspace_bytes: int,
              stream: int | None) -> int:
    return lib().sp24_gemm(A_vals, meta, a_type, layout, B, b_type, b_layout, C, M, N, K, alpha, beta, workspace,
                           workspace_bytes, stream)


def sp24_gemm_ex(A_vals: int, meta: int, a_type: int, layout: int, B: int, b_type: int, b_layout: int, C: int,
                 c_type: int, bias: int | None, M: int, N: int, K: int, alpha: float, beta: float,
                 workspace: int | None, workspace_bytes: int, stream: int | None) -> int:
    return lib().sp24_gemm_ex(A_vals, meta, a_type, layout, B, b_type, b_layout, C, c_type, bias, M, N, K, alpha,
                              beta, workspace, workspace_bytes, stream)


def sp24_decompress(A_vals: int, meta: int, A: int, M: int, K: int, dtype: int, layout: int,
                    stream: int | None) -> int:
    return lib().sp24_decompress(A_vals, meta, A, M, K, dtype, layout, stream)


def sp24_validate_meta(meta: int, M: int, K: int, dtype: int, layout: int, bad_groups: int,
                       stream: int | None) -> int:
    return lib().sp24_validate_meta(meta, M, K, dtype, layout, bad_groups, stream)


def sp24_status_string(status: int) -> str:
    return lib().sp24_status_string(status).decode()


def sp24_calib_stream(src: int, read_bytes: int, dst: int, write_bytes: int, sink: int, workgroups: int,
                      threads: int, stream) -> int:
    """Measurement aid (include/sp24_calib.h): a plain HBM stream."""
    return lib().sp24_calib_stream(src, read_bytes, dst, write_bytes, sink, workgroups, threads, stream)


def sp24_calib_mfma(a_vals: int, a_bytes: int, codes: int, code_bytes: int, b: int, b_bytes: int, a_type: int,
                    b_type: int, rounds: int, workgroups: int, sink: int, stream) -> int:
    """Measurement aid (include/sp24_calib.h): the product's sparse-MFMA
    instruction stream with its operands in registers."""
    return lib().sp24_calib_mfma(a_vals, a_bytes, codes, code_bytes, b, b_bytes, a_type, b_type, rounds, workgroups,
                                 sink, stream)


def sp24_calib_mfma_ex(a_vals: int, a_bytes: int, codes: int, code_bytes: int, b: int, b_bytes: int, a_type: int,
                       b_type: int, rounds: int, workgroups: int, shape: int, load_src, load_src_bytes: int,
                       sink: int, stream) -> int:
    """Measurement aid (include/sp24_calib.h): sp24_calib_mfma with the
    32x32 instruction shape and / or the product's direct-to-LDS loads."""
    return lib().sp24_calib_mfma_ex(a_vals, a_bytes, codes, code_bytes, b, b_bytes, a_type, b_type, rounds,
                                    workgroups, shape, load_src, load_src_bytes, sink, stream)


def sp24_version() -> int:
    return lib().sp24_version()


# ---- torch conveniences -------------------------------------------------------
def torch_dtype(code: int):
    import torch
    return {SP24_F16: torch.float16, SP24_BF16: torch.bfloat16, SP24_I8: torch.int8,
            SP24_FP8_E4M3: torch.float8_e4m3fn, SP24_BF8_E5M2: torch.float8_e5m2}[code]


def dtype_code(t) -> int:
    import torch
    m = {torch.float16: SP24_F16, torch.bfloat16: SP24_BF16, torch.int8: SP24_I8,
         torch.float8_e4m3fn: SP24_FP8_E4M3, torch.float8_e5m2: SP24_BF8_E5M2}
    if t not in m:
        raise TypeError(f"unsupported element type {t}")
    return m[t]


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def kblock_width(dtype: int) -> int:
    """Dense K columns per block of the K-blocked layout: 64 (16-bit types) or 128 (8-bit)."""
    return 64 if _ESIZE[dtype] == 2 else 128


def compressed_shapes(M: int, K: int, dtype: int, layout: int):
    """Tensor shapes (values in elements of ``dtype``, metadata in 32-bit words)
    of a compressed M x K matrix in ``layout``."""
    if layout == SP24_LAYOUT_ROW:
        return (M, K // 2), (M, K // 32)
    if layout == SP24_LAYOUT_KBLOCK:
        kb = kblock_width(dtype)
        nblk = -(-K // kb)
        mp = -(-M // 128) * 128  # metadata rows are padded to whole 128-row groups
        return (nblk, M, kb // 2), (nblk, mp, kb // 32)
    raise ValueError(f"unknown layout {layout}")


def prune_compress(A, dtype: int | None = None, layout: int = SP24_LAYOUT_KBLOCK, stream=None):
    """A: M x K device tensor (any 1- or 2-byte dtype holding the bits of
    ``dtype``).  Returns (A_vals, meta) in ``layout``: ROW gives M x K/2 values
    and M x K/32 metadata words; KBLOCK gives nblk x M x KB/2 values and
    nblk x Mp x KB/32 words (KB = kblock_width(dtype), Mp = M rounded up to
    128, words interleaved in 128-row groups as include/sp24.h describes).
    Metadata words are uint32 held in int32 tensors."""
    import torch
    if dtype is None:
        dtype = dtype_code(A.dtype)
    if A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be a contiguous 2-D tensor")
    M, K = A.shape
    vshape, mshape = compressed_shapes(M, K, dtype, layout)
    vals = torch.empty(vshape, dtype=A.dtype, device=A.device)
    meta = torch.empty(mshape, dtype=torch.int32, device=A.device)
    st = sp24_prune_compress(A.data_ptr(), vals.data_ptr(), meta.data_ptr(), M, K, dtype, layout, _stream(stream))
    if st != SP24_OK:
        raise Sp24Error(st, "sp24_prune_compress")
    return vals, meta


def gemm(A_vals, meta, B, C=None, alpha: float = 1.0, beta: float = 0.0, a_type: int | None = None,
         b_type: int | None = None, layout: int | None = None, stream=None, out_dtype=None, bias=None,
         workspace=None):
    """D = alpha * expand(A_vals, meta) @ B + beta * C (+ bias), written into C
    (allocated, uninitialised, when C is None and beta == 0).  ``layout``
    defaults to what the tensors' rank says: 2-D = ROW, 3-D = KBLOCK.
    B is K x N: either contiguous (SP24_B_KN) or the transpose of a
    contiguous N x K tensor, e.g. ``X.t()`` for activations X (SP24_B_NK).
    ``out_dtype`` (torch.float32 by default, or float16 / bfloat16; int32 for
    int8 inputs) is the type of C / D, taken from C when it is given.
    ``bias``: optional length-N float32 tensor added to every row (calls
    sp24_gemm_ex).  ``workspace``: optional uint8 device tensor of at least
    sp24_gemm_workspace_bytes() bytes, which is 0 for every problem at
    present; allocated per call when needed and not given.  Returns C."""
    import torch
    if a_type is None:
        a_type = dtype_code(A_vals.dtype)
    if b_type is None:
        b_type = dtype_code(B.dtype)
    if layout is None:
        layout = SP24_LAYOUT_KBLOCK if A_vals.dim() == 3 else SP24_LAYOUT_ROW
    K, N = B.shape
    if B.is_contiguous():
        b_layout = SP24_B_KN
    elif B.t().is_contiguous():
        b_layout = SP24_B_NK
    else:
        raise ValueError("B must be contiguous or the transpose of a contiguous tensor")
    M = A_vals.shape[0] if layout == SP24_LAYOUT_ROW else A_vals.shape[1]
    vshape, mshape = compressed_shapes(M, K, a_type, layout)
    if tuple(A_vals.shape) != vshape or tuple(meta.shape) != mshape:
        raise ValueError(f"compressed A has shapes {tuple(A_vals.shape)} / {tuple(meta.shape)}; "
                         f"K = {K} in this layout needs {vshape} / {mshape}")
    is_int = a_type == SP24_I8 and b_type == SP24_I8
    if out_dtype is None:
        out_dtype = C.dtype if C is not None else (torch.int32 if is_int else torch.float32)
    c_type = {torch.float32: SP24_F32, torch.float16: SP24_F16, torch.bfloat16: SP24_BF16,
              torch.int32: SP24_I32}.get(out_dtype)
    if c_type is None:
        raise TypeError(f"unsupported output type {out_dtype}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=out_dtype, device=B.device)
    elif C.dtype != out_dtype:
        raise TypeError(f"C is {C.dtype}, output type is {out_dtype}")
    for t in (A_vals, meta, C):
        if not t.is_contiguous():
            raise ValueError("A_vals, meta and C must be contiguous")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous() or bias.numel() != N):
        raise ValueError("bias must be a contiguous float32 tensor of N values")
    # a workspace only if the library asks for one (no kernel uses one at
    # present)
    ws_bytes = sp24_gemm_workspace_bytes(M, N, K, a_type, b_type)
    if workspace is None and ws_bytes:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=B.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if bias is None and c_type == (SP24_I32 if is_int else SP24_F32):
        st = sp24_gemm(A_vals.data_ptr(), meta.data_ptr(), a_type, layout, B.data_ptr(), b_type, b_layout,
                       C.data_ptr(), M, N, K, float(alpha), float(beta), ws_ptr, ws_len, _stream(stream))
        what = "sp24_gemm"
    else:
        st = sp24_gemm_ex(A_vals.data_ptr(), meta.data_ptr(), a_type, layout, B.data_ptr(), b_type, b_layout,
                          C.data_ptr(), c_type, None if bias is None else bias.data_ptr(), M, N, K, float(alpha),
                          float(beta), ws_ptr, ws_len, _stream(stream))
        what = "sp24_gemm_ex"
    if st != SP24_OK:
        raise Sp24Error(st, what)
    return C


def decompress(A_vals, meta, K: int, dtype: int | None = None, layout: int | None = None, stream=None):
    """Dense M x K tensor (same element type as A_vals) from compressed A.
    ``layout`` defaults to what the tensors' rank says: 2-D = ROW, 3-D = KBLOCK."""
    import torch
    if dtype is None:
        dtype = dtype_code(A_vals.dtype)
    if layout is None:
        layout = SP24_LAYOUT_KBLOCK if A_vals.dim() == 3 else SP24_LAYOUT_ROW
    M = A_vals.shape[0] if layout == SP24_LAYOUT_ROW else A_vals.shape[1]
    vshape, mshape = compressed_shapes(M, K, dtype, layout)
    if tuple(A_vals.shape) != vshape or tuple(meta.shape) != mshape:
        raise ValueError(f"compressed A has shapes {tuple(A_vals.shape)} / {tuple(meta.shape)}; "
                         f"K = {K} in this layout needs {vshape} / {mshape}")
    A = torch.empty((M, K), dtype=A_vals.dtype, device=A_vals.device)
    st = sp24_decompress(A_vals.data_ptr(), meta.data_ptr(), A.data_ptr(), M, K, dtype, layout, _stream(stream))
    if st != SP24_OK:
        raise Sp24Error(st, "sp24_decompress")
    return A


def validate_meta(meta, M: int, K: int, dtype: int, layout: int, stream=None):
    """Number of groups whose two codes are not strictly increasing (a device
    int64 tensor of one element, filled when the stream reaches the call)."""
    import torch
    out = torch.empty(1, dtype=torch.int64, device=meta.device)
    st = sp24_validate_meta(meta.data_ptr(), M, K, dtype, layout, out.data_ptr(), _stream(stream))
    if st != SP24_OK:
        raise Sp24Error(st, "sp24_validate_meta")
    return out
