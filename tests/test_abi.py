"""C ABI checks that need no GPU: the library loads, exports every function
include/sp24.h declares, and rejects bad arguments on the host before any
launch (fake pointers are never dereferenced on those paths)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from structured_sparse_matrix_sp24_amd import capi
    if not os.path.exists(capi.LIB_PATH):
        pytest.skip("libsp24.so not built")
    return capi


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(sp24_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) >= 9 and {"sp24_calib_stream", "sp24_calib_mfma"} <= set(names), names
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_calib_stream_argument_errors(L):
    f = L.sp24_calib_stream
    assert f(0, 64, P, 32, P, 4, 256, None) == 1           # null source
    assert f(P, 64, P, 96, P, 4, 256, None) == 1           # writes more than it reads
    assert f(P, 60, P, 32, P, 4, 256, None) == 1           # not a multiple of 16
    assert f(P, 64, P, 32, P, -1, 256, None) == 1          # negative workgroup count
    assert f(P, 64, P, 32, P, 4, 96, None) == 1            # threads not a multiple of 64
    assert f(P + 8, 64, P, 32, P, 4, 256, None) == 3       # misaligned
    assert f(P, 0, 0, 0, P, 4, 256, None) == 0             # nothing to do, nothing launched


def test_calib_mfma_argument_errors(L):
    f = L.sp24_calib_mfma
    F16, I8, BF = L.SP24_F16, L.SP24_I8, L.SP24_BF16
    A, Mt, B, S = P, 2 * P, 3 * P, 4 * P
    assert f(A, 8192, Mt, 2048, B, 8192, F16, BF, 1, 1, S, None) == 2          # mixed 16-bit pair
    assert f(A, 8192, Mt, 2048, B, 8192, F16, 99, 1, 1, S, None) == 2          # unknown type
    assert f(0, 8192, Mt, 2048, B, 8192, F16, F16, 1, 1, S, None) == 1         # null A
    assert f(A, 8192, Mt, 2048, B, 8192, I8, I8, 1, 1, 0, None) == 1           # null sink
    assert f(A, 8191, Mt, 2048, B, 8192, F16, F16, 1, 1, S, None) == 1         # fewer than 8 KiB of A
    assert f(A, 8192, Mt, 2047, B, 8192, F16, F16, 1, 1, S, None) == 1         # fewer than 2 KiB of codes
    assert f(A, 8192, Mt, 2048, B, 8191, F16, F16, 1, 1, S, None) == 1         # fewer than 8 KiB of B
    assert f(A, 8192, Mt, 2048, B, 8192, F16, F16, 0, 1, S, None) == 1         # rounds < 1
    assert f(A, 8192, Mt, 2048, B, 8192, F16, F16, 1, 0, S, None) == 1         # workgroups < 1
    assert f(A + 8, 8192, Mt, 2048, B, 8192, F16, F16, 1, 1, S, None) == 3     # misaligned


def test_calib_mfma_ex_argument_errors(L):
    f = L.sp24_calib_mfma_ex
    F16, I8 = L.SP24_F16, L.SP24_I8
    A, Mt, B, S, Src = P, 2 * P, 3 * P, 4 * P, 5 * P
    assert f(A, 8192, Mt, 2048, B, 8192, F16, F16, 1, 1, 8, None, 0, S, None) == 1      # shape 8
    assert f(A, 8192, Mt, 2048, B, 8192, F16, F16, 1, 1, 64, None, 0, S, None) == 1     # shape 64
    assert f(A, 8192, Mt, 2048, B, 8192, I8, I8, 1, 1, 32, Src, 1023, S, None) == 1     # load source < 1 KiB
    assert f(A, 8192, Mt, 2048, B, 8192, I8, I8, 1, 1, 32, Src + 4, 4096, S, None) == 3  # misaligned source
    assert f(A, 8192, Mt, 2048, B, 8192, F16, L.SP24_BF16, 1, 1, 32, None, 0, S, None) == 2  # mixed pair
    assert f(0, 8192, Mt, 2048, B, 8192, F16, F16, 1, 1, 16, Src, 4096, S, None) == 1   # null A


def test_size_queries(L):
    ROW, KB = L.SP24_LAYOUT_ROW, L.SP24_LAYOUT_KBLOCK
    assert L.sp24_values_bytes(8192, 8192, L.SP24_F16, ROW) == 8192 * 4096 * 2
    assert L.sp24_values_bytes(8192, 16384, L.SP24_FP8_E4M3, ROW) == 8192 * 8192
    assert L.sp24_meta_bytes(8192, 8192, L.SP24_F16, ROW) == 8192 * 8192 // 8
    # K-blocked: whole blocks of 64 B values per row, and 8 / 16 B of metadata
    # per row with the rows padded to a multiple of 128
    assert L.sp24_values_bytes(8192, 8192, L.SP24_F16, KB) == 8192 * 4096 * 2
    assert L.sp24_meta_bytes(8192, 8192, L.SP24_F16, KB) == 8192 * 8192 // 8
    assert L.sp24_values_bytes(10, 96, L.SP24_BF16, KB) == 2 * 10 * 64       # 96 = 1.5 blocks of 64
    assert L.sp24_meta_bytes(10, 96, L.SP24_BF16, KB) == 2 * 128 * 8
    assert L.sp24_values_bytes(10, 160, L.SP24_I8, KB) == 2 * 10 * 64        # 160 = 1.25 blocks of 128
    assert L.sp24_meta_bytes(10, 160, L.SP24_I8, KB) == 2 * 128 * 16
    assert L.sp24_meta_bytes(129, 64, L.SP24_F16, KB) == 1 * 256 * 8
    assert L.sp24_values_bytes(4, 64, 99, ROW) == 0
    assert L.sp24_values_bytes(4, 64, L.SP24_F16, 7) == 0
    assert L.sp24_gemm_workspace_bytes(8192, 8192, 8192, L.SP24_F16, L.SP24_F16) == 0
    assert L.sp24_version() >= 200


def test_compressed_shapes_match_size_queries(L):
    for dtype in (L.SP24_F16, L.SP24_I8):
        for layout in (L.SP24_LAYOUT_ROW, L.SP24_LAYOUT_KBLOCK):
            for M, K in [(1, 32), (7, 96), (300, 4096), (5, 160)]:
                vs, ms = L.compressed_shapes(M, K, dtype, layout)
                es = 2 if dtype == L.SP24_F16 else 1
                assert int(np.prod(vs)) * es == L.sp24_values_bytes(M, K, dtype, layout)
                assert int(np.prod(ms)) * 4 == L.sp24_meta_bytes(M, K, dtype, layout)


def test_status_strings(L):
    assert L.sp24_status_string(0) == "SP24_OK"
    assert L.sp24_status_string(3) == "SP24_ERR_MISALIGNED"
    assert L.sp24_status_string(1234) == "SP24_ERR_UNKNOWN"


P = 1 << 20  # fake, 16-byte aligned device addresses: never touched on the error paths


def test_prune_compress_argument_errors(L):
    f = L.sp24_prune_compress
    for lay in (L.SP24_LAYOUT_ROW, L.SP24_LAYOUT_KBLOCK):
        assert f(P, 2 * P, 3 * P, 4, 48, L.SP24_F16, lay, None) == 1            # K % 32
        assert f(P, 2 * P, 3 * P, -1, 64, L.SP24_F16, lay, None) == 1           # negative M
        assert f(P, 2 * P, 3 * P, 4, 64, 9, lay, None) == 2                     # unknown dtype
        assert f(P + 8, 2 * P, 3 * P, 4, 64, L.SP24_F16, lay, None) == 3        # misaligned
        assert f(P, P + 256, 3 * P, 4, 64, L.SP24_F16, lay, None) == 1          # A overlaps A_vals
        assert f(0, 2 * P, 3 * P, 4, 64, L.SP24_F16, lay, None) == 1            # null
        assert f(0, 0, 0, 0, 64, L.SP24_F16, lay, None) == 0                    # empty: nothing enqueued
    assert f(P, 2 * P, 3 * P, 4, 64, L.SP24_F16, 2, None) == 2                  # unknown layout
    # K-blocked values of 4 rows x 96 columns take 2 blocks = 512 B: meta right after 256 B overlaps
    assert f(P, 2 * P, 2 * P + 256, 4, 96, L.SP24_F16, L.SP24_LAYOUT_KBLOCK, None) == 1
    # its metadata takes 2 blocks x 128 padded rows x 8 B = 2 KiB: values 1 KiB after it overlap
    assert f(P, 3 * P + 1024, 3 * P, 4, 96, L.SP24_F16, L.SP24_LAYOUT_KBLOCK, None) == 1


def test_gemm_argument_errors(L):
    F16, I8, E4, E5, BF = L.SP24_F16, L.SP24_I8, L.SP24_FP8_E4M3, L.SP24_BF8_E5M2, L.SP24_BF16
    A, Mt, B, C = P, 2 * P, 3 * P, 8 * P
    for lay in (L.SP24_LAYOUT_ROW, L.SP24_LAYOUT_KBLOCK):
        def g(a, m, at, b, bt, c, *rest, bl=L.SP24_B_KN):
            return L.sp24_gemm(a, m, at, lay, b, bt, bl, c, *rest)
        assert g(A, Mt, F16, B, BF, C, 64, 64, 64, 1.0, 0.0, None, 0, None) == 2   # mixed 16-bit pair
        assert g(A, Mt, F16, B, E4, C, 64, 64, 64, 1.0, 0.0, None, 0, None) == 2
        assert g(A, Mt, I8, B, F16, C, 64, 64, 64, 1.0, 0.0, None, 0, None) == 2
        assert g(A, Mt, F16, B, F16, C, 64, 64, 48, 1.0, 0.0, None, 0, None) == 1   # K % 32
        assert g(A, Mt, F16, B, F16, C, 64, 12, 64, 1.0, 0.0, None, 0, None) == 2   # N % 8
        assert g(A, Mt, E4, B, E5, C, 64, 20, 64, 1.0, 0.0, None, 0, None) == 2     # N % 8
        # 8-bit B stored K x N: N % 8 up to 64 (small-N kernel), N % 16 above
        assert g(A, Mt, E4, B, E5, C, 64, 72, 64, 1.0, 0.0, None, 0, None) == 2
        assert g(A, Mt, E4, B, E5, C, 0, 72, 64, 1.0, 0.0, None, 0, None, bl=L.SP24_B_NK) == 0
        assert g(A, Mt, I8, B, I8, C, 0, 24, 64, 1.0, 0.0, None, 0, None) == 0
        assert g(A, Mt, I8, B, I8, C, 0, 72, 64, 1.0, 0.0, None, 0, None) == 2
        assert g(A, Mt, I8, B, I8, C, 64, 64, 64, 2.0, 0.0, None, 0, None) == 2     # int8 alpha
        assert g(A, Mt, I8, B, I8, C, 64, 64, 64, 1.0, 0.5, None, 0, None) == 2     # int8 beta
        assert g(A, Mt, F16, B, F16, C + 4, 64, 64, 64, 1.0, 0.0, None, 0, None) == 3
        assert g(A, Mt, F16, B, F16, B + 64, 64, 64, 64, 1.0, 0.0, None, 0, None) == 1  # C overlaps B
        assert g(A, Mt, F16, B, F16, 0, 64, 64, 64, 1.0, 0.0, None, 0, None) == 1       # null C
        assert g(A, Mt, F16, B, F16, C, 0, 64, 64, 1.0, 0.0, None, 0, None) == 0        # M == 0
        assert g(A, Mt, F16, B, F16, C, 64, 0, 64, 1.0, 0.0, None, 0, None) == 0        # N == 0
        assert g(A, Mt, F16, B, F16, C, -4, 64, 64, 1.0, 0.0, None, 0, None) == 1
        assert g(A, Mt, F16, B, F16, C, 64, 1 << 23, 64, 1.0, 0.0, None, 0, None) == 2  # 128 rows of B > 2 GiB
        assert g(A, Mt, F16, B, F16, C, 64, 64, 64, 1.0, 0.0, None, 0, None, bl=2) == 2  # unknown B layout
        assert g(A, Mt, F16, B, F16, B + 64, 64, 64, 64, 1.0, 0.0, None, 0, None, bl=L.SP24_B_NK) == 1
        # B stored N x K: 256 of its rows are addressed with 32-bit offsets, so K is bounded
        assert g(A, Mt, F16, B, F16, C, 0, 64, 1 << 22, 1.0, 0.0, None, 0, None, bl=L.SP24_B_NK) == 2
        assert g(A, Mt, F16, B, F16, C, 0, 64, 1 << 22, 1.0, 0.0, None, 0, None) == 0
        # every documented pair passes validation up to the launch (checked with M == 0)
        for a, b in [(F16, F16), (BF, BF), (I8, I8), (E4, E4), (E4, E5), (E5, E4), (E5, E5)]:
            for bl in (L.SP24_B_KN, L.SP24_B_NK):
                assert g(A, Mt, a, B, b, C, 0, 64, 64, 1.0, 0.0, None, 0, None, bl=bl) == 0
    assert L.sp24_gemm(A, Mt, F16, 5, B, F16, 0, C, 64, 64, 64, 1.0, 0.0, None, 0, None) == 2   # unknown layout
    # the row-major layout addresses a 256-row tile with 32-bit offsets: K is bounded
    big_k = 1 << 23
    assert L.sp24_gemm(A, Mt, F16, L.SP24_LAYOUT_ROW, B, F16, 0, C, 64, 64, big_k, 1.0, 0.0, None, 0, None) == 2


def test_gemm_ex_argument_errors(L):
    P = 1 << 20
    F16, BF, I8, E4, E5 = L.SP24_F16, L.SP24_BF16, L.SP24_I8, L.SP24_FP8_E4M3, L.SP24_BF8_E5M2
    F32, I32 = L.SP24_F32, L.SP24_I32
    A, Mt, B, C, bias = P, 2 * P, 3 * P, 8 * P, 16 * P
    lay, kn = L.SP24_LAYOUT_KBLOCK, L.SP24_B_KN

    def g(at, bt, ct, bi, M=0, alpha=1.0, beta=0.0, c=C):
        return L.sp24_gemm_ex(A, Mt, at, lay, B, bt, kn, c, ct, bi, M, 64, 64, alpha, beta, None, 0, None)
    # allowed output types pass validation up to the launch (M == 0)
    for at, bt in [(F16, F16), (BF, BF), (E4, E5), (E5, E5)]:
        for ct in (F32, F16, BF):
            assert g(at, bt, ct, None) == 0
            assert g(at, bt, ct, bias) == 0
    assert g(I8, I8, I32, None) == 0
    # int8 writes int32 only, without a bias; float inputs never write int32
    assert g(I8, I8, F32, None) == 2
    assert g(I8, I8, F16, None) == 2
    assert g(I8, I8, I32, bias) == 2
    assert g(F16, F16, I32, None) == 2
    assert g(F16, F16, E4, None) == 2
    assert g(F16, F16, 99, None) == 2
    # misaligned bias, bias overlapping C
    assert g(F16, F16, F16, bias + 4, M=64) == 3
    assert g(F16, F16, F16, C + 64 * 64, M=64) == 1        # bias is the last bytes of a 64x64 fp16 C
    # (a bias right after a 16-bit C, which does not overlap it, is checked on
    # the GPU with real adjacent buffers: test_gpu_parity.py)


def test_decompress_and_validate_argument_errors(L):
    d, v = L.sp24_decompress, L.sp24_validate_meta
    KB, ROW, F16 = L.SP24_LAYOUT_KBLOCK, L.SP24_LAYOUT_ROW, L.SP24_F16
    for lay in (ROW, KB):
        assert d(P, 2 * P, 3 * P, 4, 48, F16, lay, None) == 1          # K % 32
        assert d(P, 2 * P, 3 * P, 4, 64, 9, lay, None) == 2            # dtype
        assert d(P, 2 * P, 3 * P + 8, 4, 64, F16, lay, None) == 3      # misaligned A
        assert d(P, 2 * P, P + 64, 4, 64, F16, lay, None) == 1         # A overlaps A_vals
        assert d(0, 0, 0, 0, 64, F16, lay, None) == 0                  # empty
        assert v(P, 4, 64, F16, lay, 0, None) == 1                     # null counter
        assert v(P, 4, 64, F16, lay, 2 * P + 4, None) == 3             # counter not 8-byte aligned
        assert v(P, 4, 48, F16, lay, 2 * P, None) == 1                 # K % 32
        assert v(P, 4, 64, F16, 7, 2 * P, None) == 2                   # layout
