"""The K-blocked layout helper used by the parity tests, checked element by
element against the index formulas stated in include/sp24.h (CPU only)."""
import numpy as np
import pytest

from layouts import row_to_kblock
from structured_sparse_matrix_sp24_amd import workloads as wl


@pytest.mark.parametrize("dtype,M,K", [(wl.F16, 200, 224), (wl.BF16, 128, 64), (wl.I8, 37, 416), (wl.E5M2, 300, 128)])
def test_kblock_helper_matches_header_formulas(dtype, M, K):
    rng = np.random.default_rng(1)
    es = wl.ESIZE[dtype]
    vals = rng.integers(0, 2 ** (8 * es - 1), (M, K // 2)).astype(np.uint16 if es == 2 else np.uint8)
    meta = rng.integers(0, 2 ** 32, (M, K // 32), dtype=np.uint64).astype(np.uint32)
    v, m = row_to_kblock(vals, meta, dtype)
    KB = 64 if es == 2 else 128
    W, VE = KB // 32, KB // 2
    nblk = -(-K // KB)
    Mp = -(-M // 128) * 128
    assert v.shape == (nblk, M, VE) and m.shape == (nblk, Mp, W)
    for b in range(nblk):
        seg = vals[:, b * VE:(b + 1) * VE]
        assert np.array_equal(v[b, :, :seg.shape[1]], seg)
        assert not v[b, :, seg.shape[1]:].any()
        flat = m[b].reshape(-1)
        for i in range(Mp):
            words = np.zeros(W, np.uint32)
            if i < M:
                s = meta[i, b * W:(b + 1) * W]
                words[:len(s)] = s
            p, rr = divmod(i, 128)
            t, r = divmod(rr, 16)
            if es == 2:
                f16 = flat.view(np.uint16)
                for g in range(4):
                    assert f16[p * 512 + ((r * 4 + g) * 4 + t // 2) * 2 + t % 2] == words.view(np.uint16)[g]
            else:
                for g in range(4):
                    assert flat[p * 512 + (r * 4 + g) * 8 + t] == words[g]
