"""Test helper: the K-blocked compressed layout restated from include/sp24.h.

Converts the oracle's row-major compressed output (M x K/2 values, M x K/32
metadata words) into the K-blocked layout: K is cut into blocks of KB dense
columns (64 for 16-bit types, 128 for 8-bit ones), block b of every row is
stored together (values [b, i, :] = row i's KB/2 compressed values of block
b; metadata [b, i, :] = its KB/32 words), and the tail of a partial last
block is zero.  Pure data movement: no arithmetic of the method.
"""
import numpy as np

from structured_sparse_matrix_sp24_amd import workloads as wl


def kblock_width(dtype):
    return 64 if wl.ESIZE[dtype] == 2 else 128


def row_to_kblock(vals, meta, dtype):
    M, KC = vals.shape
    KB = kblock_width(dtype)
    nblk = -(-2 * KC // KB)
    VE, W = KB // 2, KB // 32
    v = np.zeros((M, nblk * VE), vals.dtype)
    v[:, :KC] = vals
    m = np.zeros((M, nblk * W), np.uint32)
    m[:, :meta.shape[1]] = meta
    v = np.ascontiguousarray(v.reshape(M, nblk, VE).transpose(1, 0, 2))
    m = np.ascontiguousarray(m.reshape(M, nblk, W).transpose(1, 0, 2))
    return v, m
