"""Host replay of the K-blocked decompress launches' index arithmetic.

Each (workgroup, thread, round) of a launch is mapped, with the kernel's own
integer expressions transcribed here, to the bytes it reads (8 bytes of
compressed values, 1 or 2 bytes of codes) and the 16-byte chunk of dense A
it writes.  The replay then checks, for whole launches:

  * every 16-byte chunk of A is written exactly once (no chunk twice, none
    missing);
  * the values a chunk is built from are its own row's compressed elements
    for its columns, and the code bytes are its own row's codes for them.
    Both are located through tests/layouts.py (the K-blocked layout restated
    from the header): tables whose entries encode (row, element) or
    (row, code byte) are moved into the K-blocked layout there and read back
    at the replayed addresses, so the check does not reuse the kernel's
    address formulas.

Two index maps are replayed at 8192 x 8192 (fp16 and int8, the sizes of the
benchmark's A) and on ragged shapes:
  * the current kernel (decompress_kblock_kernel<ES, NB, T> in
    csrc/sp24_decompress.hip, with the launch shape its host code picks);
  * the kernel it replaced (commit d3c04ff), whose output on the GPU at
    8192 x 8192 differed from run to run in a few hundred to tens of
    thousands of elements.
Both maps pass: every chunk is written once, from the right bytes.  So that
run-to-run difference did not come from the old kernel's index arithmetic
(which, compiled for gfx950, also issues its loads and stores at these
addresses with the waits in place); it is recorded as unexplained.
"""
import numpy as np
import pytest

from layouts import row_to_kblock
from structured_sparse_matrix_sp24_amd import workloads as wl


def _launch_shape_current(M, K, es):
    """Blocks per workgroup and threads, as the host code chooses them."""
    kb = 64 if es == 2 else 128
    nblk, row_tiles = -(-K // kb), -(-M // 128)
    nb = 2 if es == 2 and row_tiles * ((nblk + 1) // 2) >= 1024 else 1
    return nb, 512


def map_current(M, K, es):
    """(active, value byte address, code byte address, store byte address)
    for every (workgroup, thread, round) of the current kernel."""
    NB, T = _launch_shape_current(M, K, es)
    MB, CE = (8, 8) if es == 2 else (16, 16)
    CPR = 8 * NB
    RPR = T // CPR
    NR = 128 // RPR
    nblk = -(-K // (64 if es == 2 else 128))
    nwb = -(-nblk // NB)
    G = -(-M // 128) * nwb
    Mp = -(-M // 128) * 128
    blk = np.arange(G, dtype=np.int64)[:, None, None]
    t = np.arange(T, dtype=np.int64)[None, :, None]
    u = np.arange(NR, dtype=np.int64)[None, None, :]
    b = (blk % nwb) * NB + (t % CPR) // 8
    rt = blk // nwb
    c = t & 7
    kcol = b * (8 * CE) + c * CE
    row0 = rt * 128
    rows_here = np.minimum(M - row0, 128)
    r_first = t // CPR
    rr = r_first + RPR * u
    active = (kcol < K) & (rr < rows_here)
    src = (b * M + row0 + r_first) * 64 + c * 8
    dst = (row0 + r_first) * K * es + kcol * es
    tt, r = rr >> 4, rr & 15
    mgroup = (b * Mp + rt * 128) * MB
    if es == 2:
        maddr = mgroup + (((r * 4 + c // 2) * 4 + tt // 2) * 2 + (tt & 1)) * 2 + (c & 1)
    else:
        maddr = mgroup + ((r * 4 + c // 2) * 8 + tt) * 4 + (c & 1) * 2
    vaddr = src + RPR * 64 * u
    saddr = dst + (RPR * u) * K * es
    return active, vaddr, maddr, saddr


def map_replaced(M, K, es):
    """The same for the kernel replaced in commit d3c04ff: 256 threads, one
    block per workgroup, every round's addresses recomputed from the row."""
    MB, CE = (8, 8) if es == 2 else (16, 16)
    nblk = -(-K // (64 if es == 2 else 128))
    G = -(-M // 128) * nblk
    Mp = -(-M // 128) * 128
    blk = np.arange(G, dtype=np.int64)[:, None, None]
    t = np.arange(256, dtype=np.int64)[None, :, None]
    u = np.arange(4, dtype=np.int64)[None, None, :]
    b = blk % nblk
    rt = blk // nblk
    c = t & 7
    kcol = b * (8 * CE) + c * CE
    rr = (t >> 3) + 32 * u
    row = rt * 128 + rr
    active = (kcol < K) & (row < M)
    tt, r = rr >> 4, rr & 15
    vaddr = (b * M + row) * 64 + c * 8
    mgroup = (b * Mp + rt * 128) * MB
    if es == 2:
        maddr = mgroup + (((r * 4 + c // 2) * 4 + tt // 2) * 2 + (tt & 1)) * 2 + (c & 1)
    else:
        maddr = mgroup + ((r * 4 + c // 2) * 8 + tt) * 4 + (c & 1) * 2
    saddr = row * K * es + kcol * es
    return active, vaddr, maddr, saddr


def _bytes_of(kblock_array):
    return np.ascontiguousarray(kblock_array).reshape(-1).view(np.uint8)


def check_map(M, K, dtype, mapper):
    es = wl.ESIZE[dtype]
    active, vaddr, maddr, saddr = (np.broadcast_to(a, np.broadcast_shapes(*(x.shape for x in mapper(M, K, es))))
                                   for a in mapper(M, K, es))
    vaddr, maddr, saddr = vaddr[active], maddr[active], saddr[active]
    # every 16-byte chunk of A written exactly once
    assert (saddr % 16 == 0).all()
    counts = np.bincount(saddr // 16, minlength=M * K * es // 16)
    assert counts.size == M * K * es // 16, "a store lands past the end of A"
    assert (counts == 1).all(), f"{int((counts == 0).sum())} chunks never written, {int((counts > 1).sum())} twice"
    row = saddr // (K * es)
    kcol = (saddr % (K * es)) // es
    KC = K // 2
    n_el = 8 // es                          # compressed elements read per chunk
    first = kcol // 2                       # first compressed element of the chunk
    store = wl.STORE[dtype]
    zero_meta = np.zeros((M, K // 32), np.uint32)
    # values: tables holding row and element indices, one byte (8-bit types)
    # or one 16-bit word (16-bit types) of the index at a time
    ri = np.broadcast_to(np.arange(M, dtype=np.int64)[:, None], (M, KC))
    ci = np.broadcast_to(np.arange(KC, dtype=np.int64)[None, :], (M, KC))
    width = 8 * es
    for idx_table, expect in ((ri, row[:, None] + 0 * np.arange(n_el)), (ci, first[:, None] + np.arange(n_el))):
        for shift in range(0, 16, width):
            part = ((idx_table >> shift) & ((1 << width) - 1)).astype(store)
            kv, _ = row_to_kblock(part, zero_meta, dtype)
            got = _bytes_of(kv)[vaddr[:, None] + np.arange(8)].view(np.uint8 if es == 1 else np.uint16)
            got = got.reshape(len(vaddr), n_el).astype(np.int64)
            assert np.array_equal(got, (expect >> shift) & ((1 << width) - 1)), "values read from the wrong place"
    # codes: row-major metadata bytes holding (row, byte index) one byte at a time
    nbytes = K // 8                         # metadata bytes per row
    per_chunk = 1 if es == 2 else 2
    qb = np.broadcast_to(np.arange(nbytes, dtype=np.int64)[None, :], (M, nbytes))
    rb = np.broadcast_to(np.arange(M, dtype=np.int64)[:, None], (M, nbytes))
    zero_vals = np.zeros((M, KC), store)
    first_byte = kcol // 8                  # metadata byte of the chunk's first element
    for tab, expect in ((rb, row[:, None] + 0 * np.arange(per_chunk)),
                        (qb, first_byte[:, None] + np.arange(per_chunk))):
        for shift in (0, 8):
            m_row = np.ascontiguousarray(((tab >> shift) & 255).astype(np.uint8)).view(np.uint32)
            _, km = row_to_kblock(zero_vals, m_row, dtype)
            got = _bytes_of(km)[maddr[:, None] + np.arange(per_chunk)].astype(np.int64)
            assert np.array_equal(got, (expect >> shift) & 255), "codes read from the wrong place"


@pytest.mark.parametrize("mapper", [map_current, map_replaced])
@pytest.mark.parametrize("dtype", [wl.F16, wl.I8])
@pytest.mark.parametrize("shape", [(300, 160), (4136, 4128), (129, 8224)])
def test_decompress_kblock_map_ragged(dtype, shape, mapper):
    check_map(*shape, dtype, mapper)


@pytest.mark.slow
@pytest.mark.parametrize("mapper", [map_current, map_replaced])
@pytest.mark.parametrize("dtype", [wl.F16, wl.I8])
def test_decompress_kblock_map_full_size(dtype, mapper):
    """The 8192 x 8192 launch the old kernel got wrong on the GPU."""
    check_map(8192, 8192, dtype, mapper)


def test_replay_catches_a_planted_error():
    """The checks see an index mistake: a map that writes every row tile's
    last round one row too far down (so one row is written twice and another
    never) fails."""
    def bad(M, K, es):
        active, vaddr, maddr, saddr = map_replaced(M, K, es)
        saddr = np.where(np.arange(4)[None, None, :] == 3, saddr + K * es * (np.arange(4) == 3), saddr)
        return active, vaddr, maddr, saddr
    with pytest.raises(AssertionError):
        check_map(300, 160, wl.F16, bad)
