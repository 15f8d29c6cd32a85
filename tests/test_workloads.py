"""Host checks of the seeded input generators (no GPU, no method arithmetic)."""
import numpy as np

from structured_sparse_matrix_sp24_amd import workloads as wl


def test_small_int_bits_is_seeded_and_in_range():
    a = wl.small_int_bits((7, 300), wl.F16, 3)
    b = wl.small_int_bits((7, 300), wl.F16, 3)
    c = wl.small_int_bits((7, 300), wl.F16, 4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    v = a.view(np.float16).astype(np.float64)
    assert set(np.unique(v)) <= {-1.0, 0.0, 1.0}
    i8 = wl.small_int_bits((5, 64), wl.I8, 1, -127, 127)
    assert i8.dtype == np.int8 and i8.min() >= -127 and i8.max() <= 127


def test_small_int_bits_formats_are_exact():
    """The same integers, stored in each format, decode to the same values."""
    ints = wl.small_int_bits((4, 96), wl.I8, 9, -4, 4).astype(np.float64)
    f16 = wl.small_int_bits((4, 96), wl.F16, 9, -4, 4).view(np.float16).astype(np.float64)
    bf16 = (wl.small_int_bits((4, 96), wl.BF16, 9, -4, 4).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(ints, f16) and np.array_equal(ints, bf16.astype(np.float64))


def test_small_int_bits_repeats_one_prime_block():
    """Element (i, j) is block[(i * cols + j) mod 1,000,003]: the flat sequence
    repeats with that period and with no shorter one at the start."""
    P = 1_000_003
    x = wl.small_int_bits((3, P), wl.I8, 2, -127, 127)
    flat = x.reshape(-1)
    assert np.array_equal(flat[:P], flat[P:2 * P]) and np.array_equal(flat[:P], flat[2 * P:])
    assert not np.array_equal(flat[:1000], flat[256:1256])
