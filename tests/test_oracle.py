"""Pins for the CPU oracle: facts that do not come from the oracle's own code.

  * decode: every bit pattern of every format against torch's CPU decoder
    (a library routine), exhaustively;
  * pruning: brute force over all 4-tuples of an adversarial alphabet, checked
    against a dominance rule evaluated on torch-decoded magnitudes;
  * compression: the positions-0-and-2 pattern yields index bytes 0x88, the
    value the CDNA example kernels pass ("CDNA and CDNA2 sparse MFMA
    builtins", section "Using sparse MFMA builtins as a compute policy"); a
    hand-worked row (tests/golden/worked_example_k32.json); round trip against
    the original matrix; the generator's own int8 pattern;
  * product: dense float64 / int64 matmul of the decompressed matrix (library
    routine), identity B (the pages' verification trick: "RDNA4 dense WMMA
    builtins", section on the scalar fallback, checks C == A with B = I),
    one-hot brute force on a 16 x 16 x 32 tile, and epilogue special cases;
  * rounding to a 16-bit output: every fp16 value and tie against numpy's
    float64 -> float16 cast, float32 inputs against torch's bfloat16
    conversion, and tie closed forms.
"""
import json
import os

import numpy as np
import pytest
import torch

from structured_sparse_matrix_sp24_amd import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FLOAT_TYPES = [wl.F16, wl.BF16, wl.E4M3, wl.E5M2]
ALL_TYPES = FLOAT_TYPES + [wl.I8]
TORCH_VIEW = {wl.F16: (torch.int16, torch.float16), wl.BF16: (torch.int16, torch.bfloat16),
              wl.E4M3: (torch.uint8, torch.float8_e4m3fn), wl.E5M2: (torch.uint8, torch.float8_e5m2)}


def torch_decode(bits, dtype):
    """Independent decode through torch's CPU dtype views."""
    if dtype == wl.I8:
        return np.asarray(bits).view(np.int8).astype(np.float64)
    iv, fv = TORCH_VIEW[dtype]
    raw = np.ascontiguousarray(bits)
    raw = raw.view(np.int16) if iv == torch.int16 else raw.view(np.uint8)
    return torch.from_numpy(raw.copy()).view(fv).to(torch.float64).numpy()


def all_patterns(dtype):
    n = 65536 if wl.ESIZE[dtype] == 2 else 256
    return np.arange(n, dtype=np.int64).astype(wl.STORE[dtype] if dtype != wl.I8 else np.uint8).view(wl.STORE[dtype])


@pytest.mark.parametrize("dtype", FLOAT_TYPES + [wl.I8])
def test_decode_exhaustive_matches_torch(orc, dtype):
    bits = all_patterns(dtype)
    ours = orc.decode(bits, dtype)
    ref = torch_decode(bits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros must keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_format_landmarks(orc):
    # E4M3 "FN": 0x7E is the largest finite value 448, 0x7F is NaN (no Inf);
    # E5M2: 0x7B = 57344 max, 0x7C = Inf.  fp16 0x7BFF = 65504, bf16 0x3F80 = 1.
    assert orc.decode(np.array([0x7E], np.uint8), wl.E4M3)[0] == 448.0
    assert np.isnan(orc.decode(np.array([0x7F], np.uint8), wl.E4M3)[0])
    assert orc.decode(np.array([0x7B], np.uint8), wl.E5M2)[0] == 57344.0
    assert np.isinf(orc.decode(np.array([0x7C], np.uint8), wl.E5M2)[0])
    assert orc.decode(np.array([0x7BFF], np.uint16), wl.F16)[0] == 65504.0
    assert orc.decode(np.array([0x3F80], np.uint16), wl.BF16)[0] == 1.0
    assert orc.decode(np.array([0x01], np.uint8), wl.E4M3)[0] == 2.0 ** -9


def _alphabet(dtype):
    """9 values: +-0, ties, extremes, a subnormal and a NaN where the format has one."""
    if dtype == wl.I8:
        return np.array([0, 1, -1, 5, -5, 127, -127, -128, 2], dtype=np.int8)
    if dtype == wl.F16:
        v = [0x0000, 0x8000, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF, 0x0001, 0x7E00, 0x4000]
    elif dtype == wl.BF16:
        v = [0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F, 0x0001, 0x7FC0, 0x4000]
    elif dtype == wl.E4M3:
        v = [0x00, 0x80, 0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x7F, 0x40]
    else:
        v = [0x00, 0x80, 0x3C, 0xBC, 0x7B, 0xFB, 0x01, 0x7E, 0x40]
    return np.array(v, dtype=np.int64).astype(wl.STORE[dtype])


def _rank(vals, dtype):
    """Magnitude rank from torch-decoded values: NaN above everything, -0 == +0."""
    x = torch_decode(vals, dtype)
    return np.where(np.isnan(x), np.inf, np.abs(x)), np.isnan(x)


@pytest.mark.parametrize("dtype", ALL_TYPES)
def test_prune_bruteforce_dominance(orc, dtype):
    alpha = _alphabet(dtype)
    idx = np.indices((9, 9, 9, 9)).reshape(4, -1).T          # 6561 tuples
    pad = (-len(idx)) % 8
    idx = np.concatenate([idx, idx[:pad]])
    A = alpha[idx].reshape(-1, 32)
    vals, meta = orc.prune_compress(A, dtype)
    M = A.shape[0]
    codes = ((meta[:, :, None] >> (2 * np.arange(16, dtype=np.uint32))) & 3).reshape(M, 16)
    p0, p1 = codes[:, 0::2], codes[:, 1::2]                   # M x 8
    assert (p0 < p1).all(), "exactly two distinct kept slots, ascending"
    G = A.reshape(M, 8, 4)
    mag, isnan = _rank(G.reshape(-1), dtype)
    mag, isnan = mag.reshape(M, 8, 4), isnan.reshape(M, 8, 4)
    for g_row in range(M):
        for g in range(8):
            kept = (int(p0[g_row, g]), int(p1[g_row, g]))
            for k in kept:
                for d in set(range(4)) - set(kept):
                    mk, md = mag[g_row, g, k], mag[g_row, g, d]
                    nk, nd = isnan[g_row, g, k], isnan[g_row, g, d]
                    bigger = (nk and not nd) or (mk > md and not nd)
                    tie = (nk == nd) and (nk or mk == md)
                    assert bigger or (tie and k < d), (G[g_row, g], kept)
    # kept values are copied bit for bit, in ascending position order
    rows = np.arange(M)[:, None]
    grp = np.arange(8)[None, :]
    assert np.array_equal(vals[:, 0::2], G[rows, grp, p0])
    assert np.array_equal(vals[:, 1::2], G[rows, grp, p1])


@pytest.mark.parametrize("dtype", ALL_TYPES)
def test_round_trip_and_idempotence(orc, dtype):
    c = wl.random_case(7, 48, 8, 160, dtype, dtype)
    vals, meta = orc.prune_compress(c.A, dtype)
    dense = orc.decompress(vals, meta, dtype)
    M, K = c.A.shape
    codes = ((meta[:, :, None] >> (2 * np.arange(16, dtype=np.uint32))) & 3).reshape(M, K // 2)
    kept = np.zeros((M, K), bool)
    r = np.arange(M)[:, None]
    kept[r, 4 * (np.arange(K // 2) // 2)[None, :] + codes] = True
    assert (kept.reshape(M, K // 4, 4).sum(-1) == 2).all()
    A_u = c.A.view(np.uint8 if wl.ESIZE[dtype] == 1 else np.uint16)
    d_u = dense.view(A_u.dtype)
    assert np.array_equal(d_u[kept], A_u[kept]), "kept slots hold the original bits"
    assert (d_u[~kept] == 0).all(), "dropped slots hold +0"
    v2, m2 = orc.prune_compress(dense, dtype)
    assert np.array_equal(v2.view(A_u.dtype), vals.view(A_u.dtype)) and np.array_equal(m2, meta)


def test_tiny_config_fixed_pattern_is_0x88(orc):
    w = wl.make("tiny_f16")
    vals, meta = orc.prune_compress(w.A, wl.F16)
    assert meta.shape == (64, 4)
    assert (meta == 0x88888888).all()
    assert np.array_equal(vals[:, 0::2], w.A[:, 0::4])
    assert np.array_equal(vals[:, 1::2], w.A[:, 2::4])


def test_int8_metadata_equals_generated_pattern(orc):
    w = wl.make("i8_8192", M=64, K=256, N=32)
    vals, meta = orc.prune_compress(w.A, wl.I8)
    pairs = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])
    codes = ((meta[:, :, None] >> (2 * np.arange(16, dtype=np.uint32))) & 3).reshape(64, 128)
    pick = w.notes["pattern_pick"]
    assert np.array_equal(codes[:, 0::2], pairs[pick, 0])
    assert np.array_equal(codes[:, 1::2], pairs[pick, 1])
    assert (vals != 0).all()


def test_all_six_patterns_occur_evenly(orc):
    c = wl.random_case(3, 256, 8, 1024, wl.F16, wl.F16)
    _, meta = orc.prune_compress(c.A, wl.F16)
    nib = ((meta[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF).reshape(-1)
    counts = {int(v): int((nib == v).sum()) for v in np.unique(nib)}
    assert set(counts) == {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}
    for v in counts.values():
        assert abs(v / nib.size - 1 / 6) < 0.01


def test_golden_worked_example(orc):
    gold = json.load(open(os.path.join(GOLDEN, "worked_example_k32.json")))
    A = np.array([gold["A_row"]], dtype=np.int8)
    B = np.stack([np.arange(32) + 1, (-1) ** np.arange(32)], axis=1).astype(np.int8)
    for dtype in (wl.I8, wl.F16):
        Ab = A if dtype == wl.I8 else wl.quantize(A.astype(np.float64), dtype)
        Bb = B if dtype == wl.I8 else wl.quantize(B.astype(np.float64), dtype)
        vals, meta = orc.prune_compress(Ab, dtype)
        assert list(meta[0]) == gold["expected_meta"]
        assert list(orc.decode(vals, dtype)[0]) == gold["expected_vals"]
        if dtype == wl.I8:
            D = orc.gemm_i64(vals, meta, Bb)
        else:
            D, _ = orc.gemm_f64(vals, meta, dtype, Bb, dtype)
        assert list(D[0]) == gold["expected_D"]


@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.BF16, wl.BF16), (wl.E4M3, wl.E5M2),
                                           (wl.E5M2, wl.E5M2), (wl.E4M3, wl.E4M3), (wl.E5M2, wl.E4M3)])
def test_gemm_equals_dense_matmul(orc, a_type, b_type):
    c = wl.random_case(11, 40, 24, 96, a_type, b_type, beta=1.0, alpha=0.75)
    vals, meta = orc.prune_compress(c.A, a_type)
    D, S = orc.gemm_f64(vals, meta, a_type, c.B, b_type, c.C, alpha=0.75, beta=1.0)
    Ad = torch.from_numpy(torch_decode(orc.decompress(vals, meta, a_type), a_type))
    Bd = torch.from_numpy(torch_decode(c.B, b_type))
    ref = 0.75 * (Ad @ Bd).numpy() + 1.0 * c.C.astype(np.float64)
    absref = 0.75 * (Ad.abs() @ Bd.abs()).numpy() + np.abs(c.C.astype(np.float64))
    assert np.abs(D - ref).max() <= 1e-12 * absref.max()
    assert np.allclose(S, absref, rtol=1e-12, atol=0)


def test_gemm_int8_exact_and_beta(orc):
    c = wl.random_case(5, 33, 17, 128, wl.I8, wl.I8, beta=1.0)
    vals, meta = orc.prune_compress(c.A, wl.I8)
    Ad = torch.from_numpy(orc.decompress(vals, meta, wl.I8).astype(np.int64))
    Bd = torch.from_numpy(c.B.astype(np.int64))
    ref = (Ad @ Bd).numpy()
    assert np.array_equal(orc.gemm_i64(vals, meta, c.B), ref)
    assert np.array_equal(orc.gemm_i64(vals, meta, c.B, c.C, beta_one=True), ref + c.C)
    # worst case of the int8 configuration's size fits int32: (K/2) * 127^2
    K = 8192
    vals = np.full((1, K // 2), -127, np.int8)
    meta = np.full((1, K // 32), 0x88888888, np.uint32)
    B = np.full((K, 1), -127, np.int8)
    assert orc.gemm_i64(vals, meta, B)[0, 0] == (K // 2) * 127 * 127
    with pytest.raises(OverflowError):
        orc.gemm_i64(vals, meta, B, np.full((1, 1), 2**31 - 1000, np.int32), beta_one=True)


@pytest.mark.parametrize("dtype", FLOAT_TYPES)
def test_identity_B_returns_decompressed_A(orc, dtype):
    c = wl.random_case(2, 20, 64, 64, dtype, dtype)
    vals, meta = orc.prune_compress(c.A, dtype)
    one = wl.quantize(np.ones(1), dtype)[0]
    Bid = np.zeros((64, 64), dtype=wl.STORE[dtype])
    Bid[np.arange(64), np.arange(64)] = one
    D, _ = orc.gemm_f64(vals, meta, dtype, Bid, dtype)
    assert np.array_equal(D, torch_decode(orc.decompress(vals, meta, dtype), dtype))


def test_identity_B_int8(orc):
    c = wl.random_case(4, 20, 64, 64, wl.I8, wl.I8)
    vals, meta = orc.prune_compress(c.A, wl.I8)
    Bid = np.eye(64, dtype=np.int8)
    assert np.array_equal(orc.gemm_i64(vals, meta, Bid), orc.decompress(vals, meta, wl.I8).astype(np.int64))


def test_onehot_bruteforce_16x16x32(orc):
    rng = np.random.default_rng(0)
    nibs = np.array([0x4, 0x8, 0xC, 0x9, 0xD, 0xE], np.uint32)
    B = wl.quantize((np.arange(32 * 16) + 1).reshape(32, 16).astype(np.float64), wl.F16)  # exact ints
    Bv = torch_decode(B, wl.F16)
    one = wl.quantize(np.ones(1), wl.F16)[0]
    for i in range(16):
        for c in range(16):
            meta = np.zeros((16, 1), np.uint32)
            for r in range(16):
                for g in range(8):
                    meta[r, 0] |= nibs[rng.integers(0, 6)] << np.uint32(4 * g)
            vals = np.zeros((16, 16), np.uint16)
            vals[i, c] = one
            D, _ = orc.gemm_f64(vals, meta, wl.F16, B, wl.F16)
            code = int(meta[i, 0] >> np.uint32(2 * c)) & 3
            expect = np.zeros((16, 16))
            expect[i] = Bv[4 * (c // 2) + code]
            assert np.array_equal(D, expect)


def test_points_agree_with_full_product(orc):
    c = wl.random_case(9, 24, 40, 96, wl.BF16, wl.BF16, beta=0.5)
    vals, meta = orc.prune_compress(c.A, wl.BF16)
    D, S = orc.gemm_f64(vals, meta, wl.BF16, c.B, wl.BF16, c.C, beta=0.5)
    ii, jj = np.meshgrid(np.arange(24), np.arange(40), indexing="ij")
    P, PS = orc.gemm_points_f64(vals, meta, wl.BF16, c.B, wl.BF16, ii.ravel(), jj.ravel(), c.C, beta=0.5)
    assert np.array_equal(P, D.ravel()) and np.array_equal(PS, S.ravel())
    c8 = wl.random_case(9, 24, 40, 96, wl.I8, wl.I8, beta=1.0)
    v8, m8 = orc.prune_compress(c8.A, wl.I8)
    D8 = orc.gemm_i64(v8, m8, c8.B, c8.C, beta_one=True)
    P8 = orc.gemm_points_i64(v8, m8, c8.B, ii.ravel(), jj.ravel(), c8.C, beta_one=True)
    assert np.array_equal(P8, D8.ravel())


def test_epilogue_special_cases(orc):
    import ctypes
    c = wl.random_case(1, 8, 8, 32, wl.F16, wl.F16, beta=1.0)
    vals, meta = orc.prune_compress(c.A, wl.F16)
    D, _ = orc.gemm_f64(vals, meta, wl.F16, c.B, wl.F16, c.C, alpha=0.0, beta=2.0)
    assert np.array_equal(D, 2.0 * c.C.astype(np.float64))
    # beta == 0: C is never read, so NaN in C cannot reach D
    lib = orc._load()
    Cnan = np.full((8, 8), np.nan, np.float32)
    Dn = np.empty((8, 8), np.float64)
    rc = lib.orc_gemm_f64(vals.ctypes.data, meta.ctypes.data, wl.F16, c.B.ctypes.data, wl.F16,
                          Cnan.ctypes.data, None, Dn.ctypes.data, None, 8, 8, 32, 1.0, 0.0)
    assert rc == 0 and not np.isnan(Dn).any()


def test_bias_is_added_per_column(orc):
    """D with a bias = D without it + bias[j] in every row (and |bias| in the
    error scale); checked against the dense product, as the product pins do."""
    c = wl.random_case(21, 12, 40, 64, wl.BF16, wl.BF16, beta=1.0)
    vals, meta = orc.prune_compress(c.A, wl.BF16)
    bias = np.random.default_rng(3).standard_normal(40).astype(np.float32)
    D, S = orc.gemm_f64(vals, meta, wl.BF16, c.B, wl.BF16, c.C, alpha=-1.5, beta=0.5, bias=bias)
    Ad = torch.from_numpy(torch_decode(orc.decompress(vals, meta, wl.BF16), wl.BF16))
    Bd = torch.from_numpy(torch_decode(c.B, wl.BF16))
    ref = -1.5 * (Ad @ Bd).numpy() + 0.5 * c.C.astype(np.float64) + bias.astype(np.float64)[None, :]
    absref = 1.5 * (Ad.abs() @ Bd.abs()).numpy() + 0.5 * np.abs(c.C.astype(np.float64)) + \
        np.abs(bias.astype(np.float64))[None, :]
    assert np.abs(D - ref).max() <= 1e-12 * absref.max()
    assert np.allclose(S, absref, rtol=1e-12, atol=0)


# ---- rounding to a 16-bit output --------------------------------------------------
def _f16_grid_and_ties():
    """Every finite fp16 value, and every midpoint between neighbours (the ties),
    and points a hair either side of each midpoint."""
    v = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = (v[:-1] + v[1:]) / 2
    eps = np.abs(mid) * 2.0 ** -40 + 2.0 ** -1000
    return np.concatenate([v, mid, mid - eps, mid + eps])


def test_round_to_f16_matches_numpy(orc):
    """fp16: numpy's float64 -> float16 cast rounds directly, to nearest even
    (a library routine); checked on every value, every tie and its neighbours,
    both signs, random magnitudes from far below the subnormals to far beyond
    the largest finite value, and the special values."""
    rng = np.random.default_rng(0)
    x = _f16_grid_and_ties()
    x = np.concatenate([x, -x, np.exp2(rng.uniform(-30, 20, 20000)) * rng.choice([-1.0, 1.0], 20000),
                        [0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.999, 65520.0, 65536.0, 2.0 ** -25,
                         3 * 2.0 ** -26, 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.round_to(x, orc.F16), ref)
    nan = orc.round_to(np.array([np.nan, -np.nan]), orc.F16)
    assert all((b & 0x7C00) == 0x7C00 and (b & 0x3FF) != 0 for b in nan)


def test_round_to_bf16_matches_torch(orc):
    """bf16: torch's CPU float32 -> bfloat16 conversion rounds to nearest even
    (a library routine).  The inputs are float32 values (so that the check
    does not depend on how torch narrows float64): random bit patterns over
    the whole finite range, every tie of the bf16 grid around a spread of
    exponents, and its neighbours."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x7F800000, 200000, dtype=np.int64).astype(np.uint32)
    hi = np.arange(0, 0x7F80, 7, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, (hi + 0x10000) | 0x8000])
    f32 = np.concatenate([bits, ties, np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 1, 0x8000], np.uint32)])
    f32 = np.concatenate([f32, f32 | np.uint32(0x80000000)]).view(np.float32)
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.round_to(f32.astype(np.float64), orc.BF16), ref)
    # closed forms: ties go to the even neighbour
    one = orc.round_to(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30]), orc.BF16)
    assert list(one) == [0x3F80, 0x3F82, 0x3F81]


def test_bad_arguments_rejected(orc):
    with pytest.raises(ValueError):
        orc.prune_compress(np.zeros((4, 48), np.uint16), wl.F16)   # K not a multiple of 32


# ---- metadata validity count and decompression of invalid codes ---------------
def test_count_invalid_pins(orc):
    """Invalid = the two codes of a group are not strictly increasing."""
    assert orc.count_invalid(np.full((3, 4), 0x88888888, np.uint32), 128) == 0
    assert orc.count_invalid(np.zeros((5, 2), np.uint32), 64) == 5 * 16      # every code 0: all groups bad
    # brute force over the 16 code pairs of group 3 in a word whose other groups are (0, 2)
    for c0 in range(4):
        for c1 in range(4):
            w = 0x88888888 & ~(0xF << 12) | (c0 << 12) | (c1 << 14)
            assert orc.count_invalid(np.array([[w]], np.uint32), 32) == int(c0 >= c1)
    # compression never produces invalid metadata
    A = wl.random_case(4, 33, 16, 256, wl.F16, wl.F16).A
    _, meta = orc.prune_compress(A, wl.F16)
    assert orc.count_invalid(meta, 256) == 0


def test_decompress_invalid_codes_second_value_wins(orc):
    """With both codes of a group naming the same slot, that slot holds the second value."""
    vals = np.zeros((1, 16), np.uint16)
    vals[0, 0], vals[0, 1] = 0x3C00, 0x4000  # 1.0 and 2.0
    meta = np.array([[0x88888888 & ~0xF | (2 | 2 << 2)]], np.uint32)  # group 0: codes (2, 2)
    d = orc.decompress(vals, meta, wl.F16)
    assert d[0, 2] == 0x4000 and d[0, 0] == 0 and d[0, 1] == 0 and d[0, 3] == 0
