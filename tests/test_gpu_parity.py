"""GPU parity: libsp24 (through its C ABI binding) against the CPU oracle.

Bar: compressed values and metadata bit-exact for every type; int8 products
bit-exact; floating products within |err| <= 1e-4 * S + 1e-6 per element,
where S = |alpha| * sum_c |a*b| + |beta*c| is computed by the oracle in fp64.
(Single products are formed exactly and an fp32 chain of n additions errs
by at most ~n * 2^-24 * S; the kernels' longest chain is K/64 = 256
instructions at K = 16384, far inside 1e-4.  The matrix units' own
rounding inside an 8-bit instruction, which matters only for inputs of
widely different magnitudes, is pinned in test_gpu_edge_values.py.)

Small cases are compared element by element over the whole output.  The
full benchmark-size workloads are compared at every output
(test_workload_full_output) and, in the other layouts and repeated runs, on
sampled outputs (random points plus the first and last rows and columns), in
the same launch configuration the benchmark times (K-blocked layout).  The oracle produces the row-major
compressed layout; K-blocked inputs and expected outputs are the same data
moved by tests/layouts.py.
"""
import numpy as np
import pytest

import oracle
from layouts import row_to_kblock
from structured_sparse_matrix_sp24_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sparse_matrix_sp24_amd as p
    p.sp24_version()  # raises if libsp24.so is missing: there is no other path
    return p


DEV = "cuda:0"
ROW, KBLOCK = 0, 1
LAYOUTS = [ROW, KBLOCK]
KN, NK = 0, 1  # B stored K x N, or transposed (N x K)


def n_supported(N, b_type, b_layout):
    """The library's rule for N: a multiple of 8, and of 16 for 8-bit B
    stored K x N with N > 64."""
    if N % 8:
        return False
    return not (wl.ESIZE[b_type] == 1 and b_layout == KN and N > 64 and N % 16)
TVIEW = {wl.F16: torch.int16, wl.BF16: torch.int16, wl.I8: torch.int8, wl.E4M3: torch.uint8, wl.E5M2: torch.uint8}
TTYPE = {wl.F16: torch.float16, wl.BF16: torch.bfloat16, wl.I8: torch.int8, wl.E4M3: torch.float8_e4m3fn,
         wl.E5M2: torch.float8_e5m2}
NPVIEW = {torch.int16: np.int16, torch.int8: np.int8, torch.uint8: np.uint8}


def to_dev(bits, dtype):
    v = TVIEW[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(NPVIEW[v])).to(DEV).view(TTYPE[dtype])


def to_host_bits(t, dtype):
    v = TVIEW[dtype]
    return t.view(v).cpu().numpy().view(wl.STORE[dtype])


def in_layout(vals, meta, dtype, layout):
    """Oracle (row-major) compressed data moved into `layout`."""
    return (vals, meta) if layout == ROW else row_to_kblock(vals, meta, dtype)


def run_compress(pkg, A_bits, dtype, layout=KBLOCK):
    A = to_dev(A_bits, dtype)
    vals, meta = pkg.prune_compress(A, dtype, layout)
    torch.cuda.synchronize()
    return vals, meta


def check_compress(pkg, A_bits, dtype, layout=KBLOCK):
    vals, meta = run_compress(pkg, A_bits, dtype, layout)
    ov, om = oracle.prune_compress(A_bits, dtype)
    ev, em = in_layout(ov, om, dtype, layout)
    gv = to_host_bits(vals, dtype)
    gm = meta.cpu().numpy().view(np.uint32)
    assert np.array_equal(gm, em), "metadata differs"
    assert np.array_equal(gv.view(ev.dtype), ev), "compressed values differ"
    return ov, om


def b_on_dev(B_bits, b_type, b_layout):
    """K x N device view of B: contiguous, or the transpose of a contiguous N x K copy."""
    return to_dev(B_bits, b_type) if b_layout == KN else to_dev(np.ascontiguousarray(B_bits.T), b_type).t()


def run_gemm(pkg, vals_bits, meta_words, a_type, B_bits, b_type, C=None, alpha=1.0, beta=0.0, layout=KBLOCK,
             b_layout=KN):
    vals_bits, meta_words = in_layout(vals_bits, meta_words, a_type, layout)
    V = to_dev(vals_bits, a_type)
    Mt = torch.from_numpy(np.ascontiguousarray(meta_words).view(np.int32)).to(DEV)
    B = b_on_dev(B_bits, b_type, b_layout)
    Ct = None if C is None else torch.from_numpy(np.ascontiguousarray(C)).to(DEV)
    D = pkg.gemm(V, Mt, B, Ct, alpha=alpha, beta=beta, a_type=a_type, b_type=b_type, layout=layout)
    torch.cuda.synchronize()
    return D


def check_gemm_full(pkg, vals, meta, a_type, B, b_type, C=None, alpha=1.0, beta=0.0, layout=KBLOCK, b_layout=KN):
    """vals / meta: the oracle's row-major compressed A (moved into `layout` for the GPU)."""
    D = run_gemm(pkg, vals, meta, a_type, B, b_type, C, alpha, beta, layout, b_layout).cpu().numpy()
    if a_type == wl.I8:
        ref = oracle.gemm_i64(vals, meta, B, C, beta_one=(beta == 1.0))
        assert np.array_equal(D.astype(np.int64), ref)
    else:
        ref, S = oracle.gemm_f64(vals, meta, a_type, B, b_type, C, alpha=alpha, beta=beta)
        err = np.abs(D.astype(np.float64) - ref)
        bad = err > 1e-4 * S + 1e-6
        assert not bad.any(), f"{bad.sum()} elements outside bound; worst ratio {np.max(err / (S + 1e-30)):.3g}"


def sample_points(M, N, n, seed=0):
    g = np.random.default_rng(seed)
    ii = [g.integers(0, M, n)]
    jj = [g.integers(0, N, n)]
    for r in (0, M - 1):           # whole first / last rows
        cols = np.linspace(0, N - 1, min(N, 512)).astype(np.int64)
        ii.append(np.full(len(cols), r)); jj.append(cols)
    for c in (0, N - 1):           # whole first / last columns
        rows = np.linspace(0, M - 1, min(M, 512)).astype(np.int64)
        ii.append(rows); jj.append(np.full(len(rows), c))
    return np.concatenate(ii).astype(np.int64), np.concatenate(jj).astype(np.int64)


def check_gemm_sampled(D, vals, meta, w, n=4096):
    ii, jj = sample_points(w.M, w.N, n)
    got = D[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)].cpu().numpy()
    if w.a_type == wl.I8:
        ref = oracle.gemm_points_i64(vals, meta, w.B, ii, jj, w.C, beta_one=(w.beta == 1.0))
        assert np.array_equal(got.astype(np.int64), ref)
    else:
        ref, S = oracle.gemm_points_f64(vals, meta, w.a_type, w.B, w.b_type, ii, jj, w.C, alpha=w.alpha,
                                        beta=w.beta)
        err = np.abs(got.astype(np.float64) - ref)
        assert (err <= 1e-4 * S + 1e-6).all(), f"worst ratio {np.max(err / (S + 1e-30)):.3g}"


# ---- compression -------------------------------------------------------------
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16, wl.I8, wl.E4M3, wl.E5M2])
@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (129, 160), (257, 1024), (64, 4096), (200, 224)])
def test_compress_random(pkg, dtype, shape, layout):
    M, K = shape
    _say(f"compress dtype={dtype} M={M} K={K} layout={layout}")
    c = wl.random_case(13, M, 16, K, dtype, dtype)
    check_compress(pkg, c.A, dtype, layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16, wl.I8, wl.E4M3])
@pytest.mark.parametrize("shape", [(4136, 4128), (4104, 4224)])
def test_compress_many_workgroups(pkg, dtype, shape, layout):
    """Shapes large enough for the K-blocked launch to give 16-bit workgroups
    two blocks each, with a ragged last row tile, a partial last block and an
    odd block count (the second block of the last group lies past K)."""
    M, K = shape
    _say(f"compress dtype={dtype} M={M} K={K} layout={layout}")
    c = wl.random_case(17, M, 16, K, dtype, dtype)
    check_compress(pkg, c.A, dtype, layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16, wl.E4M3, wl.E5M2, wl.I8])
def test_compress_adversarial_alphabet(pkg, dtype, layout):
    """Ties, signed zeros, extremes, subnormals and NaN in every position."""
    _say(f"compress adversarial dtype={dtype} layout={layout}")
    from test_oracle import _alphabet
    alpha = _alphabet(dtype)
    idx = np.indices((9, 9, 9, 9)).reshape(4, -1).T
    pad = (-len(idx)) % 8
    A = alpha[np.concatenate([idx, idx[:pad]])].reshape(-1, 32)
    check_compress(pkg, A, dtype, layout)


def test_compress_empty(pkg):
    A = torch.empty((0, 64), dtype=torch.float16, device=DEV)
    vals, meta = pkg.prune_compress(A, layout=ROW)
    assert vals.shape == (0, 32) and meta.shape == (0, 2)
    vals, meta = pkg.prune_compress(A, layout=KBLOCK)
    assert vals.shape == (1, 0, 32) and meta.shape == (1, 0, 2)


# ---- products, whole-output comparison ----------------------------------------
PAIRS = [(wl.F16, wl.F16), (wl.BF16, wl.BF16), (wl.I8, wl.I8), (wl.E4M3, wl.E4M3), (wl.E4M3, wl.E5M2),
         (wl.E5M2, wl.E4M3), (wl.E5M2, wl.E5M2)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("M,N,K", [(300, 272, 160), (512, 512, 512), (17, 96, 256), (256, 256, 32),
                                   (96, 48, 352), (40, 16, 128), (600, 64, 1024), (1, 128, 64),
                                   (257, 8, 4128), (130, 24, 384), (70, 40, 640), (33, 56, 256)])
def test_gemm_random(pkg, a_type, b_type, M, N, K, layout):
    assert n_supported(N, b_type, KN)
    _say(f"gemm a={a_type} b={b_type} M={M} N={N} K={K} layout={layout}")
    c = wl.random_case(21, M, N, K, a_type, b_type)
    vals, meta = oracle.prune_compress(c.A, a_type)
    check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, layout=layout)


# More 256 x 256 tiles than compute units (several tiles per compute unit, the
# dispatch order of the XCD-aware tile walk over a grid that is not a multiple
# of 8), ragged M and N (edge tiles write fewer rows and columns), K of
# exactly 3 k-steps, K ending in a partial k-step, both layouts and B layouts,
# and beta != 0 (C read in the epilogue).  Every output is compared with the
# oracle.
@pytest.mark.slow
@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("M,N,K,layout,b_layout,beta", [
    (4100, 4368, 192, KBLOCK, KN, 0.0),    # 16-bit: 3 k-steps
    (4100, 4368, 384, KBLOCK, KN, 1.0),    # 8-bit: 3 k-steps
    (4352, 4104, 544, ROW, NK, 0.0),       # partial last k-step
    (4224, 4360, 416, KBLOCK, NK, 1.0),
])
def test_gemm_many_tiles(pkg, a_type, b_type, M, N, K, layout, b_layout, beta):
    _say(f"gemm many tiles a={a_type} b={b_type} M={M} N={N} K={K} layout={layout} b_layout={b_layout} beta={beta}")
    w = wl.random_case(41, M, N, K, a_type, b_type, beta=beta)
    vals, meta = oracle.prune_compress(w.A, a_type)
    D = run_gemm(pkg, vals, meta, a_type, w.B, b_type, w.C, w.alpha, w.beta, layout, b_layout).cpu().numpy()
    ref, S = oracle_full_threaded(vals, meta, w)
    if a_type == wl.I8:
        assert np.array_equal(D.astype(np.int64), ref)
    else:
        err = np.abs(D.astype(np.float64) - ref)
        bad = err > 1e-4 * S + 1e-6
        assert not bad.any(), f"{bad.sum()} elements outside bound; worst ratio {np.max(err / (S + 1e-30)):.3g}"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("M,N,K", [(300, 272, 160), (512, 512, 544), (17, 96, 256), (96, 48, 352),
                                   (40, 16, 128), (600, 64, 1024), (1, 128, 64), (257, 8, 4128),
                                   (130, 24, 384), (70, 40, 640), (96, 72, 288)])
def test_gemm_random_b_transposed(pkg, a_type, b_type, M, N, K, layout):
    """B stored N x K (K contiguous)."""
    assert n_supported(N, b_type, NK)
    _say(f"gemm B^T a={a_type} b={b_type} M={M} N={N} K={K} layout={layout}")
    c = wl.random_case(23, M, N, K, a_type, b_type)
    vals, meta = oracle.prune_compress(c.A, a_type)
    check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, layout=layout, b_layout=NK)


# Small-N chunks: each wave takes every 8th k-step and works through them in
# chunks of 8, 4 or 2 (N <= 16, 32, 64).  K is chosen so that waves get more
# than one chunk, a partial last chunk, different step counts, and a partial
# last k-step (the K tail).
@pytest.mark.parametrize("b_layout", [KN, NK])
@pytest.mark.parametrize("a_type,b_type", [(wl.BF16, wl.BF16), (wl.I8, wl.I8), (wl.E4M3, wl.E5M2)])
@pytest.mark.parametrize("N,steps_extra", [(16, 0), (16, 19), (32, 5), (48, 3), (64, 1)])
def test_gemm_small_n_chunks(pkg, a_type, b_type, N, steps_extra, b_layout):
    ks = 64 if wl.ESIZE[a_type] == 2 else 128
    K = ks * (8 * 8 + steps_extra) + 32      # 8 full chunks' worth for D = 8, extra steps, a 32-wide tail
    M = 128 if N == 16 else 40               # 8 row tiles (the XCD-grouped tile order) or a ragged 2.5
    _say(f"gemm small-N chunks a={a_type} M={M} N={N} K={K} b_layout={b_layout}")
    c = wl.random_case(41, M, N, K, a_type, b_type)
    vals, meta = oracle.prune_compress(c.A, a_type)
    check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, b_layout=b_layout)


@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.I8, wl.I8), (wl.E5M2, wl.E4M3)])
@pytest.mark.parametrize("N", [16, 48, 512])
def test_b_layouts_give_identical_bits(pkg, a_type, b_type, N):
    """Both B layouts deliver the same fragments to the same instruction
    sequence: outputs agree bit for bit (K with a ragged last step)."""
    _say(f"B layouts agree a={a_type} N={N}")
    c = wl.random_case(37, 520, N, 736 if wl.ESIZE[a_type] == 2 else 800, a_type, b_type)
    A = to_dev(c.A, a_type)
    V, Mt = pkg.prune_compress(A, a_type, KBLOCK)
    D1 = pkg.gemm(V, Mt, b_on_dev(c.B, b_type, KN), a_type=a_type, b_type=b_type)
    D2 = pkg.gemm(V, Mt, b_on_dev(c.B, b_type, NK), a_type=a_type, b_type=b_type)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int32), D2.view(torch.int32))


@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.I8, wl.I8), (wl.E5M2, wl.E4M3)])
@pytest.mark.parametrize("N", [32, 512])
def test_layouts_give_identical_bits(pkg, a_type, b_type, N):
    """Both layouts feed the same instruction sequence: outputs agree bit for bit."""
    _say(f"layouts agree a={a_type} N={N}")
    c = wl.random_case(31, 520, N, 736, a_type, b_type)
    A = to_dev(c.A, a_type)
    B = to_dev(c.B, b_type)
    Vr, Mr = pkg.prune_compress(A, a_type, ROW)
    Vk, Mk = pkg.prune_compress(A, a_type, KBLOCK)
    Dr = pkg.gemm(Vr, Mr, B, a_type=a_type, b_type=b_type, layout=ROW)
    Dk = pkg.gemm(Vk, Mk, B, a_type=a_type, b_type=b_type, layout=KBLOCK)
    torch.cuda.synchronize()
    assert torch.equal(Dr.view(torch.int32), Dk.view(torch.int32))


@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.BF16, wl.BF16), (wl.E4M3, wl.E5M2)])
@pytest.mark.parametrize("N", [32, 320])
@pytest.mark.parametrize("b_layout", [KN, NK])
def test_gemm_alpha_beta(pkg, a_type, b_type, N, b_layout):
    _say(f"gemm alpha/beta a={a_type} N={N} b_layout={b_layout}")
    c = wl.random_case(5, 130, N, 192, a_type, b_type, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, a_type)
    check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, c.C, alpha=-0.5, beta=1.5, b_layout=b_layout)
    check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, c.C, alpha=0.0, beta=2.0, b_layout=b_layout)


@pytest.mark.parametrize("N", [32, 272])
@pytest.mark.parametrize("b_layout", [KN, NK])
def test_gemm_int8_beta_one(pkg, N, b_layout):
    _say(f"gemm int8 beta=1 N={N} b_layout={b_layout}")
    c = wl.random_case(6, 77, N, 256, wl.I8, wl.I8, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, wl.I8)
    check_gemm_full(pkg, vals, meta, wl.I8, c.B, wl.I8, c.C, beta=1.0, b_layout=b_layout)


@pytest.mark.parametrize("N", [48, 512])
def test_gemm_beta_zero_ignores_nan_C(pkg, N):
    _say(f"gemm beta=0 with NaN C N={N}")
    c = wl.random_case(8, 64, N, 128, wl.F16, wl.F16)
    vals, meta = oracle.prune_compress(c.A, wl.F16)
    Cn = np.full((64, N), np.nan, np.float32)
    D = run_gemm(pkg, vals, meta, wl.F16, c.B, wl.F16, Cn, beta=0.0)
    assert not torch.isnan(D).any()


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16, wl.E4M3, wl.E5M2, wl.I8])
@pytest.mark.parametrize("K", [128, 512])
def test_gemm_identity_B_returns_A(pkg, dtype, K):
    """B = I_K: D must equal the decompressed A exactly (one nonzero term per output)."""
    _say(f"gemm identity dtype={dtype} K={K}")
    c = wl.random_case(3, 100, 16, K, dtype, dtype)
    vals, meta = oracle.prune_compress(c.A, dtype)
    one = np.int8(1) if dtype == wl.I8 else wl.quantize(np.ones(1), dtype)[0]
    Bid = np.zeros((K, K), dtype=wl.STORE[dtype])
    Bid[np.arange(K), np.arange(K)] = one
    D = run_gemm(pkg, vals, meta, dtype, Bid, dtype).cpu().numpy().astype(np.float64)
    dense = oracle.decode(oracle.decompress(vals, meta, dtype), dtype)
    assert np.array_equal(D, dense)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_K_zero(pkg, layout):
    C = torch.full((8, 64), 3.0, device=DEV)
    vs, ms = pkg.compressed_shapes(8, 0, pkg.SP24_F16, layout)
    V = torch.empty(vs, dtype=torch.float16, device=DEV)
    Mt = torch.empty(ms, dtype=torch.int32, device=DEV)
    B = torch.empty((0, 64), dtype=torch.float16, device=DEV)
    pkg.gemm(V, Mt, B, C, beta=0.5, layout=layout)
    torch.cuda.synchronize()
    assert (C == 1.5).all()


# ---- 16-bit output and bias (sp24_gemm_ex) ---------------------------------------
OUT_T = {wl.F16: torch.float16, wl.BF16: torch.bfloat16}


def grid_spacing(x, dtype):
    """Spacing of the fp16 / bf16 grid at |x| (the subnormal spacing below the
    smallest normal value)."""
    mb, emin = (10, -14) if dtype == wl.F16 else (7, -126)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return np.exp2(e - mb)


def run_gemm_ex(pkg, vals, meta, a_type, B_bits, b_type, C_dev, out_dtype, bias, alpha, beta, b_layout=KN,
                layout=KBLOCK):
    v, m = in_layout(vals, meta, a_type, layout)
    V = to_dev(v, a_type)
    Mt = torch.from_numpy(np.ascontiguousarray(m).view(np.int32)).to(DEV)
    B = b_on_dev(B_bits, b_type, b_layout)
    bt = None if bias is None else torch.from_numpy(bias).to(DEV)
    D = pkg.gemm(V, Mt, B, C_dev, alpha=alpha, beta=beta, a_type=a_type, b_type=b_type, layout=layout,
                 out_dtype=out_dtype, bias=bt)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("b_layout", [KN, NK])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("N", [32, 272])
@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.BF16, wl.BF16), (wl.E4M3, wl.E5M2)])
@pytest.mark.parametrize("out", [wl.F16, wl.BF16])
def test_gemm_out16_bias(pkg, out, a_type, b_type, N, with_bias, b_layout):
    """D = round16(alpha * A B + beta * C + bias): within the fp32 bound of the
    oracle's exact value plus one step of the output grid."""
    _say(f"gemm 16-bit out={out} a={a_type} N={N} bias={with_bias} b_layout={b_layout}")
    M, K = 130, 224
    c = wl.random_case(31, M, N, K, a_type, b_type, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, a_type)
    rng = np.random.default_rng(7)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    C16 = torch.from_numpy(c.C).to(OUT_T[out])            # C held in the output type
    C32 = C16.to(torch.float32).numpy()                    # exactly its values, for the oracle
    D = run_gemm_ex(pkg, vals, meta, a_type, c.B, b_type, C16.to(DEV), OUT_T[out], bias, -0.5, 1.5, b_layout)
    got = oracle.decode(D.view(torch.int16).cpu().numpy().view(np.uint16), out)
    ref, S = oracle.gemm_f64(vals, meta, a_type, c.B, b_type, C32, alpha=-0.5, beta=1.5, bias=bias)
    err = np.abs(got - ref)
    assert (err <= 1e-4 * S + 1e-6 + grid_spacing(ref, out)).all(), f"worst {np.max(err - 1e-4 * S):.3g}"
    # where the exact value is far from a rounding boundary the bits are the
    # oracle's rounding.  16-bit inputs: products are exact in fp32 and an
    # fp32 sum of at most K/32 + 4 terms (k-steps, then the epilogue's) is off
    # by less than (K/32 + 4) * 2^-24 * S.  8-bit float inputs: the units sum
    # each run of 8 products on a coarser grid (test_gpu_edge_values.py), so
    # only the parity bound itself applies there.
    t = ref / grid_spacing(ref, out)
    fp32_err = (K / 32 + 4) * 2.0 ** -24 * S if wl.ESIZE[a_type] == 2 else 1e-4 * S + 1e-6
    far = (np.abs(t - np.round(t)) < 0.25) & (fp32_err < 0.1 * grid_spacing(ref, out))
    if wl.ESIZE[a_type] == 2:
        assert far.mean() > 0.3
    exp_bits = oracle.round_to(ref[far], out)
    assert np.array_equal(D.view(torch.int16).cpu().numpy().view(np.uint16)[far], exp_bits)


@pytest.mark.parametrize("beta_zero", [False, True])
@pytest.mark.parametrize("k_tail", [0, 32])
@pytest.mark.parametrize("b_layout", [KN, NK])
@pytest.mark.parametrize("out", [None, wl.F16, wl.BF16])
@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.I8, wl.I8), (wl.E5M2, wl.E4M3)])
def test_gemm_one_wave_modes(pkg, a_type, b_type, out, b_layout, k_tail, beta_zero):
    """A grid of at most one tile per compute unit, where the product stores
    its output with ordinary stores and, with beta != 0, reads the tile's C
    ahead during 32 (32-bit C) or 16 (16-bit C) of its load steps, from 48
    before the last: 56 or 57 k-steps (the window opens and closes inside
    the loop; with k_tail the last step is partial), ragged M and N
    (rows of the last pieces past M, columns past N), 32-bit and 16-bit C
    (one or two tile rows per piece), beta != 0 and beta == 0; every output
    against the oracle."""
    if a_type == wl.I8 and out is not None:
        pytest.skip("int8 has a 32-bit output only")
    M, N = 701, 528  # N % 16 == 0: 8-bit B stored K x N above N = 64 needs it
    K = 56 * (64 if wl.ESIZE[a_type] == 2 else 128) + k_tail
    _say(f"gemm one-wave modes a={a_type} out={out} b_layout={b_layout} K={K} beta_zero={beta_zero}")
    c = wl.random_case(53, M, N, K, a_type, b_type, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, a_type)
    if out is None:
        alpha, beta = (1.0, 1.0) if a_type == wl.I8 else (0.75, -1.25)
        if beta_zero:
            beta = 0.0
        check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, c.C, alpha, beta, KBLOCK, b_layout)
        return
    beta = 0.0 if beta_zero else -1.25
    C16 = torch.from_numpy(c.C).to(OUT_T[out])
    C32 = C16.to(torch.float32).numpy()
    D = run_gemm_ex(pkg, vals, meta, a_type, c.B, b_type, C16.to(DEV), OUT_T[out], None, 0.75, beta, b_layout)
    got = oracle.decode(D.view(torch.int16).cpu().numpy().view(np.uint16), out)
    ref, S = oracle.gemm_f64(vals, meta, a_type, c.B, b_type, C32, alpha=0.75, beta=beta)
    err = np.abs(got - ref)
    assert (err <= 1e-4 * S + 1e-6 + grid_spacing(ref, out)).all(), f"worst {np.max(err - 1e-4 * S):.3g}"


@pytest.mark.parametrize("M", [4096, 4104])
@pytest.mark.parametrize("a_type,b_type", [(wl.F16, wl.F16), (wl.I8, wl.I8)])
def test_gemm_tile_count_boundary(pkg, a_type, b_type, M):
    """Either side of one tile per compute unit: 4096 x 4096 is 256 output
    tiles of 256 x 256 (ordinary output stores, C read ahead in the main
    loop), 4104 x 4096 is 272 (streaming stores, C read in the epilogue);
    beta != 0, every output against the oracle."""
    N, K = 4096, 96 if wl.ESIZE[a_type] == 2 else 160
    _say(f"gemm tile-count boundary a={a_type} M={M} N={N} K={K}")
    c = wl.random_case(57, M, N, K, a_type, b_type, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, a_type)
    alpha, beta = (1.0, 1.0) if a_type == wl.I8 else (0.75, -1.25)
    check_gemm_full(pkg, vals, meta, a_type, c.B, b_type, c.C, alpha, beta, KBLOCK, KN)


@pytest.mark.parametrize("N", [48, 320])
def test_gemm_bias_f32_out(pkg, N):
    _say(f"gemm bias fp32 out N={N}")
    c = wl.random_case(32, 96, N, 160, wl.BF16, wl.BF16, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, wl.BF16)
    bias = np.random.default_rng(9).standard_normal(N).astype(np.float32) * 10
    D = run_gemm_ex(pkg, vals, meta, wl.BF16, c.B, wl.BF16, torch.from_numpy(c.C).to(DEV), torch.float32, bias,
                    0.25, 2.0).cpu().numpy().astype(np.float64)
    ref, S = oracle.gemm_f64(vals, meta, wl.BF16, c.B, wl.BF16, c.C, alpha=0.25, beta=2.0, bias=bias)
    assert (np.abs(D - ref) <= 1e-4 * S + 1e-6).all()


@pytest.mark.parametrize("out", [wl.F16, wl.BF16])
def test_gemm_bias_adjacent_to_16bit_C(pkg, out):
    """C (M x N, 16-bit) and the bias (N fp32) in one allocation, the bias
    starting at the first byte after C: the call accepts it (the two do not
    overlap), and the result is the oracle's within the bound plus one step
    of the output grid, with the bias itself left unchanged."""
    M, N, K = 64, 64, 128
    _say(f"gemm bias adjacent to 16-bit C out={out}")
    c = wl.random_case(33, M, N, K, wl.F16, wl.F16, beta=1.0)
    vals, meta = oracle.prune_compress(c.A, wl.F16)
    bias = np.random.default_rng(11).standard_normal(N).astype(np.float32)
    C16 = torch.from_numpy(c.C).to(OUT_T[out])
    buf = torch.empty(M * N * 2 + N * 4, dtype=torch.uint8, device=DEV)
    Cd = buf[:M * N * 2].view(OUT_T[out]).view(M, N)
    bd = buf[M * N * 2:].view(torch.float32)
    Cd.copy_(C16.to(DEV))
    bd.copy_(torch.from_numpy(bias).to(DEV))
    v, m = in_layout(vals, meta, wl.F16, KBLOCK)
    V = to_dev(v, wl.F16)
    Mt = torch.from_numpy(np.ascontiguousarray(m).view(np.int32)).to(DEV)
    pkg.gemm(V, Mt, to_dev(c.B, wl.F16), Cd, alpha=1.0, beta=0.5, layout=KBLOCK, out_dtype=OUT_T[out], bias=bd)
    torch.cuda.synchronize()
    got = oracle.decode(Cd.view(torch.int16).cpu().numpy().view(np.uint16), out)
    ref, S = oracle.gemm_f64(vals, meta, wl.F16, c.B, wl.F16, C16.to(torch.float32).numpy(), alpha=1.0, beta=0.5,
                             bias=bias)
    assert (np.abs(got - ref) <= 1e-4 * S + 1e-6 + grid_spacing(ref, out)).all()
    assert np.array_equal(bd.cpu().numpy(), bias)


@pytest.mark.parametrize("out", [wl.F16, wl.BF16])
def test_gemm_K_zero_out16_bias(pkg, out):
    """K = 0: D = round16(beta * C + bias) whatever alpha is."""
    M, N = 8, 64
    rng = np.random.default_rng(5)
    C16 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(OUT_T[out])
    bias = rng.standard_normal(N).astype(np.float32)
    vs, ms = pkg.compressed_shapes(M, 0, pkg.SP24_F16, KBLOCK)
    V = torch.empty(vs, dtype=torch.float16, device=DEV)
    Mt = torch.empty(ms, dtype=torch.int32, device=DEV)
    B = torch.empty((0, N), dtype=torch.float16, device=DEV)
    Cd = C16.to(DEV)
    pkg.gemm(V, Mt, B, Cd, alpha=float("inf"), beta=0.5, layout=KBLOCK, out_dtype=OUT_T[out],
             bias=torch.from_numpy(bias).to(DEV))
    torch.cuda.synchronize()
    ref = 0.5 * C16.to(torch.float64).numpy() + bias.astype(np.float64)[None, :]
    got = oracle.decode(Cd.view(torch.int16).cpu().numpy().view(np.uint16), out)
    assert (np.abs(got - ref) <= 1e-6 * np.abs(ref) + grid_spacing(ref, out)).all()


# ---- the largest shapes the boundary accepts ---------------------------------
# The C ABI bounds every buffer range one workgroup addresses below 2 GiB:
# N * sizeof(b) * 128 (a k-step of B stored K x N, 8-bit), 256 * K/2 * sizeof(a)
# (a row tile of A in the ROW layout) and 256 * K * sizeof(b) (a column tile
# of B stored N x K).  These run each limit at its largest accepted value,
# with integer inputs so the exact product is known, and check sampled
# outputs (whole first and last rows and columns included).
MAX_BYTES = 0x7FFFFF00  # the largest per-workgroup range the library accepts


def _max_case(pkg, M, N, K, dtype, layout, b_layout, lim):
    hi = 127 if dtype == wl.I8 else 1
    A = wl.small_int_bits((M, K), dtype, 31, -hi, hi)
    B = wl.small_int_bits((K, N), dtype, 32, -hi, hi)
    assert lim <= MAX_BYTES
    ov, om = check_compress(pkg, A, dtype, layout)
    D = run_gemm(pkg, ov, om, dtype, B, dtype, layout=layout, b_layout=b_layout)
    if K <= 4096:  # N is the large dimension: sampled points
        w = wl.Workload(f"max_{M}x{N}x{K}", M, N, K, dtype, dtype, 1.0, 0.0, A, B, None)
        check_gemm_sampled(D, ov, om, w, n=64)
        return
    # K is the large dimension: whole output rows (first, last and two
    # others), each from the oracle's full product of that one row of A,
    # which streams B once per row instead of once per point
    rows = sorted({0, M - 1, M // 3, (2 * M) // 3})
    got = D[rows].cpu().numpy().astype(np.float64)
    for n, i in enumerate(rows):
        ref, S = oracle.gemm_f64(ov[i:i + 1], om[i:i + 1], dtype, B, dtype)
        err = np.abs(got[n] - ref[0])
        assert (err <= 1e-4 * S[0] + 1e-6).all(), f"row {i}: worst ratio {np.max(err / (S[0] + 1e-30)):.3g}"


@pytest.mark.parametrize("dtype", [wl.F16, wl.I8])
def test_gemm_largest_n(pkg, dtype):
    """N at the limit for B stored K x N: 128 rows of B just below 2 GiB."""
    es = wl.ESIZE[dtype]
    N = (MAX_BYTES // 128 // es) // 16 * 16
    M, K = (20, 96) if es == 2 else (16, 160)  # a partial last k-step either way
    _say(f"gemm largest N dtype={dtype} M={M} N={N} K={K}")
    _max_case(pkg, M, N, K, dtype, KBLOCK, KN, N * es * 128)


def test_gemm_largest_k_row_layout(pkg):
    """K at the limit for the ROW layout: a 256-row tile of A just below 2 GiB."""
    K = (MAX_BYTES // 256 // 2 * 2) // 32 * 32
    _say(f"gemm largest K (ROW) M=40 N=72 K={K}")
    _max_case(pkg, 40, 72, K, wl.F16, ROW, KN, 256 * K // 2 * 2)


def test_gemm_largest_k_b_transposed(pkg):
    """K at the limit for B stored N x K: a 256-column tile of B just below 2 GiB."""
    K = (MAX_BYTES // 256 // 2) // 32 * 32
    _say(f"gemm largest K (B N x K) M=24 N=72 K={K}")
    _max_case(pkg, 24, 72, K, wl.F16, KBLOCK, NK, 256 * K * 2)


def test_operands_past_4gib(pkg):
    """Compressed A larger than 4 GiB (fp16 131112 x 40992: 10.7 GB dense,
    5.4 GB of values), so byte offsets of later K-blocks need more than 32
    bits.  Compress is checked bit-exact on the first, a middle and the last
    (ragged, 40-row) 128-row group of every block; the product on whole
    output rows of those groups."""
    M, K, N = 131072 + 40, 40960 + 32, 72
    dtype = wl.F16
    _say(f"operands past 4 GiB: M={M} K={K} N={N}")
    A = wl.small_int_bits((M, K), dtype, 41)
    B = wl.small_int_bits((K, N), dtype, 42)
    At = to_dev(A, dtype)
    vals, meta = pkg.prune_compress(At, dtype, KBLOCK)
    del At
    torch.cuda.synchronize()
    nblk, VE, Mp = -(-K // 64), 32, -(-M // 128) * 128
    assert tuple(vals.shape) == (nblk, M, VE) and tuple(meta.shape) == (nblk, Mp, 2)
    groups = [(0, 128), (65536, 128), (131072, 40)]
    for r0, g in groups:
        ov, om = oracle.prune_compress(A[r0:r0 + g], dtype)
        ev, em = row_to_kblock(ov, om, dtype)
        gv = to_host_bits(vals[:, r0:r0 + g, :], dtype)
        gm = meta[:, r0:r0 + 128, :].cpu().numpy().view(np.uint32)
        assert np.array_equal(gm, em), f"metadata of rows {r0}.. differs"
        assert np.array_equal(gv.view(ev.dtype), ev), f"values of rows {r0}.. differs"
    D = pkg.gemm(vals, meta, to_dev(B, dtype), None, a_type=dtype, b_type=dtype, layout=KBLOCK)
    torch.cuda.synchronize()
    for r0, g in groups:
        rows = [r0, r0 + g - 1]
        ov, om = oracle.prune_compress(A[rows], dtype)
        ref, S = oracle.gemm_f64(ov, om, dtype, B, dtype)
        got = D[rows].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        assert (err <= 1e-4 * S + 1e-6).all(), f"rows {rows}: worst ratio {np.max(err / (S + 1e-30)):.3g}"


def test_launches_in_pieces(pkg):
    """Problems that need more workgroups than one launch is given (2^18; a
    dispatch counts its work-items in 32 bits): int8 A of 2^25 + 200 rows x
    128 (4.3 GB), so the K-blocked compress and decompress (one 128-row
    group per workgroup) take two launches, and the small-N product (16 rows
    per workgroup) nine.  Compared with the oracle on whole 128-row groups on
    both sides of the compress pieces' boundary and the ragged end, and on
    the rows on both sides of every boundary between product pieces."""
    M, K, N = (1 << 25) + 200, 128, 8
    dtype = wl.I8
    _say(f"launches in pieces: M={M} K={K} N={N}")
    A = wl.small_int_bits((M, K), dtype, 61, -127, 127)
    B = wl.small_int_bits((K, N), dtype, 62, -127, 127)
    At = to_dev(A, dtype)
    vals, meta = pkg.prune_compress(At, dtype, KBLOCK)
    del At
    torch.cuda.synchronize()
    groups = [(0, 128), ((1 << 25) - 128, 128), (1 << 25, 128), ((1 << 25) + 128, 72)]
    for r0, g in groups:
        ov, om = oracle.prune_compress(A[r0:r0 + g], dtype)
        ev, em = row_to_kblock(ov, om, dtype)
        assert np.array_equal(meta[:, r0:r0 + 128, :].cpu().numpy().view(np.uint32), em), f"metadata of rows {r0}.."
        assert np.array_equal(to_host_bits(vals[:, r0:r0 + g, :], dtype).view(ev.dtype), ev), f"values of rows {r0}.."
    _say("launches in pieces: decompress")
    Ad = pkg.decompress(vals, meta, K, dtype, KBLOCK)
    torch.cuda.synchronize()
    for r0, g in groups:
        ov, om = oracle.prune_compress(A[r0:r0 + g], dtype)
        assert np.array_equal(to_host_bits(Ad[r0:r0 + g], dtype), oracle.decompress(ov, om, dtype)), f"rows {r0}.."
    del Ad
    _say("launches in pieces: small-N product")
    D = pkg.gemm(vals, meta, to_dev(B, dtype), None, a_type=dtype, b_type=dtype, layout=KBLOCK)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(p * (1 << 22) - 16, p * (1 << 22) + 16) for p in range(1, 9)] +
                          [np.arange(0, 16), np.arange(M - 40, M)])
    ov, om = oracle.prune_compress(A[rows], dtype)
    assert np.array_equal(D[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.int64),
                          oracle.gemm_i64(ov, om, B))


def test_gemm_K_zero_past_2e32_elements(pkg):
    """K == 0 (D = beta * C) on an fp16 output of more than 2^32 elements
    (8.6 GB): the kernel covers it with a bounded grid that walks the whole
    output.  beta = 2 on small integers is exact, so every checked element
    equals 2 * C exactly: whole rows at the start, on both sides of element
    2^32 and at the end."""
    M, N = (1 << 16) + 8, 1 << 16
    _say(f"K = 0 with M={M} N={N}")
    g = torch.Generator(device=DEV)
    g.manual_seed(71)
    C = torch.randint(-1000, 1001, (M, N), dtype=torch.int16, device=DEV, generator=g).to(torch.float16)
    rows = torch.tensor([0, 1, (1 << 16) - 1, 1 << 16, (1 << 16) + 1, M - 1], device=DEV)
    before = C[rows].float().cpu().numpy().astype(np.float64)
    vs, ms = pkg.compressed_shapes(M, 0, pkg.SP24_F16, KBLOCK)
    V = torch.empty(vs, dtype=torch.float16, device=DEV)
    Mt = torch.empty(ms, dtype=torch.int32, device=DEV)
    B = torch.empty((0, N), dtype=torch.float16, device=DEV)
    pkg.gemm(V, Mt, B, C, beta=2.0, layout=KBLOCK)
    torch.cuda.synchronize()
    after = C[rows].float().cpu().numpy().astype(np.float64)
    assert np.array_equal(after, 2.0 * before)


def test_gemm_gpu_compressed_input(pkg):
    """Compress on the GPU and multiply the result directly."""
    _say("gemm on GPU-compressed input")
    c = wl.random_case(12, 320, 288, 256, wl.BF16, wl.BF16)
    A = to_dev(c.A, wl.BF16)
    B = to_dev(c.B, wl.BF16)
    vals, meta = pkg.prune_compress(A)
    D = pkg.gemm(vals, meta, B).cpu().numpy()
    ov, om = oracle.prune_compress(c.A, wl.BF16)
    ref, S = oracle.gemm_f64(ov, om, wl.BF16, c.B, wl.BF16)
    assert (np.abs(D - ref) <= 1e-4 * S + 1e-6).all()


# ---- the named workloads at their full sizes -----------------------------------
@pytest.mark.slow
@pytest.mark.parametrize("name,b_layout", [("tiny_f16", KN), ("f16_4096", KN), ("bf16_linear_n16", KN),
                                           ("bf16_linear_n4096", KN), ("i8_8192", KN), ("fp8_bf8_8192x16384", KN),
                                           ("bf8_bf8_8192x16384", KN), ("f16_8192", KN),
                                           ("bf16_linear_n16", NK), ("bf16_linear_n4096", NK), ("f16_8192", NK)])
def test_workload_full_size(pkg, name, b_layout):
    _say(f"workload {name}: generating inputs")
    w = wl.make(name)
    _say(f"workload {name}: M={w.M} N={w.N} K={w.K} compress")
    A = to_dev(w.A, w.a_type)
    vals_d, meta_d = pkg.prune_compress(A, w.a_type, KBLOCK)
    torch.cuda.synchronize()
    ov, om = oracle.prune_compress(w.A, w.a_type)
    ev, em = row_to_kblock(ov, om, w.a_type)
    assert np.array_equal(meta_d.cpu().numpy().view(np.uint32), em), "metadata differs"
    assert np.array_equal(to_host_bits(vals_d, w.a_type).view(ev.dtype), ev), "values differ"
    del ev, em
    for _ in range(2):  # the same bits on every run
        v2, m2 = pkg.prune_compress(A, w.a_type, KBLOCK)
        assert torch.equal(v2.view(torch.uint8), vals_d.view(torch.uint8)) and torch.equal(m2, meta_d)
        del v2, m2
    if name == "tiny_f16":
        assert (om == 0x88888888).all()
    if name == "i8_8192":
        codes = ((om[:, :, None] >> (2 * np.arange(16, dtype=np.uint32))) & 3).reshape(w.M, w.K // 2)
        pairs = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])
        assert np.array_equal(codes[:, 0::2], pairs[w.notes["pattern_pick"], 0])
    del A
    _say(f"workload {name}: gemm (b_layout={b_layout})")
    B = b_on_dev(w.B, w.b_type, b_layout)
    C = None if w.C is None else torch.from_numpy(w.C).to(DEV)
    D = pkg.gemm(vals_d, meta_d, B, C, alpha=w.alpha, beta=w.beta, a_type=w.a_type, b_type=w.b_type)
    torch.cuda.synchronize()
    if w.M * w.N <= 64 * 64:
        check_gemm_full(pkg, ov, om, w.a_type, w.B, w.b_type, w.C, w.alpha, w.beta, b_layout=b_layout)
    else:
        check_gemm_sampled(D, ov, om, w)
    for _ in range(2):  # the summation order is fixed, so every run gives the same bits
        C2 = None if w.C is None else torch.from_numpy(w.C).to(DEV)
        D2 = pkg.gemm(vals_d, meta_d, B, C2, alpha=w.alpha, beta=w.beta, a_type=w.a_type, b_type=w.b_type)
        torch.cuda.synchronize()
        assert torch.equal(D2.view(torch.int32), D.view(torch.int32)), "product differs between runs"
        del D2, C2


def oracle_full_threaded(vals, meta, w, max_threads=16):
    """The oracle's whole product (and scale S for floats), rows split over
    host threads (the oracle call releases the interpreter lock)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(len(os.sched_getaffinity(0)), max_threads))
    bounds = np.linspace(0, w.M, threads + 1).astype(int)

    def part(i):
        r0, r1 = bounds[i], bounds[i + 1]
        if w.a_type == wl.I8:
            C = None if w.C is None else w.C[r0:r1]
            return oracle.gemm_i64(vals[r0:r1], meta[r0:r1], w.B, C, beta_one=(w.beta == 1.0)), None
        C = None if w.C is None else w.C[r0:r1]
        return oracle.gemm_f64(vals[r0:r1], meta[r0:r1], w.a_type, w.B, w.b_type, C, alpha=w.alpha, beta=w.beta)

    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(part, range(threads)))
    ref = np.concatenate([p[0] for p in parts])
    S = None if w.a_type == wl.I8 else np.concatenate([p[1] for p in parts])
    return ref, S


@pytest.mark.slow
@pytest.mark.parametrize("name", ["f16_8192", "i8_8192", "fp8_bf8_8192x16384", "bf8_bf8_8192x16384", "f16_4096",
                                  "bf16_linear_n4096", "bf16_linear_n16"])
def test_workload_full_output(pkg, name):
    """Every configured workload's product compared with the oracle at every
    output (not sampled), in the launch configuration the benchmark times
    (K-blocked A from the GPU compressor, B stored K x N; C and beta as the
    workload has them)."""
    _say(f"workload {name} full output: generating inputs")
    w = wl.make(name)
    A = to_dev(w.A, w.a_type)
    vals_d, meta_d = pkg.prune_compress(A, w.a_type, KBLOCK)
    del A
    C = None if w.C is None else torch.from_numpy(w.C).to(DEV)
    D = pkg.gemm(vals_d, meta_d, to_dev(w.B, w.b_type), C, alpha=w.alpha, beta=w.beta, a_type=w.a_type,
                 b_type=w.b_type)
    torch.cuda.synchronize()
    got = D.cpu().numpy()
    del D, vals_d, meta_d
    _say(f"workload {name} full output: oracle compress")
    ov, om = oracle.prune_compress(w.A, w.a_type)
    _say(f"workload {name} full output: oracle product on host threads")
    ref, S = oracle_full_threaded(ov, om, w)
    if w.a_type == wl.I8:
        bad = got.astype(np.int64) != ref
        assert not bad.any(), f"{int(bad.sum())} of {bad.size} outputs differ"
    else:
        err = np.abs(got.astype(np.float64) - ref)
        bad = ~(err <= 1e-4 * S + 1e-6)
        assert not bad.any(), f"{int(bad.sum())} of {bad.size} outputs outside the bound"
        _say(f"workload {name} full output: worst |err| / S = {np.max(err / (S + 1e-30)):.3g}")


@pytest.mark.parametrize("name", ["f16_8192", "i8_8192", "bf16_linear_n16"])
def test_workload_full_size_row_layout(pkg, name):
    """The benchmark workloads through the ROW (row-major) compressed layout:
    compress bit-exact, the product on sampled outputs, both repeated."""
    _say(f"workload {name} (ROW layout): generating inputs")
    w = wl.make(name)
    A = to_dev(w.A, w.a_type)
    ov, om = oracle.prune_compress(w.A, w.a_type)
    ref_v = None
    for _ in range(2):
        vals_d, meta_d = pkg.prune_compress(A, w.a_type, ROW)
        torch.cuda.synchronize()
        if ref_v is None:
            assert np.array_equal(meta_d.cpu().numpy().view(np.uint32), om), "metadata differs"
            assert np.array_equal(to_host_bits(vals_d, w.a_type).view(ov.dtype), ov), "values differ"
            ref_v, ref_m = vals_d, meta_d
        else:
            assert torch.equal(vals_d.view(torch.uint8), ref_v.view(torch.uint8)) and torch.equal(meta_d, ref_m)
    del A
    B = b_on_dev(w.B, w.b_type, KN)
    D0 = None
    for _ in range(2):
        C = None if w.C is None else torch.from_numpy(w.C).to(DEV)
        D = pkg.gemm(ref_v, ref_m, B, C, alpha=w.alpha, beta=w.beta, a_type=w.a_type, b_type=w.b_type)
        torch.cuda.synchronize()
        if D0 is None:
            check_gemm_sampled(D, ov, om, w)
            D0 = D
        else:
            assert torch.equal(D.view(torch.int32), D0.view(torch.int32)), "product differs between runs"


# ---- decompression and metadata validation -------------------------------------------
def _rand_meta(seed, M, K):
    """Random code words: every code value, valid and invalid groups alike."""
    g = np.random.default_rng(seed)
    return g.integers(0, 2 ** 32, (M, K // 32), dtype=np.uint64).astype(np.uint32)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16, wl.I8, wl.E4M3, wl.E5M2])
@pytest.mark.parametrize("shape", [(1, 32), (129, 160), (300, 4096), (64, 96)])
def test_decompress_matches_oracle(pkg, dtype, shape, layout):
    M, K = shape
    _say(f"decompress dtype={dtype} M={M} K={K} layout={layout}")
    c = wl.random_case(17, M, 16, K, dtype, dtype)
    ov, om = oracle.prune_compress(c.A, dtype)
    for vals, meta in ((ov, om), (ov, _rand_meta(5, M, K))):  # compressor output, then arbitrary codes
        ev, em = in_layout(vals, meta, dtype, layout)
        V = to_dev(ev, dtype)
        Mt = torch.from_numpy(np.ascontiguousarray(em).view(np.int32)).to(DEV)
        D = pkg.decompress(V, Mt, K, dtype, layout)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(D, dtype), oracle.decompress(vals, meta, dtype))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", [wl.F16, wl.I8])
@pytest.mark.parametrize("shape", [(8192, 8192), (4136, 4128)])
def test_decompress_full_size_repeatable(pkg, dtype, shape, layout):
    """Decompression of a full benchmark-size A (and a ragged one whose 16-bit
    workgroups take two blocks), three times into fresh buffers, each compared
    with the oracle over the whole output: a kernel that is right on small
    shapes can still be wrong, or differ from run to run, at full size."""
    M, K = shape
    _say(f"decompress full size dtype={dtype} M={M} K={K} layout={layout}")
    A = wl.small_int_bits((M, K), dtype, 51, -127, 127) if dtype == wl.I8 else \
        wl.random_case(53, M, 16, K, dtype, dtype).A
    ov, om = oracle.prune_compress(A, dtype)
    expect = oracle.decompress(ov, om, dtype)
    ev, em = in_layout(ov, om, dtype, layout)
    V = to_dev(ev, dtype)
    Mt = torch.from_numpy(np.ascontiguousarray(em).view(np.int32)).to(DEV)
    for rep in range(3):
        D = pkg.decompress(V, Mt, K, dtype, layout)
        torch.cuda.synchronize()
        got = to_host_bits(D, dtype)
        assert np.array_equal(got, expect), f"run {rep}: {int((got != expect).sum())} elements differ"
        del D
    # validation at the same size: the compressor's codes are all valid, and
    # arbitrary codes are counted as the oracle counts them
    assert int(pkg.validate_meta(Mt, M, K, dtype, layout).item()) == 0
    rm = _rand_meta(7, M, K)
    _, erm = in_layout(ov, rm, dtype, layout)
    Rt = torch.from_numpy(np.ascontiguousarray(erm).view(np.int32)).to(DEV)
    for _ in range(2):
        assert int(pkg.validate_meta(Rt, M, K, dtype, layout).item()) == oracle.count_invalid(rm, K)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", [wl.F16, wl.I8])
@pytest.mark.parametrize("shape", [(1, 32), (129, 160), (300, 4096), (70, 96), (1000, 4160), (3, 8224)])
def test_validate_meta_counts_like_oracle(pkg, dtype, shape, layout):
    M, K = shape
    _say(f"validate dtype={dtype} M={M} K={K} layout={layout}")
    vals = np.zeros((M, K // 2), wl.STORE[dtype])
    for meta, expect in ((_rand_meta(9, M, K), None), (np.full((M, K // 32), 0x88888888, np.uint32), 0)):
        _, em = in_layout(vals, meta, dtype, layout)
        Mt = torch.from_numpy(np.ascontiguousarray(em).view(np.int32)).to(DEV)
        n = int(pkg.validate_meta(Mt, M, K, dtype, layout).item())
        ref = oracle.count_invalid(meta, K)
        assert n == ref
        if expect is not None:
            assert n == expect


def test_gpu_compress_then_decompress_is_prune(pkg):
    """decompress(compress(A)) on the GPU equals the oracle's pruned A."""
    c = wl.random_case(23, 257, 16, 352, wl.BF16, wl.BF16)
    A = to_dev(c.A, wl.BF16)
    for layout in LAYOUTS:
        V, Mt = pkg.prune_compress(A, layout=layout)
        D = pkg.decompress(V, Mt, 352, layout=layout)
        assert int(pkg.validate_meta(Mt, 257, 352, wl.BF16, layout).item()) == 0
        torch.cuda.synchronize()
        ov, om = oracle.prune_compress(c.A, wl.BF16)
        assert np.array_equal(to_host_bits(D, wl.BF16), oracle.decompress(ov, om, wl.BF16))
