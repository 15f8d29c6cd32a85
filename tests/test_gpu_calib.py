"""GPU checks of the measurement aids in include/sp24_calib.h (not steps of
the 2:4 method): the plain stream reads every byte once and copies the
prefix it is asked to, and the matrix-core stream is deterministic and sees
its operands."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sparse_matrix_sp24_amd as p
    p.sp24_version()
    return p


@pytest.mark.parametrize("workgroups,threads", [(0, 256), (0, 512), (7, 256), (64, 512)])
@pytest.mark.parametrize("read_bytes,write_bytes", [(16, 16), (48 * 1024 + 16, 4096), (3 << 20, (3 << 20) - 16)])
def test_calib_stream_reads_all_and_copies_prefix(pkg, workgroups, threads, read_bytes, write_bytes):
    print(f"calib_stream wg={workgroups} t={threads} r={read_bytes} w={write_bytes}", flush=True)
    g = torch.Generator().manual_seed(read_bytes + workgroups)
    src = torch.randint(0, 256, (read_bytes,), dtype=torch.uint8, generator=g).to(DEV)
    dst = torch.zeros(max(write_bytes, 16), dtype=torch.uint8, device=DEV)
    launched = workgroups if workgroups else -(-read_bytes // (128 * threads))
    sink = torch.zeros(launched, dtype=torch.int32, device=DEV)
    st = pkg.sp24_calib_stream(src.data_ptr(), read_bytes, dst.data_ptr(), write_bytes, sink.data_ptr(), workgroups,
                               threads, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    s = src.cpu().numpy()
    assert np.array_equal(dst.cpu().numpy()[:write_bytes], s[:write_bytes])
    # each 16-byte piece is read by exactly one workgroup, so the xor over
    # the workgroups' sinks is the xor of every 32-bit word of the source
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(s.view(np.uint32))


@pytest.mark.parametrize("pair", ["f16", "i8", "fp8_bf8"])
def test_calib_mfma_deterministic_and_data_dependent(pkg, pair):
    """Two launches on the same operands give the same sinks; with B all
    zero every accumulator stays zero (so every sink is zero), and with
    random operands they are not all zero."""
    a_type, b_type = {"f16": (pkg.SP24_F16, pkg.SP24_F16), "i8": (pkg.SP24_I8, pkg.SP24_I8),
                      "fp8_bf8": (pkg.SP24_FP8_E4M3, pkg.SP24_BF8_E5M2)}[pair]
    print(f"calib_mfma {pair}", flush=True)
    g = torch.Generator().manual_seed(5)
    n_a, n_c, n_b = 3 * 8192, 5 * 2048, 2 * 8192
    # random bytes with the sign/exponent bits of each element kept small so
    # the float types hold finite values
    a = (torch.randint(0, 256, (n_a,), dtype=torch.uint8, generator=g) & 0x3B).to(DEV)
    b = (torch.randint(0, 256, (n_b,), dtype=torch.uint8, generator=g) & 0x3B).to(DEV)
    # positions 0 and 1 in every group
    codes = torch.from_numpy(np.full(n_c // 4, 0x44444444, np.uint32).view(np.int32)).to(DEV)
    wgs, rounds = 6, 3
    sh = torch.cuda.current_stream().cuda_stream

    def run(bt):
        sink = torch.zeros(wgs, dtype=torch.int32, device=DEV)
        assert pkg.sp24_calib_mfma(a.data_ptr(), n_a, codes.data_ptr(), n_c, bt.data_ptr(), n_b, a_type, b_type,
                                   rounds, wgs, sink.data_ptr(), sh) == 0
        torch.cuda.synchronize()
        return sink.cpu().numpy()

    s1, s2 = run(b), run(b)
    assert np.array_equal(s1, s2)
    assert s1.any()
    assert not run(torch.zeros_like(b)).any()


@pytest.mark.parametrize("pair", ["f16", "bf16", "i8", "fp8_bf8"])
def test_calib_mfma_ex_shapes_and_loads(pkg, pair):
    """The 32x32 stream is deterministic and sees its operands (zero B gives
    zero sinks); the direct-to-LDS loads change no accumulator (the sinks
    equal those of the same call without them, in both shapes); shape 16
    without loads is sp24_calib_mfma."""
    a_type, b_type = {"f16": (pkg.SP24_F16, pkg.SP24_F16), "bf16": (pkg.SP24_BF16, pkg.SP24_BF16),
                      "i8": (pkg.SP24_I8, pkg.SP24_I8),
                      "fp8_bf8": (pkg.SP24_FP8_E4M3, pkg.SP24_BF8_E5M2)}[pair]
    print(f"calib_mfma_ex {pair}", flush=True)
    g = torch.Generator().manual_seed(11)
    n_a, n_c, n_b = 3 * 8192, 5 * 2048, 2 * 8192
    a = (torch.randint(0, 256, (n_a,), dtype=torch.uint8, generator=g) & 0x3B).to(DEV)
    b = (torch.randint(0, 256, (n_b,), dtype=torch.uint8, generator=g) & 0x3B).to(DEV)
    codes = torch.from_numpy(np.full(n_c // 4, 0x44444444, np.uint32).view(np.int32)).to(DEV)
    src = torch.randint(0, 256, (3 * 1024 + 512,), dtype=torch.uint8, generator=g).to(DEV)  # uses its first 2 KiB
    wgs, rounds = 5, 4
    sh = torch.cuda.current_stream().cuda_stream

    def run(bt, shape, loads):
        sink = torch.zeros(wgs, dtype=torch.int32, device=DEV)
        assert pkg.sp24_calib_mfma_ex(a.data_ptr(), n_a, codes.data_ptr(), n_c, bt.data_ptr(), n_b, a_type, b_type,
                                      rounds, wgs, shape, src.data_ptr() if loads else None,
                                      src.numel() if loads else 0, sink.data_ptr(), sh) == 0
        torch.cuda.synchronize()
        return sink.cpu().numpy()

    base = torch.zeros(wgs, dtype=torch.int32, device=DEV)
    assert pkg.sp24_calib_mfma(a.data_ptr(), n_a, codes.data_ptr(), n_c, b.data_ptr(), n_b, a_type, b_type, rounds,
                               wgs, base.data_ptr(), sh) == 0
    torch.cuda.synchronize()
    s16 = run(b, 16, False)
    assert np.array_equal(s16, base.cpu().numpy())
    assert np.array_equal(run(b, 16, True), s16)
    s32 = run(b, 32, False)
    assert s32.any()
    assert np.array_equal(run(b, 32, False), s32)
    assert np.array_equal(run(b, 32, True), s32)
    assert not run(torch.zeros_like(b), 32, True).any()
