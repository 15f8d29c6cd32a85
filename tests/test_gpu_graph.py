"""The two hot-path calls captured in a HIP graph and replayed.

sp24_prune_compress and sp24_gemm only enqueue kernels on the caller's
stream (no allocation, no memset, no host synchronisation), so a caller can
capture them.  Each case captures compress + product (with a copy of C into
D first when beta != 0), replays the graph several times with eager work and
synchronisations in between, clears the outputs before each replay, and
checks every replay bit for bit against the same calls made eagerly, which
the parity tests compare with the oracle.
"""
import numpy as np
import pytest

from structured_sparse_matrix_sp24_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
TVIEW = {wl.F16: torch.float16, wl.BF16: torch.bfloat16, wl.I8: torch.int8, wl.E4M3: torch.float8_e4m3fn,
         wl.E5M2: torch.float8_e5m2}
NPV = {wl.F16: np.int16, wl.BF16: np.int16, wl.I8: np.int8, wl.E4M3: np.uint8, wl.E5M2: np.uint8}
F32, I32 = 6, 7  # output types of include/sp24.h (SP24_F32, SP24_I32)


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sparse_matrix_sp24_amd as p
    p.sp24_version()
    return p


def _dev(bits, t):
    return torch.from_numpy(np.ascontiguousarray(bits).view(NPV[t])).to(DEV).view(TVIEW[t])


@pytest.mark.parametrize("a_type,b_type,M,N,K,beta,out", [
    (wl.F16, wl.F16, 300, 272, 640, 0.0, F32),     # large-tile kernel, ragged M
    (wl.BF16, wl.BF16, 520, 16, 1024, 0.0, F32),   # small-N kernel
    (wl.I8, wl.I8, 512, 512, 512, 1.0, I32),       # int8, D = acc + C
    (wl.E4M3, wl.E5M2, 256, 96, 384, 0.5, wl.F16),    # 8-bit floats, fp16 output with beta * C and a bias
])
def test_graph_replay_matches_eager(pkg, a_type, b_type, M, N, K, beta, out):
    print(f"graph a={a_type} b={b_type} M={M} N={N} K={K} beta={beta} out={out}", flush=True)
    c = wl.random_case(31, M, N, K, a_type, b_type)
    A, B = _dev(c.A, a_type), _dev(c.B, b_type)
    lay = pkg.SP24_LAYOUT_KBLOCK
    vs, ms = pkg.compressed_shapes(M, K, a_type, lay)
    ct = {F32: torch.float32, I32: torch.int32, wl.F16: torch.float16}[out]
    g = torch.Generator().manual_seed(7)
    C0 = (torch.randint(-50, 50, (M, N), generator=g) if out == I32 else torch.randn(M, N, generator=g)).to(ct).to(DEV)
    bias = torch.randn(N, generator=g).to(DEV) if out == wl.F16 else None
    ws_bytes = pkg.sp24_gemm_workspace_bytes(M, N, K, a_type, b_type)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)

    def step(vals, meta, D, stream):
        sh = stream.cuda_stream
        assert pkg.sp24_prune_compress(A.data_ptr(), vals.data_ptr(), meta.data_ptr(), M, K, a_type, lay, sh) == 0
        if beta != 0.0:
            D.copy_(C0)
        st = pkg.sp24_gemm_ex(vals.data_ptr(), meta.data_ptr(), a_type, lay, B.data_ptr(), b_type, pkg.SP24_B_KN,
                              D.data_ptr(), out, None if bias is None else bias.data_ptr(), M, N, K, 1.0, beta,
                              ws.data_ptr(), ws_bytes, sh)
        assert st == 0

    # eager reference
    ev = torch.empty(vs, dtype=A.dtype, device=DEV)
    em = torch.empty(ms, dtype=torch.int32, device=DEV)
    eD = torch.empty((M, N), dtype=ct, device=DEV)
    step(ev, em, eD, torch.cuda.current_stream())
    torch.cuda.synchronize()

    # capture
    gv = torch.empty(vs, dtype=A.dtype, device=DEV)
    gm = torch.empty(ms, dtype=torch.int32, device=DEV)
    gD = torch.empty((M, N), dtype=ct, device=DEV)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(gv, gm, gD, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays; clear the outputs so each replay must rewrite them
        for t in (gv, gm, gD):
            t.view(torch.uint8).fill_(0xA5)
        x = torch.randn(1024, 1024, device=DEV)
        (x @ x).sum().item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gm, em), f"replay {rep}: metadata differs"
        assert torch.equal(gv.view(torch.uint8), ev.view(torch.uint8)), f"replay {rep}: values differ"
        assert torch.equal(gD.view(torch.uint8), eD.view(torch.uint8)), f"replay {rep}: product differs"
