#!/usr/bin/env python3
"""Benchmark of the 2:4 sparse hot path on one MI355X.

One step = sp24_prune_compress(A) followed by sp24_gemm(A_vals, meta, B) on a
seeded synthetic workload (default: fp16, M = N = K = 8192, A and B ~ N(0,1),
A pruned to 2:4 by the compress kernel, fp32 output, beta = 0).  Inputs are
resident in HBM before the timed region; the timed region is exactly --steps
steps bracketed by torch.cuda.synchronize().  Before the --warmup steps the
step runs untimed for --settle-s seconds (default 0.2) so the GPU's clocks
have left their idle state: with only a few milliseconds of warm-up the
timed steps measured about 7 % slower than in steady state.

Prints ONE JSON line: value = dense-equivalent TFLOP/s of the whole step
(2*M*N*K per step / step time); `roofline` describes the dominant kernel
(the GEMM) against the sparse-MFMA peak, timed with HIP events on the stream
the kernels run on; `cpu_baseline` times the CPU oracle on a bounded row
sample on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks.  The sparse matrix-core peak is twice the dense one
# (one 16x16x64 fp16 smfmac = 32768 dense-equivalent flop per 16 cycles per
# SIMD: 1024 SIMDs * 2048 flop/clk * 2.4 GHz = 5033 TFLOP/s).
PEAK_SPARSE_TFLOPS = {"fp16": 5033.2, "bf16": 5033.2, "int8": 10066.3, "fp8": 10066.3}
PEAK_HBM_GBPS = 8000.0

# Call bookkeeping for kernel-trace summaries.  Each library call here
# launches exactly one kernel, so counting the calls of each entry point
# tells which dispatches of a trace of this run belong to which measured
# region; the regions are printed to stderr at the end ("bench-regions").
CALLS = {"compress": 0, "gemm": 0, "stream": 0}
REGIONS = {}


def region_open(name, key):
    REGIONS[name] = {"calls_of": key, "first": CALLS[key]}


def region_close(name):
    r = REGIONS[name]
    r["end"] = CALLS[r["calls_of"]]


# the headline metric (the default workload); other workloads name themselves
METRIC = "dense-equiv TFLOP/s of 2:4 sparse GEMM (fp16, 8192^3) + % of smfmac peak"

WORKLOADS = {
    # name -> (workload key, dtype label)
    "f16_8192": "fp16",
    "f16_4096": "fp16",
    "bf16_linear_n16": "bf16",
    "bf16_linear_n4096": "bf16",
    "i8_8192": "int8",
    "fp8_bf8_8192x16384": "fp8",
    "bf8_bf8_8192x16384": "fp8",
}


def src_hash(*rel):
    h = hashlib.sha256()
    for r in rel:
        with open(os.path.join(ROOT, r), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_name(workload, layout, b_layout):
    """Stem of the profiles/ files for a run: the workload, plus the layouts
    when they are not the defaults (kblock, kn)."""
    extra = "" if (layout, b_layout) == ("kblock", "kn") else f"_{layout}_{b_layout}"
    return f"{workload}{extra}"


def load_traffic(name, kernel_src_hash):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
    scaled by the same counters' reading for a plain copy of known size.
    Returned only if taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_src_hash") != kernel_src_hash:
        return None
    return t.get("gemm_bytes_per_launch")


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, rows, max_threads=16):
    """Time the oracle (as it stands) on `rows` rows of the workload on the
    host cores: prune+compress of those rows of A and those rows of the
    product (full N and K).  One row block per thread, at most `max_threads`
    threads (the CPU share that goes with one GPU on the GPU hosts)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    oracle.build(force=False)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    threads = max(1, min(affinity, max_threads, rows))
    A = np.ascontiguousarray(w.A[:rows])
    bounds = np.linspace(0, rows, threads + 1).astype(int)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: oracle.prune_compress(A[bounds[i]:bounds[i + 1]], w.a_type), range(threads)))
    t1 = time.perf_counter()
    if w.a_type == oracle.I8:
        work = lambda i: oracle.gemm_i64(parts[i][0], parts[i][1], w.B)  # noqa: E731
    else:
        work = lambda i: oracle.gemm_f64(parts[i][0], parts[i][1], w.a_type, w.B, w.b_type, want_abs=False)  # noqa: E731
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(threads)))
    t2 = time.perf_counter()
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": round(flops / (t2 - t0) / 1e12, 6),
        "unit": "TFLOP/s (dense-equivalent, prune+compress+product)",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} of {w.M} rows: prune+compress of those rows of A and those rows of the product "
                  f"(full N={w.N}, K={w.K}); fp64/int64 plain C, one row block per thread",
        "threads_used": threads,
        "host_cpu_count": os.cpu_count(),
        "affinity_cpu_count": affinity,
        "cpu_model": cpu_model(),
        "compress_s": round(t1 - t0, 3),
        "product_s": round(t2 - t1, 3),
    }


def compress_launch_shape(M, K, es, layout):
    """(workgroups, threads) of the compress kernel the library launches."""
    if layout == 1:  # K-blocked
        nblk, row_tiles = -(-K // (64 if es == 2 else 128)), -(-M // 128)
        if es == 2:
            nb = 2 if row_tiles * (-(-nblk // 2)) >= 1024 else 1
            return row_tiles * (-(-nblk // nb)), 512
        return row_tiles * nblk, 512
    return -(-(M * K * es // 16) // 1024), 256


def stream_floor(pkg, read_bytes, write_bytes, workgroups, threads, stream, rot_bytes=2 << 30):
    """Microseconds per launch of sp24_calib_stream (a plain stream of the
    same bytes; workgroups > 0: that grid, grid-stride; 0: one pass with
    eight loads in flight per thread), on data that is not in any cache:
    rotating over >= rot_bytes of buffers, one untimed pass, then one pass
    of back-to-back launches between two HIP events."""
    import torch
    read_bytes, write_bytes = -(-read_bytes // 16) * 16, -(-write_bytes // 16) * 16
    n = max(2, -(-rot_bytes // (read_bytes + write_bytes)))
    src = [torch.empty(read_bytes, dtype=torch.uint8, device="cuda:0") for _ in range(n)]
    dst = [torch.empty(max(write_bytes, 16), dtype=torch.uint8, device="cuda:0") for _ in range(n)]
    launched = workgroups if workgroups > 0 else -(-read_bytes // (128 * threads))  # 0: one pass
    sink = torch.zeros(launched, dtype=torch.int32, device="cuda:0")
    sh = stream.cuda_stream

    def one(i):
        st = pkg.sp24_calib_stream(src[i].data_ptr(), read_bytes, dst[i].data_ptr(), write_bytes, sink.data_ptr(),
                                   workgroups, threads, sh)
        CALLS["stream"] += 1
        if st:
            raise pkg.Sp24Error(st, "sp24_calib_stream")

    for i in range(n):
        one(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    name = f"stream_floor_{read_bytes}_{write_bytes}_{workgroups}_{threads}"
    region_open(name, "stream")
    e0.record(stream)
    for i in range(n):
        one(i)
    e1.record(stream)
    region_close(name)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    del src, dst
    torch.cuda.empty_cache()
    return us


def measure_cold(pkg, w, A, vals, meta, B, C, layout, b_layout, stream, ws, rot_bytes=2 << 30):
    """Kernels on data that is not in any cache.  Each call works on its own
    copy of its inputs (and outputs), rotating over at least `rot_bytes` of
    copies, so that by the time a copy is used again more than the 256 MB
    Infinity Cache has been streamed since; one untimed pass over the
    rotation, then one pass timed between two HIP events on the launch
    stream (back-to-back launches: the launch overhead is hidden, as in a
    batch).  compress: copies of A, A_vals and meta; gemm: copies of A_vals
    and meta (and of B when it is larger than 1 MiB; a small-N B is the
    activations, which a caller has just written)."""
    import torch
    sh = stream.cuda_stream

    def rotate(tensors, bytes_each, fn, key):
        n = max(2, -(-rot_bytes // max(1, bytes_each)))
        copies = [[t.clone() for t in tensors] for _ in range(n)]
        torch.cuda.synchronize()
        for c in copies:
            fn(*c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        region_open("cold_" + key, key)
        e0.record(stream)
        for c in copies:
            fn(*c)
        e1.record(stream)
        region_close("cold_" + key)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n * 1e3
        del copies
        torch.cuda.empty_cache()
        return us, n

    def check(st, what):
        if st:
            raise pkg.Sp24Error(st, what)

    def comp(a, v, m):
        CALLS["compress"] += 1
        check(pkg.sp24_prune_compress(a.data_ptr(), v.data_ptr(), m.data_ptr(), w.M, w.K, w.a_type, layout, sh),
              "sp24_prune_compress")

    cb = vals.numel() * vals.element_size() + meta.numel() * meta.element_size()
    ab = A.numel() * A.element_size()
    comp_us, nc = rotate([A, vals, meta], ab + cb, comp, "compress")
    big_b = B.numel() * B.element_size() > (1 << 20)

    def gem(v, m, *rest):
        CALLS["gemm"] += 1
        b = rest[0] if big_b else B
        check(pkg.sp24_gemm(v.data_ptr(), m.data_ptr(), w.a_type, layout, b.data_ptr(), w.b_type, b_layout,
                            C.data_ptr(), w.M, w.N, w.K, w.alpha, w.beta, ws.data_ptr(), ws.numel(), sh),
              "sp24_gemm")

    gin = [vals, meta] + ([B] if big_b else [])
    gbytes = sum(t.numel() * t.element_size() for t in gin)
    gemm_us, ng = rotate(gin, gbytes, gem, "gemm")
    return comp_us, nc, gemm_us, ng


def mfma_ceiling(pkg, w, vals, meta, B, layout, stream, launches=10, shape=16, loads=False):
    """TFLOP/s (dense-equivalent) of sp24_calib_mfma_ex: the product's sparse
    instructions for this type pair with their operands (taken from this
    workload's compressed A, codes and B) held in registers, no memory
    traffic.  One workgroup per CU and as many instructions per launch as the
    product issues; back-to-back launches between two HIP events.  shape 32
    issues the 32x32 instructions of the pair instead (the same work);
    loads=True adds the product's direct-to-LDS loads per wave and k-step
    (1 KiB each, from the first 2 MiB of B, which stays in the L2 as the
    product's staged tiles mostly do)."""
    import torch
    from structured_sparse_matrix_sp24_amd import workloads as wl
    kstep = 64 if wl.ESIZE[w.a_type] == 2 else 128
    tiles = -(-w.M // 256) * -(-w.N // 256)
    rounds = max(1, tiles * -(-w.K // kstep) // 256)
    wgs = 256
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda:0")
    vb = pkg.sp24_values_bytes(w.M, w.K, w.a_type, layout)
    mb = pkg.sp24_meta_bytes(w.M, w.K, w.a_type, layout)
    bb = B.numel() * B.element_size()
    src, src_bytes = (B.data_ptr(), min(bb, 2 << 20)) if loads else (None, 0)

    def one():
        st = pkg.sp24_calib_mfma_ex(vals.data_ptr(), vb, meta.data_ptr(), mb, B.data_ptr(), bb, w.a_type, w.b_type,
                                    rounds, wgs, shape, src, src_bytes, sink.data_ptr(), stream.cuda_stream)
        if st:
            raise pkg.Sp24Error(st, "sp24_calib_mfma_ex")

    for _ in range(3):
        one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        one()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / launches * 1e3
    flop = wgs * 8.0 * rounds * 32 * 2 * 16 * 16 * kstep
    return us, flop / us / 1e6, rounds, wgs


def dense_reference(w, A, B, b_layout_nk, stream, launches=10):
    """The same product with the dense, pruned A through the platform's own
    dense GEMM (torch -> hipBLASLt): fp16 / bf16 with a 16-bit output
    (torch.matmul), int8 with an int32 output (torch._int_mm), 8-bit floats
    with an fp32 output (torch._scaled_mm, unit scales).  Returns (us, what)
    or (None, reason).  Context for what the 2:4 layout buys; not part of
    the step."""
    import torch
    from structured_sparse_matrix_sp24_amd import workloads as wl
    Bkn = B.t() if b_layout_nk else B  # K x N view
    try:
        if w.a_type in (wl.F16, wl.BF16):
            Bc = Bkn.contiguous()
            fn = lambda: torch.matmul(A, Bc)  # noqa: E731
            what = "torch.matmul (hipBLASLt), 16-bit output"
        elif w.a_type == wl.I8:
            Bc = Bkn.contiguous()
            fn = lambda: torch._int_mm(A, Bc)  # noqa: E731
            what = "torch._int_mm (hipBLASLt), int32 output"
        else:
            Bt = Bkn.t().contiguous().t()  # column-major K x N, as _scaled_mm wants
            one = torch.ones((), dtype=torch.float32, device=A.device)
            fn = lambda: torch._scaled_mm(A, Bt, one, one, out_dtype=torch.float32)  # noqa: E731
            what = "torch._scaled_mm (hipBLASLt), fp32 output, unit scales"
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches * 1e3, what
    except Exception as e:  # a type pair the platform library does not take
        return None, f"not measured: {type(e).__name__}: {str(e)[:120]}"


def measure_next_rows(pkg, w, vals, meta, B, layout, b_layout, stream, ws, launches=20):
    """The calls adjacent to the hot path, each timed over back-to-back
    launches between two HIP events on the launch stream: sp24_decompress
    (bytes: values + metadata + dense A), sp24_validate_meta (bytes: metadata)
    and, for floating inputs, sp24_gemm_ex with a 16-bit output and a bias."""
    import torch
    from structured_sparse_matrix_sp24_amd import workloads as wl
    sh = stream.cuda_stream
    es = wl.ESIZE[w.a_type]
    cbytes = pkg.sp24_values_bytes(w.M, w.K, w.a_type, layout) + pkg.sp24_meta_bytes(w.M, w.K, w.a_type, layout)
    mbytes = pkg.sp24_meta_bytes(w.M, w.K, w.a_type, layout)
    dense = torch.empty(w.M * w.K * es, dtype=torch.uint8, device="cuda:0")
    bad = torch.zeros(1, dtype=torch.int64, device="cuda:0")

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    def check(st, what):
        if st:
            raise pkg.Sp24Error(st, what)

    out = {}
    us = timed(lambda: check(pkg.sp24_decompress(vals.data_ptr(), meta.data_ptr(), dense.data_ptr(), w.M, w.K,
                                                  w.a_type, layout, sh), "sp24_decompress"), launches)
    nb = cbytes + w.M * w.K * es
    out["decompress"] = {"us": round(us, 2), "bytes": nb, "GB/s": round(nb / us / 1e3, 1),
                         "frac_hbm": round(nb / us / 1e3 / PEAK_HBM_GBPS, 4)}
    us = timed(lambda: check(pkg.sp24_validate_meta(meta.data_ptr(), w.M, w.K, w.a_type, layout, bad.data_ptr(),
                                                     sh), "sp24_validate_meta"), launches)
    out["validate_meta"] = {"us": round(us, 2), "bytes": mbytes, "GB/s": round(mbytes / us / 1e3, 1),
                            "frac_hbm": round(mbytes / us / 1e3 / PEAK_HBM_GBPS, 4)}
    if w.a_type != wl.I8:
        D16 = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda:0")
        bias = torch.ones(w.N, dtype=torch.float32, device="cuda:0")
        def gemm_ex():
            CALLS["gemm"] += 1  # the same product kernel as sp24_gemm
            check(pkg.sp24_gemm_ex(vals.data_ptr(), meta.data_ptr(), w.a_type, layout, B.data_ptr(), w.b_type,
                                   b_layout, D16.data_ptr(), wl.F16, bias.data_ptr(), w.M, w.N, w.K, 1.0, 0.0,
                                   ws.data_ptr(), ws.numel(), sh), "sp24_gemm_ex")

        us = timed(gemm_ex, 5)
        tf = 2.0 * w.M * w.N * w.K / (us * 1e-6) / 1e12
        out["gemm_ex_f16_out_bias"] = {"us": round(us, 1), "TFLOP/s": round(tf, 1)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.2,
                    help="untimed seconds of steps before the warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="f16_8192", choices=sorted(WORKLOADS))
    ap.add_argument("--layout", default="kblock", choices=["kblock", "row"],
                    help="compressed layout the step writes and the GEMM reads")
    ap.add_argument("--b-layout", default="kn", choices=["kn", "nk"],
                    help="how B is stored: K x N (kn) or transposed, N x K (nk, e.g. activations)")
    ap.add_argument("--cpu-rows", type=int, default=None, help="rows of the oracle sample (default: sized to ~15 s)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache measurement (compress and gemm rotating over 2 GiB of input copies)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the matrix-core ceiling (sp24_calib_mfma) of the large-N products")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip timing the same product through the platform's dense GEMM (context)")
    ap.add_argument("--next-rows", action="store_true",
                    help="also time the adjacent calls (decompress, validate_meta, 16-bit output with bias) "
                         "after the timed steps and add them to the line as next_rows")
    ap.add_argument("--gemm-only-launches", type=int, default=0,
                    help="after the timed steps, launch only the GEMM this many times (for profilers)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes 5 times (counter calibration) and exit")
    args = ap.parse_args()

    if args.copy_bytes:
        import torch
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 5}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only (the 2:4 path has no inter-GPU step); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import structured_sparse_matrix_sp24_amd as pkg
    from structured_sparse_matrix_sp24_amd import workloads as wl

    pkg.sp24_version()  # fails loudly if libsp24.so is missing
    dev = torch.device("cuda:0")
    w = wl.make(args.workload)
    label = WORKLOADS[args.workload]
    tview = {wl.F16: (np.int16, torch.float16), wl.BF16: (np.int16, torch.bfloat16), wl.I8: (np.int8, torch.int8),
             wl.E4M3: (np.uint8, torch.float8_e4m3fn), wl.E5M2: (np.uint8, torch.float8_e5m2)}

    def up(bits, t):
        nv, tv = tview[t]
        return torch.from_numpy(np.ascontiguousarray(bits).view(nv)).to(dev).view(tv)

    A = up(w.A, w.a_type)
    B = up(w.B, w.b_type)
    b_layout = {"kn": pkg.SP24_B_KN, "nk": pkg.SP24_B_NK}[args.b_layout]
    if b_layout == pkg.SP24_B_NK:  # the same B, stored transposed (set-up, not timed)
        B = B.t().contiguous()
    out_dtype = torch.int32 if w.a_type == wl.I8 else torch.float32
    C = torch.from_numpy(w.C).to(dev) if w.C is not None else torch.empty((w.M, w.N), dtype=out_dtype, device=dev)
    C0 = C.clone() if w.beta != 0.0 else None
    layout = {"kblock": pkg.SP24_LAYOUT_KBLOCK, "row": pkg.SP24_LAYOUT_ROW}[args.layout]
    vshape, mshape = pkg.compressed_shapes(w.M, w.K, w.a_type, layout)
    vals = torch.empty(vshape, dtype=A.dtype, device=dev)
    meta = torch.empty(mshape, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # small-N products split K over workgroups and need a workspace whose
    # counters start at zero (the library leaves them at zero)
    ws_bytes = pkg.sp24_gemm_workspace_bytes(w.M, w.N, w.K, w.a_type, w.b_type)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def compress():
        CALLS["compress"] += 1
        st = pkg.sp24_prune_compress(A.data_ptr(), vals.data_ptr(), meta.data_ptr(), w.M, w.K, w.a_type, layout,
                                      sh)
        if st:
            raise pkg.Sp24Error(st, "sp24_prune_compress")

    def gemm():
        CALLS["gemm"] += 1
        st = pkg.sp24_gemm(vals.data_ptr(), meta.data_ptr(), w.a_type, layout, B.data_ptr(), w.b_type, b_layout,
                           C.data_ptr(), w.M, w.N, w.K, w.alpha, w.beta, ws.data_ptr(), ws_bytes, sh)
        if st:
            raise pkg.Sp24Error(st, "sp24_gemm")

    def reset_c():
        if C0 is not None:  # beta != 0: keep each step's C input identical
            C.copy_(C0)

    # clock settle: untimed steps for about --settle-s seconds, then the warm-up steps
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(8):
            reset_c()
            compress()
            gemm()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        reset_c()
        compress()
        gemm()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    region_open("steps_compress", "compress")
    region_open("steps_gemm", "gemm")
    t0 = time.perf_counter()
    for s in range(args.steps):
        e0, e1, e2 = ev[s]
        e0.record(stream)
        compress()
        e1.record(stream)
        gemm()
        e2.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    region_close("steps_compress")
    region_close("steps_gemm")
    if C0 is not None:
        # the timed loop accumulated beta*C repeatedly; restore and run one clean step
        reset_c()
        compress()
        gemm()
        torch.cuda.synchronize()
    comp_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    gemm_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    for _ in range(args.gemm_only_launches):
        gemm()
    torch.cuda.synchronize()
    next_rows = measure_next_rows(pkg, w, vals, meta, B, layout, b_layout, stream, ws) if args.next_rows else None
    cold = None if args.no_cold else measure_cold(pkg, w, A, vals, meta, B, C, layout, b_layout, stream, ws)
    ceiling = variants = None
    if not (args.no_ceiling or w.N <= 64):
        ceiling = mfma_ceiling(pkg, w, vals, meta, B, layout, stream)
        variants = {name: mfma_ceiling(pkg, w, vals, meta, B, layout, stream, shape=sh_, loads=ld_)
                    for name, sh_, ld_ in (("with_loads", 16, True), ("shape_32x32", 32, False),
                                           ("shape_32x32_with_loads", 32, True))}
    dense = None
    if not args.no_dense:
        # the pruned A, dense: the product the sparse kernel computes
        Ap = torch.empty_like(A)
        st = pkg.sp24_decompress(vals.data_ptr(), meta.data_ptr(), Ap.data_ptr(), w.M, w.K, w.a_type, layout, sh)
        if st:
            raise pkg.Sp24Error(st, "sp24_decompress")
        dense = dense_reference(w, Ap, B, b_layout == pkg.SP24_B_NK, stream)
        del Ap

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flop = 2.0 * w.M * w.N * w.K
    es_a = wl.ESIZE[w.a_type]
    es_b = wl.ESIZE[w.b_type]
    cbytes = pkg.sp24_values_bytes(w.M, w.K, w.a_type, layout) + pkg.sp24_meta_bytes(w.M, w.K, w.a_type, layout)
    comp_bytes = es_a * w.M * w.K + cbytes
    gemm_bytes = cbytes + es_b * w.K * w.N + 4 * w.M * w.N * (2 if w.beta != 0.0 else 1)
    gemm_tflops = flop / (gemm_ms * 1e-3) / 1e12
    comp_gbps = comp_bytes / (comp_ms * 1e-3) / 1e9
    gemm_gbps = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    khash = src_hash("structured_sparse_matrix_sp24_amd/csrc/sp24_gemm.hip",
                     "structured_sparse_matrix_sp24_amd/csrc/sp24_internal.hpp")
    traffic = load_traffic(traffic_name(args.workload, args.layout, args.b_layout), khash)
    hbm_bound = w.N <= 64
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gemm_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gemm_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "kernel": "sp24 gemm (small-N)", "kernel_ms": round(gemm_ms, 5),
                "algorithmic_bytes": gemm_bytes}
    else:
        peak = PEAK_SPARSE_TFLOPS[label]
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / peak, 4), "traffic": traffic,
                "kernel": "sp24 gemm (256x256 tile)", "kernel_ms": round(gemm_ms, 5),
                "algorithmic_flop": flop}
    res = {
        "metric": METRIC if args.workload == "f16_8192" else
        f"dense-equiv TFLOP/s of 2:4 sparse GEMM ({args.workload}, "
        f"{w.M}x{w.N}x{w.K}) + % of smfmac peak",
        "value": round(flop / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp16": "f16", "bf16": "bf16", "int8": "i8", "fp8": "fp8"}[label] + "->f32" if label != "int8"
        else "i8->i32",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": w.M, "N": w.N, "K": w.K, "a_type": wl_name(w.a_type),
                   "b_type": wl_name(w.b_type), "alpha": w.alpha, "beta": w.beta, "layout": args.layout,
                   "b_layout": args.b_layout,
                   "step": "sp24_prune_compress(A) + sp24_gemm(A_vals, meta, B, C)"},
        "gemm_tflops": round(gemm_tflops, 1),
        "gemm_frac_sparse_peak": round(gemm_tflops / PEAK_SPARSE_TFLOPS[label], 4),
        "gemm_ms": round(gemm_ms, 5),
        "compress_ms": round(comp_ms, 5),
        "compress_gbps": round(comp_gbps, 1),
        "compress_frac_hbm": round(comp_gbps / PEAK_HBM_GBPS, 4),
        "roofline": roof,
        "kernel_src_hash": khash,
    }
    if cold is not None:
        c_us, nc, g_us, ng = cold
        # the best of: a plain stream with the kernel's own grid, and one-pass
        # streams of 256 and 512 threads per workgroup
        def best_floor(rb, wb, grid):
            got = [(stream_floor(pkg, rb, wb, g, t, stream), [g, t]) for g, t in (grid, (0, 256), (0, 512))]
            return min(got)
        cwg, cth = compress_launch_shape(w.M, w.K, es_a, layout)
        floor_c, shape_c = best_floor(es_a * w.M * w.K, cbytes, (cwg, cth))
        floor_g = shape_g = None
        if hbm_bound:  # the small-N product: one 16-row tile per 512-thread workgroup
            floor_g, shape_g = best_floor(cbytes + es_b * w.K * w.N, 4 * w.M * w.N * (2 if w.beta != 0.0 else 1),
                                          (-(-w.M // 16), 512))
        res["cold"] = {
            "note": "each launch on its own copy of its inputs, rotating over >= 2 GiB of copies; "
                    "back-to-back launches between two HIP events",
            "compress": {"us": round(c_us, 2), "copies": nc, "bytes": comp_bytes,
                         "GB/s": round(comp_bytes / c_us / 1e3, 1),
                         "frac_hbm": round(comp_bytes / c_us / 1e3 / PEAK_HBM_GBPS, 4),
                         "stream_floor_us": round(floor_c, 2),
                         "stream_floor_GB/s": round(comp_bytes / floor_c / 1e3, 1),
                         "frac_of_floor": round(floor_c / c_us, 4),
                         "floor_launch": shape_c},
            "gemm": {"us": round(g_us, 2), "copies": ng, "bytes": gemm_bytes,
                     "GB/s": round(gemm_bytes / g_us / 1e3, 1),
                     "frac_hbm": round(gemm_bytes / g_us / 1e3 / PEAK_HBM_GBPS, 4),
                     "TFLOP/s": round(flop / g_us / 1e6, 1),
                     "frac_sparse_peak": round(flop / g_us / 1e6 / PEAK_SPARSE_TFLOPS[label], 4)},
        }
        if floor_g is not None:
            res["cold"]["gemm"].update({"stream_floor_us": round(floor_g, 2),
                                        "stream_floor_GB/s": round(gemm_bytes / floor_g / 1e3, 1),
                                        "frac_of_floor": round(floor_g / g_us, 4),
                                        "floor_launch": shape_g})
    if ceiling is not None:
        c_us, c_tf, c_rounds, c_wgs = ceiling
        res["mfma_ceiling"] = {
            "note": "sp24_calib_mfma: the product's sparse instructions on this workload's operands held in "
                    "registers, no memory traffic; as many instructions per launch as the product",
            "us": round(c_us, 1), "TFLOP/s": round(c_tf, 1),
            "frac_sparse_peak": round(c_tf / PEAK_SPARSE_TFLOPS[label], 4),
            "gemm_frac_of_ceiling": round(gemm_tflops / c_tf, 4),
            "launch": {"workgroups": c_wgs, "rounds": c_rounds},
            "variants_note": "with_loads: the same stream with the product's direct-to-LDS loads per wave and k-step "
                             "issued between the instructions (no fragment reads); shape_32x32: the pair's 32x32 "
                             "sparse instructions instead, the same work",
        }
        for name, (v_us, v_tf, _, _) in variants.items():
            res["mfma_ceiling"][name] = {"us": round(v_us, 1), "TFLOP/s": round(v_tf, 1),
                                         "frac_sparse_peak": round(v_tf / PEAK_SPARSE_TFLOPS[label], 4),
                                         "gemm_frac": round(gemm_tflops / v_tf, 4)}
    if dense is not None:
        d_us, d_what = dense
        res["dense_reference"] = {"what": d_what, "note": "the same product with the dense (pruned) A, for context"}
        if d_us is not None:
            res["dense_reference"].update({"us": round(d_us, 1), "TFLOP/s": round(flop / d_us / 1e6, 1),
                                           "sparse_speedup": round(d_us / (gemm_ms * 1e3), 3)})
    if next_rows is not None:
        res["next_rows"] = next_rows
    if not args.no_cpu:
        rows = args.cpu_rows
        if rows is None:
            # the oracle does ~2e9 multiply-adds per second per core on an MI355X
            # host (measured): ~4.8e11 of them is ~15 s on 16 cores (capped at all M rows)
            rows = max(1, min(w.M, int(4.8e11 / max(1, w.N * w.K // 2))))
        res["cpu_baseline"] = cpu_baseline(w, rows)
    print("bench-regions " + json.dumps(REGIONS), file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def wl_name(t):
    return {1: "fp16", 2: "bf16", 3: "int8", 4: "fp8_e4m3", 5: "bf8_e5m2"}[t]


if __name__ == "__main__":
    main()
