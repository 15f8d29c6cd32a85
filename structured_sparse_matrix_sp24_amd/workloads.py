"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

Both the GPU path and the CPU oracle are fed from here, so they see
byte-identical inputs.  Nothing in this module prunes, compresses or
multiplies: it draws numbers and rounds them into the storage formats.

Recipe (shared by every workload):
  * one ``numpy.random.Generator(PCG64(SeedSequence([seed, stream])))`` per
    tensor, stream A=0, B=1, C=2, sparsity pattern=3;
  * draws in float64, then rounded to the element type with torch's CPU
    round-to-nearest-even conversion (values for fp8 E4M3 clipped to +-448
    first, the format's largest finite value);
  * large tensors are drawn in row blocks of a fixed size, so the same
    (seed, shape) always gives the same bits.

Element type codes match the library's public enum: 1 fp16, 2 bf16, 3 int8,
4 fp8 E4M3 (OCP), 5 bf8 E5M2 (OCP).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16, BF16, I8, E4M3, E5M2 = 1, 2, 3, 4, 5
ESIZE = {F16: 2, BF16: 2, I8: 1, E4M3: 1, E5M2: 1}
STORE = {F16: np.uint16, BF16: np.uint16, I8: np.int8, E4M3: np.uint8, E5M2: np.uint8}
_CHUNK = 1 << 22  # elements per draw block


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def quantize(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values into the storage bits of ``dtype`` (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    if dtype == F16:
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    if dtype == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == E4M3:
        return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if dtype == E5M2:
        return t.to(torch.float8_e5m2).view(torch.uint8).numpy()
    if dtype == I8:
        return np.rint(x).astype(np.int8)
    raise ValueError(dtype)


def _normal_bits(g, shape, dtype, std=1.0):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORE[dtype])
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = quantize(g.standard_normal(e - s) * std, dtype)
    return out.reshape(shape)


def _uniform_bits(g, shape, dtype, lo, hi):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORE[dtype])
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = quantize(g.uniform(lo, hi, e - s), dtype)
    return out.reshape(shape)


def _uniform_int8(g, shape, nonzero=False):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int8)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        if nonzero:  # uniform over [-127,-1] U [1,127]
            v = g.integers(1, 255, e - s)  # 1..254
            out[s:e] = np.where(v <= 127, v - 128, v - 127).astype(np.int8)
        else:
            out[s:e] = g.integers(-127, 128, e - s).astype(np.int8)
    return out.reshape(shape)


@dataclass
class Workload:
    name: str
    M: int
    N: int
    K: int
    a_type: int
    b_type: int
    alpha: float
    beta: float
    A: np.ndarray            # dense M x K bits (before pruning)
    B: np.ndarray            # K x N bits
    C: np.ndarray | None     # M x N float32 / int32, or None when beta == 0
    notes: dict = field(default_factory=dict)


# name -> (M, N, K, a_type, b_type, alpha, beta, A recipe, B recipe, C recipe)
SPECS = {
    # fp16, A pre-sparsified at positions 0 and 2 of every group, U[-1,1].
    "tiny_f16": dict(M=64, N=64, K=128, a=F16, b=F16, alpha=1.0, beta=0.0, A="uniform_pos02", B="uniform", C=None),
    # fp16 4096^3, dense N(0,1) A pruned by magnitude, C ~ N(0,1), beta = 1.
    "f16_4096": dict(M=4096, N=4096, K=4096, a=F16, b=F16, alpha=1.0, beta=1.0, A="normal", B="normal", C="normal"),
    # bf16 LLM-linear shapes: weight 4096 x 4096 ~ N(0, 0.02^2), activations N(0,1).
    "bf16_linear_n16": dict(M=4096, N=16, K=4096, a=BF16, b=BF16, alpha=1.0, beta=0.0, A="normal_0.02", B="normal", C=None),
    "bf16_linear_n4096": dict(M=4096, N=4096, K=4096, a=BF16, b=BF16, alpha=1.0, beta=0.0, A="normal_0.02", B="normal", C=None),
    # int8 8192^3, A already 2:4 (random pattern per group), values nonzero uniform.
    "i8_8192": dict(M=8192, N=8192, K=8192, a=I8, b=I8, alpha=1.0, beta=0.0, A="i8_random24", B="i8_uniform", C=None),
    # fp8 E4M3 A x bf8 E5M2 B, and bf8 x bf8, M=N=8192, K=16384.
    "fp8_bf8_8192x16384": dict(M=8192, N=8192, K=16384, a=E4M3, b=E5M2, alpha=1.0, beta=0.0, A="normal", B="normal", C=None),
    "bf8_bf8_8192x16384": dict(M=8192, N=8192, K=16384, a=E5M2, b=E5M2, alpha=1.0, beta=0.0, A="normal", B="normal", C=None),
    # the headline: fp16 8192^3, dense N(0,1) A pruned by magnitude, beta = 0.
    "f16_8192": dict(M=8192, N=8192, K=8192, a=F16, b=F16, alpha=1.0, beta=0.0, A="normal", B="normal", C=None),
}


def make(name: str, seed: int = 0, M=None, N=None, K=None) -> Workload:
    """Build a named workload (optionally at another shape with the same recipe)."""
    sp = dict(SPECS[name])
    M = sp["M"] if M is None else M
    N = sp["N"] if N is None else N
    K = sp["K"] if K is None else K
    a, b = sp["a"], sp["b"]
    gA, gB, gC, gP = (_rng(seed, s) for s in range(4))
    notes = {}
    rA = sp["A"]
    if rA == "normal":
        A = _normal_bits(gA, (M, K), a)
    elif rA == "normal_0.02":
        A = _normal_bits(gA, (M, K), a, std=0.02)
    elif rA == "uniform_pos02":
        A = _uniform_bits(gA, (M, K), a, -1.0, 1.0)
        A.reshape(M, K // 4, 4)[:, :, 1] = 0
        A.reshape(M, K // 4, 4)[:, :, 3] = 0
        # a kept slot that rounded to +-0 is drawn again until it is nonzero
        kept = A.reshape(M, K // 4, 4)[:, :, 0::2]
        mag = 0x7FFF if ESIZE[a] == 2 else 0x7F
        while True:
            zero = (kept.astype(np.int64) & mag) == 0
            if not zero.any():
                break
            kept[zero] = quantize(gA.uniform(-1.0, 1.0, int(zero.sum())), a)
        A.reshape(M, K // 4, 4)[:, :, 0::2] = kept
        notes["fixed_pattern"] = (0, 2)
    elif rA == "i8_random24":
        pairs = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)], dtype=np.int64)
        pick = np.empty(M * (K // 4), dtype=np.int64)
        for s in range(0, pick.size, _CHUNK):
            e = min(pick.size, s + _CHUNK)
            pick[s:e] = gP.integers(0, 6, e - s)
        vals = _uniform_int8(gA, (M * (K // 4), 2), nonzero=True)
        A = np.zeros((M * (K // 4), 4), dtype=np.int8)
        rows = np.arange(M * (K // 4))
        A[rows, pairs[pick, 0]] = vals[:, 0]
        A[rows, pairs[pick, 1]] = vals[:, 1]
        A = A.reshape(M, K)
        notes["pattern_pick"] = pick.reshape(M, K // 4)
    else:
        raise ValueError(rA)
    rB = sp["B"]
    if rB == "normal":
        B = _normal_bits(gB, (K, N), b)
    elif rB == "uniform":
        B = _uniform_bits(gB, (K, N), b, -1.0, 1.0)
    elif rB == "i8_uniform":
        B = _uniform_int8(gB, (K, N))
    else:
        raise ValueError(rB)
    C = None
    if sp["C"] == "normal":
        C = gC.standard_normal((M, N)).astype(np.float32)
    return Workload(name, M, N, K, a, b, sp["alpha"], sp["beta"], A, B, C, notes)


def small_int_bits(shape, dtype: int, seed: int, lo: int = -1, hi: int = 1) -> np.ndarray:
    """Integers in [lo, hi] for tensors too large to draw element by element
    (billions of elements: fp64 normals would need tens of GB of host
    memory).  One seeded block of a prime length P = 1,000,003 is drawn and
    repeated over the row-major flat index, so element (i, j) is
    block[(i * cols + j) mod P]; P shares no factor with any tile size.
    Stored as `dtype`; exact in every format for the ranges the tests use.
    With |a|, |b| <= 1 every partial sum of a product is an integer below
    2^24 for K <= 2^25, so such products are exact in fp32."""
    shape = tuple(int(x) for x in shape)
    v = _rng(seed, 4).integers(lo, hi + 1, 1_000_003)
    if dtype == I8:
        bits = v.astype(np.int8)
    elif dtype == F16:
        bits = v.astype(np.float16).view(np.uint16)
    elif dtype == BF16:
        bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    else:
        bits = quantize(v.astype(np.float64), dtype)
    out = np.empty(shape, dtype=bits.dtype)
    flat = out.reshape(-1)
    for s in range(0, flat.size, bits.size):  # repeat the block over the flat index
        n = min(bits.size, flat.size - s)
        flat[s:s + n] = bits[:n]
    return out


def random_case(seed: int, M: int, N: int, K: int, a_type: int, b_type: int, beta: float = 0.0,
                alpha: float = 1.0, std: float = 1.0) -> Workload:
    """Seeded random dense-A case of an arbitrary shape (for parity sweeps)."""
    gA, gB, gC = (_rng(seed, s) for s in range(3))
    if a_type == I8:
        A = _uniform_int8(gA, (M, K))
    else:
        A = _normal_bits(gA, (M, K), a_type, std=std)
    if b_type == I8:
        B = _uniform_int8(gB, (K, N))
    else:
        B = _normal_bits(gB, (K, N), b_type)
    C = None
    if beta != 0.0:
        if a_type == I8:
            C = gC.integers(-(1 << 20), 1 << 20, (M, N)).astype(np.int32)
        else:
            C = gC.standard_normal((M, N)).astype(np.float32)
    return Workload(f"random_{M}x{N}x{K}", M, N, K, a_type, b_type, alpha, beta, A, B, C)
