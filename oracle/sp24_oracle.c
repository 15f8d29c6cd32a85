/*
 * sp24_oracle.c -- plain, slow, CPU reference for 2:4 structured sparsity.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test-suite, the smoke check and the CPU leg of
 * the benchmark load it.  It shares no source with the GPU path.
 *
 * What it computes, and where that is defined:
 *   - 2:4 structured sparsity: in every run of 4 consecutive K-elements of A,
 *     2 are kept and 2 are zero ("CDNA and CDNA2 sparse MFMA builtins",
 *     section "Structured sparsity (4:2 pattern)"; "RDNA4 sparse WMMA
 *     builtins", section "Structured sparsity (2:4 pattern)").
 *   - Compression: walk K in groups of 4 and store the kept values one after
 *     the other, halving K; a 2-bit position code per kept value is the
 *     sparsity index (same sections).  Codes are packed LSB-first; with the
 *     positions-0-and-2 pattern one byte covering two groups reads 0x88, the
 *     index value the CDNA example kernels pass (section "Using sparse MFMA
 *     builtins as a compute policy").
 *   - Product: D = alpha * expand(A_vals, index) * B + beta * C, where the
 *     index aligns each compressed A value with its row of B (section
 *     "Structured sparsity"; the ISA page for v_smfmac_f32_32x32x32_bf8_bf8,
 *     section "Semantics": D = A(sparse) * B + D).
 *   - Output rounding (the library's 16-bit output option): the exact fp64
 *     result is rounded once to the nearest fp16 / bf16 value, ties to even.
 *     The pages' RDNA4 builtins accumulate into FP16 / BF16 ("RDNA4 sparse
 *     WMMA builtins", sections "FP16-accumulate builtins" and
 *     "BF16-accumulate builtins"); the CDNA sparse instructions accumulate in
 *     FP32 only, so the library rounds the fp32 result at the end instead.
 *   - The pruning rule (keep the two largest magnitudes, ties to the lower
 *     position) is not fixed by the pages, which only say weights are pruned
 *     offline ("RDNA4 sparse WMMA builtins", section "Instruction
 *     throughput" note); it is the reading used throughout this library.
 *
 * Arithmetic: every floating value is decoded exactly into double from its
 * bit pattern (formats written out below from their definitions), products
 * and sums are taken in double; int8 work is done in int64.  No SIMD, no
 * BLAS, no blocking.
 *
 * Element type codes (same numbers as the library's public enum, restated
 * here so that this file depends on nothing else):
 *   1 = fp16 (IEEE binary16), 2 = bf16, 3 = int8, 4 = fp8 E4M3 (OCP "FN"),
 *   5 = bf8 E5M2 (OCP).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F16 1
#define ORC_BF16 2
#define ORC_I8 3
#define ORC_E4M3 4
#define ORC_E5M2 5

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_OVERFLOW 2

int orc_elem_size(int dtype) {
  switch (dtype) {
    case ORC_F16: case ORC_BF16: return 2;
    case ORC_I8: case ORC_E4M3: case ORC_E5M2: return 1;
    default: return 0;
  }
}

/* Generic binary float decode: sign | exponent (ebits) | mantissa (mbits).
 * IEEE-style: exponent 0 -> subnormal, all-ones exponent -> Inf/NaN unless
 * the format has no infinities (E4M3FN: only S.1111.111 is NaN). */
static double decode_float(uint32_t bits, int ebits, int mbits, int has_inf) {
  const uint32_t sign = (bits >> (ebits + mbits)) & 1u;
  const uint32_t e = (bits >> mbits) & ((1u << ebits) - 1u);
  const uint32_t m = bits & ((1u << mbits) - 1u);
  const int bias = (1 << (ebits - 1)) - 1;
  const uint32_t emax = (1u << ebits) - 1u;
  double v;
  if (has_inf && e == emax) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (!has_inf && e == emax && m == (1u << mbits) - 1u) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, 1 - bias - mbits);
  } else {
    v = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
  }
  return sign ? -v : v;
}

/* Exact value of one stored element (bits in the low bits of `bits`). */
double orc_decode(uint32_t bits, int dtype) {
  switch (dtype) {
    case ORC_F16: return decode_float(bits & 0xFFFFu, 5, 10, 1);
    case ORC_BF16: return decode_float(bits & 0xFFFFu, 8, 7, 1);
    case ORC_E4M3: return decode_float(bits & 0xFFu, 4, 3, 0);
    case ORC_E5M2: return decode_float(bits & 0xFFu, 5, 2, 1);
    case ORC_I8: return (double)(int8_t)(bits & 0xFFu);
    default: return NAN;
  }
}

/* Magnitude key used to rank the 4 elements of a group.  For the float
 * formats the bit pattern with the sign cleared is monotone in |x| (NaN sorts
 * above Inf, -0 equals +0); for int8 it is |x| (so -128 ranks highest). */
/* Nearest fp16 (dtype 1) or bf16 (dtype 2) bit pattern to x, ties to even
 * (the IEEE default rounding), written from the formats' definitions:
 * fp16 = 1 sign, 5 exponent (bias 15), 10 fraction bits; bf16 = 1, 8 (bias
 * 127), 7.  Values of magnitude at or beyond the point halfway between the
 * largest finite value and the next power of two become Inf; NaN becomes
 * the quiet NaN with the sign of x and the top fraction bit set. */
uint32_t orc_round_to(double x, int dtype) {
  int ebits, mbits;
  if (dtype == ORC_F16) { ebits = 5; mbits = 10; }
  else if (dtype == ORC_BF16) { ebits = 8; mbits = 7; }
  else return 0;
  const int bias = (1 << (ebits - 1)) - 1, emin = 1 - bias, emax = bias;
  const uint32_t sign = signbit(x) ? 1u << (ebits + mbits) : 0u;
  const uint32_t inf = ((1u << ebits) - 1u) << mbits;
  if (isnan(x)) return sign | inf | (1u << (mbits - 1));
  double a = fabs(x);
  if (isinf(a)) return sign | inf;
  if (a == 0.0) return sign;
  /* quantum: spacing of representable values in the binade of a (the
   * subnormal spacing below the smallest normal) */
  int e;
  frexp(a, &e);  /* a = f * 2^e, 0.5 <= f < 1, so floor(log2 a) = e - 1 */
  int qe = (e - 1 < emin ? emin : e - 1) - mbits;
  double y = ldexp(a, -qe);  /* exact: a power-of-two scaling */
  double f = floor(y), d = y - f;
  if (d > 0.5 || (d == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
  double r = ldexp(f, qe);   /* the rounded magnitude, exact */
  const double maxfin = ldexp(2.0 - ldexp(1.0, -mbits), emax);
  if (r > maxfin) return sign | inf;
  if (r < ldexp(1.0, emin)) /* subnormal (or zero): field 0, fraction r / 2^(emin - mbits) */
    return sign | (uint32_t)ldexp(r, mbits - emin);
  frexp(r, &e);
  const int ex = e - 1;
  const uint32_t frac = (uint32_t)(ldexp(r, mbits - ex) - ldexp(1.0, mbits));
  return sign | ((uint32_t)(ex + bias) << mbits) | frac;
}

uint32_t orc_key(uint32_t bits, int dtype) {
  switch (dtype) {
    case ORC_F16: case ORC_BF16: return bits & 0x7FFFu;
    case ORC_E4M3: case ORC_E5M2: return bits & 0x7Fu;
    case ORC_I8: { int v = (int8_t)(bits & 0xFFu); return (uint32_t)(v < 0 ? -v : v); }
    default: return 0;
  }
}

static uint32_t load_elem(const void* base, int64_t idx, int esz) {
  if (esz == 2) return ((const uint16_t*)base)[idx];
  return ((const uint8_t*)base)[idx];
}
static void store_elem(void* base, int64_t idx, int esz, uint32_t v) {
  if (esz == 2) ((uint16_t*)base)[idx] = (uint16_t)v;
  else ((uint8_t*)base)[idx] = (uint8_t)v;
}

/* Choose the 2 kept positions of one group of 4: order the positions by
 * (key descending, position ascending) and keep the first two; return them
 * as p0 < p1. */
static void choose_two(const uint32_t key[4], int* p0, int* p1) {
  int order[4] = {0, 1, 2, 3};
  /* insertion sort, stable on position for equal keys */
  for (int a = 1; a < 4; ++a) {
    int cur = order[a];
    int b = a - 1;
    while (b >= 0 && key[order[b]] < key[cur]) {
      order[b + 1] = order[b];
      --b;
    }
    order[b + 1] = cur;
  }
  int x = order[0], y = order[1];
  *p0 = x < y ? x : y;
  *p1 = x < y ? y : x;
}

/* Prune dense A (M x K, row-major, K contiguous) to 2:4 and compress it.
 *   vals: M x K/2 elements of the same type: vals[i][2g] = A[i][4g+p0],
 *         vals[i][2g+1] = A[i][4g+p1] (bits copied verbatim).
 *   meta: M x K/32 uint32 words; the 2-bit code (position 0..3 inside the
 *         group) of compressed element c of row i sits at bits
 *         [2*(c%16), 2*(c%16)+1] of meta[i][c/16].
 * K must be a multiple of 32. */
int orc_prune_compress(const void* A, void* vals, uint32_t* meta, int64_t M, int64_t K, int dtype) {
  const int esz = orc_elem_size(dtype);
  if (esz == 0 || M < 0 || K < 0 || K % 32 != 0) return ORC_BAD_ARG;
  const int64_t KC = K / 2, KW = K / 32;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t w = 0; w < KW; ++w) meta[i * KW + w] = 0u;
    for (int64_t g = 0; g < K / 4; ++g) {
      uint32_t bits[4], key[4];
      for (int p = 0; p < 4; ++p) {
        bits[p] = load_elem(A, i * K + 4 * g + p, esz);
        key[p] = orc_key(bits[p], dtype);
      }
      int p0, p1;
      choose_two(key, &p0, &p1);
      const int64_t c0 = 2 * g, c1 = 2 * g + 1;
      store_elem(vals, i * KC + c0, esz, bits[p0]);
      store_elem(vals, i * KC + c1, esz, bits[p1]);
      meta[i * KW + c0 / 16] |= (uint32_t)p0 << (2 * (c0 % 16));
      meta[i * KW + c1 / 16] |= (uint32_t)p1 << (2 * (c1 % 16));
    }
  }
  return ORC_OK;
}

/* Code (0..3) of compressed element c of row i. */
static int code_of(const uint32_t* meta, int64_t KW, int64_t i, int64_t c) {
  return (int)((meta[i * KW + c / 16] >> (2 * (c % 16))) & 3u);
}

/* Expand compressed A back to dense M x K: the slots named by the codes get
 * the stored bits, all other slots hold +0 (all-zero bits).  If both codes of
 * a group name the same slot, the second value written wins. */
int orc_decompress(const void* vals, const uint32_t* meta, void* A, int64_t M, int64_t K, int dtype) {
  const int esz = orc_elem_size(dtype);
  if (esz == 0 || M < 0 || K < 0 || K % 32 != 0) return ORC_BAD_ARG;
  const int64_t KC = K / 2, KW = K / 32;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t k = 0; k < K; ++k) store_elem(A, i * K + k, esz, 0u);
    for (int64_t c = 0; c < KC; ++c) {
      const int64_t k = 4 * (c / 2) + code_of(meta, KW, i, c);
      store_elem(A, i * K + k, esz, load_elem(vals, i * KC + c, esz));
    }
  }
  return ORC_OK;
}

/* Number of groups whose two codes are not strictly increasing (p0 >= p1):
 * metadata that compression never produces and that the product's hardware
 * form leaves undefined.  Plain count over rows and groups. */
int64_t orc_count_invalid(const uint32_t* meta, int64_t M, int64_t K) {
  if (M < 0 || K < 0 || K % 32 != 0) return -1;
  const int64_t KW = K / 32;
  int64_t bad = 0;
  for (int64_t i = 0; i < M; ++i)
    for (int64_t g = 0; g < K / 4; ++g)
      if (code_of(meta, KW, i, 2 * g) >= code_of(meta, KW, i, 2 * g + 1)) ++bad;
  return bad;
}

static double* decode_table(int dtype) {
  const int esz = orc_elem_size(dtype);
  const int n = esz == 2 ? 65536 : 256;
  double* t = (double*)malloc(sizeof(double) * (size_t)n);
  if (!t) return NULL;
  for (int b = 0; b < n; ++b) t[b] = orc_decode((uint32_t)b, dtype);
  return t;
}

/* Floating-point sparse product, straight from the compressed form:
 *   acc[i][j] = sum_c dec(vals[i][c]) * dec(B[4*(c/2) + code(i,c)][j])
 *   D[i][j]   = alpha * acc[i][j] + beta * C[i][j] + bias[j]
 * (C not read if beta == 0; no bias term if bias is NULL).
 * B is K x N row-major (N contiguous); C is M x N, given as float32 values
 * (a 16-bit C is passed widened, which is exact); D is M x N double.
 * If absD is not NULL it receives |alpha| * sum_c |a * b| + |beta * C| +
 * |bias|, the scale used by the error bound of the comparison. */
int orc_gemm_f64(const void* vals, const uint32_t* meta, int a_type, const void* B, int b_type,
                 const float* C, const float* bias, double* D, double* absD, int64_t M, int64_t N, int64_t K,
                 double alpha, double beta) {
  const int ea = orc_elem_size(a_type), eb = orc_elem_size(b_type);
  if (ea == 0 || eb == 0 || a_type == ORC_I8 || b_type == ORC_I8) return ORC_BAD_ARG;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return ORC_BAD_ARG;
  const int64_t KC = K / 2, KW = K / 32;
  double* ta = decode_table(a_type);
  double* tb = decode_table(b_type);
  double* acc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double* aacc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  if (!ta || !tb || !acc || !aacc) { free(ta); free(tb); free(acc); free(aacc); return ORC_BAD_ARG; }
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) { acc[j] = 0.0; aacc[j] = 0.0; }
    for (int64_t c = 0; c < KC; ++c) {
      const double a = ta[load_elem(vals, i * KC + c, ea)];
      const int64_t k = 4 * (c / 2) + code_of(meta, KW, i, c);
      for (int64_t j = 0; j < N; ++j) {
        const double p = a * tb[load_elem(B, k * N + j, eb)];
        acc[j] += p;
        aacc[j] += fabs(p);
      }
    }
    for (int64_t j = 0; j < N; ++j) {
      double d = alpha * acc[j];
      double s = fabs(alpha) * aacc[j];
      if (beta != 0.0) {
        const double cv = (double)C[i * N + j];
        d += beta * cv;
        s += fabs(beta * cv);
      }
      if (bias) {
        d += (double)bias[j];
        s += fabs((double)bias[j]);
      }
      D[i * N + j] = d;
      if (absD) absD[i * N + j] = s;
    }
  }
  free(ta); free(tb); free(acc); free(aacc);
  return ORC_OK;
}

/* int8 sparse product, exact in int64:
 *   D[i][j] = sum_c vals[i][c] * B[4*(c/2) + code(i,c)][j]  (+ C[i][j] if beta_one)
 * Returns ORC_OVERFLOW (after filling D) if any result leaves int32 range. */
int orc_gemm_i64(const int8_t* vals, const uint32_t* meta, const int8_t* B, const int32_t* C,
                 int64_t* D, int64_t M, int64_t N, int64_t K, int beta_one) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return ORC_BAD_ARG;
  const int64_t KC = K / 2, KW = K / 32;
  int rc = ORC_OK;
  int64_t* acc = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
  if (!acc) return ORC_BAD_ARG;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) acc[j] = 0;
    for (int64_t c = 0; c < KC; ++c) {
      const int64_t a = vals[i * KC + c];
      const int64_t k = 4 * (c / 2) + code_of(meta, KW, i, c);
      for (int64_t j = 0; j < N; ++j) acc[j] += a * (int64_t)B[k * N + j];
    }
    for (int64_t j = 0; j < N; ++j) {
      int64_t d = acc[j] + (beta_one ? (int64_t)C[i * N + j] : 0);
      if (d > INT32_MAX || d < INT32_MIN) rc = ORC_OVERFLOW;
      D[i * N + j] = d;
    }
  }
  free(acc);
  return rc;
}

/* The same products at chosen output points only (for spot checks at sizes
 * where the full product takes too long on the CPU).  Points (ii[p], jj[p]). */
int orc_gemm_points_f64(const void* vals, const uint32_t* meta, int a_type, const void* B, int b_type,
                        const float* C, int64_t M, int64_t N, int64_t K, double alpha, double beta,
                        int64_t npts, const int64_t* ii, const int64_t* jj, double* out, double* absout) {
  const int ea = orc_elem_size(a_type), eb = orc_elem_size(b_type);
  if (ea == 0 || eb == 0 || a_type == ORC_I8 || b_type == ORC_I8) return ORC_BAD_ARG;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return ORC_BAD_ARG;
  const int64_t KC = K / 2, KW = K / 32;
  for (int64_t p = 0; p < npts; ++p) {
    const int64_t i = ii[p], j = jj[p];
    if (i < 0 || i >= M || j < 0 || j >= N) return ORC_BAD_ARG;
    double acc = 0.0, aacc = 0.0;
    for (int64_t c = 0; c < KC; ++c) {
      const double a = orc_decode(load_elem(vals, i * KC + c, ea), a_type);
      const int64_t k = 4 * (c / 2) + code_of(meta, KW, i, c);
      const double prod = a * orc_decode(load_elem(B, k * N + j, eb), b_type);
      acc += prod;
      aacc += fabs(prod);
    }
    double d = alpha * acc, s = fabs(alpha) * aacc;
    if (beta != 0.0) {
      const double cv = (double)C[i * N + j];
      d += beta * cv;
      s += fabs(beta * cv);
    }
    out[p] = d;
    if (absout) absout[p] = s;
  }
  return ORC_OK;
}

int orc_gemm_points_i64(const int8_t* vals, const uint32_t* meta, const int8_t* B, const int32_t* C,
                        int64_t M, int64_t N, int64_t K, int beta_one, int64_t npts, const int64_t* ii,
                        const int64_t* jj, int64_t* out) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return ORC_BAD_ARG;
  const int64_t KC = K / 2, KW = K / 32;
  int rc = ORC_OK;
  for (int64_t p = 0; p < npts; ++p) {
    const int64_t i = ii[p], j = jj[p];
    if (i < 0 || i >= M || j < 0 || j >= N) return ORC_BAD_ARG;
    int64_t acc = 0;
    for (int64_t c = 0; c < KC; ++c) {
      const int64_t k = 4 * (c / 2) + code_of(meta, KW, i, c);
      acc += (int64_t)vals[i * KC + c] * (int64_t)B[k * N + j];
    }
    if (beta_one) acc += C[i * N + j];
    if (acc > INT32_MAX || acc < INT32_MIN) rc = ORC_OVERFLOW;
    out[p] = acc;
  }
  return rc;
}
