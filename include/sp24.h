/*
 * sp24.h -- C ABI of libsp24: 2:4 structured-sparse compression and
 * sparse x dense multiply-accumulate on AMD Instinct MI355X (gfx950).
 *
 * The operation (sources: "CDNA and CDNA2 sparse MFMA builtins", sections
 * "Structured sparsity (4:2 pattern)" and the builtin reference; "RDNA4
 * sparse WMMA builtins", section "Structured sparsity (2:4 pattern)"; the ISA
 * page for v_smfmac_f32_32x32x32_bf8_bf8, section "Semantics"):
 *
 *   A (M x K) keeps 2 of every 4 consecutive elements along K.  It is stored
 *   as A_vals (M x K/2, the kept values in ascending position order) plus a
 *   2-bit position code per kept value (the sparsity index).  The product is
 *   D = alpha * expand(A_vals, meta) * B + beta * C, accumulated in fp32
 *   (int32 for int8).
 *
 * Dense layouts (row-major, dense leading dimensions, no padding):
 *   A       M x K elements of the input type, K contiguous.
 *   B       SP24_B_KN: K x N elements, N contiguous (the default);
 *           SP24_B_NK: stored as N x K elements, K contiguous (B transposed,
 *           e.g. the activations of a linear layer).  K is the dense K.
 *   C / D   M x N float32 (int32 when both inputs are int8), updated in place.
 *
 * Compressed layouts (sp24_layout).  In both, the 2-bit code (0..3, position
 * inside its group of 4) of compressed element c of a row sits at bits
 * [2*(c%16), 2*(c%16)+1] of that row's metadata word c/16 (LSB first; with
 * the positions-0-and-2 pattern every byte reads 0x88, the index value the
 * pages' CDNA examples pass to the instruction).
 *   SP24_LAYOUT_ROW     A_vals is M x K/2 elements, row-major; meta is
 *                       M x K/32 uint32 words, row-major.  The reference
 *                       layout.
 *   SP24_LAYOUT_KBLOCK  GEMM-ready: K is cut into blocks of KB dense columns
 *                       (KB = 64 for 16-bit types, 128 for 8-bit types; each
 *                       block is 64 bytes of compressed values per row), and
 *                       block b of all rows is stored together.  ceil(K/KB)
 *                       blocks; the tail of a last partial block is zero.
 *                       Values: bytes [(b*M + i)*64, +64) = row i, block b.
 *                       Metadata: per block, Mp = M rounded up to 128 rows,
 *                       MB = KB/8 bytes per row (8 or 16), block b at bytes
 *                       [b*Mp*MB, +Mp*MB), rows past M zero.  A row's codes
 *                       for the block are 4 words c_0..c_3 (16 bits each for
 *                       16-bit types, 32 bits for 8-bit types; word g holds
 *                       the codes of the row's compressed elements
 *                       KB/8*g .. in the order above).  Inside block b, the
 *                       words of the 128 rows 128p+16t+r (t < 8, r < 16) are
 *                       stored, from byte (b*Mp + 128p)*MB on,
 *                         16-bit: u16 index ((r*4 + g)*4 + t/2)*2 + t%2,
 *                         8-bit:  u32 index  (r*4 + g)*8 + t,
 *                       so the 8 words one matrix-core lane needs for the 8
 *                       row tiles of a 128-row group are contiguous.  One
 *                       k-step of a 256-row tile is then a single contiguous
 *                       16 KiB run of values and 2 or 4 KiB of metadata.
 *
 * Element types (sp24_dtype): fp16 (IEEE binary16), bf16, int8 (two's
 * complement), fp8 E4M3 and bf8 E5M2 (both OCP: E4M3 has no infinities and
 * a largest finite value of 448).  Supported (a_type, b_type) pairs for
 * sp24_gemm: (F16,F16), (BF16,BF16), (I8,I8), and any pair of the two 8-bit
 * float types.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *     every buffer.  The library keeps no state between calls and allocates
 *     no memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls only enqueue kernels on it (no memset, no copy, no host
 *     synchronisation), so they may be captured into a HIP graph.  A kernel
 *     fault shows up at the caller's next synchronisation.
 *   - Argument errors are detected on the host, before anything is
 *     launched, and returned as an sp24_status code; nothing is enqueued.
 *   - Calls are thread-safe.
 */
#ifndef SP24_H
#define SP24_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SP24_F16 = 1,
  SP24_BF16 = 2,
  SP24_I8 = 3,
  SP24_FP8_E4M3 = 4,
  SP24_BF8_E5M2 = 5,
  SP24_F32 = 6, /* output (C / D) type only */
  SP24_I32 = 7  /* output (C / D) type only */
} sp24_dtype;

typedef enum {
  SP24_LAYOUT_ROW = 0,
  SP24_LAYOUT_KBLOCK = 1
} sp24_layout;

typedef enum {
  SP24_B_KN = 0,
  SP24_B_NK = 1
} sp24_b_layout;

typedef enum {
  SP24_OK = 0,
  SP24_ERR_INVALID_VALUE = 1, /* bad shape, null pointer, overlap, workspace too small */
  SP24_ERR_UNSUPPORTED = 2,   /* type pair, alpha/beta or leading dimension not supported */
  SP24_ERR_MISALIGNED = 3,    /* a base pointer is not 16-byte aligned */
  SP24_ERR_LAUNCH = 4         /* the HIP runtime refused the kernel launch */
} sp24_status;

/* Bytes of A_vals for an M x K matrix of `dtype` in `layout`:
 * ROW: M * (K/2) * element size; KBLOCK: ceil(K/KB) * M * 64.
 * Returns 0 for an unknown dtype or layout or negative sizes. */
size_t sp24_values_bytes(int64_t M, int64_t K, int dtype, int layout);

/* Bytes of the metadata: ROW: M * (K/32) * 4; KBLOCK: ceil(K/KB) * Mp * KB/8
 * with Mp = M rounded up to a multiple of 128. */
size_t sp24_meta_bytes(int64_t M, int64_t K, int dtype, int layout);

/* Workspace that sp24_gemm needs for this problem (currently always 0: the
 * kernels reduce split-K partial sums on chip). */
size_t sp24_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int a_type, int b_type);

/*
 * sp24_prune_compress -- dense A -> (A_vals, meta).
 *
 * Prunes every group of 4 consecutive K-elements of each row to its two
 * largest-magnitude elements and compresses the result: the two kept values
 * of each group are stored one after the other and their positions become
 * the group's codes ("CDNA and CDNA2 sparse MFMA builtins", section
 * "Structured sparsity (4:2 pattern)").  Which two to keep is not fixed by
 * the pages, which leave pruning to an offline pass.  Magnitude is compared on the bit
 * pattern with the sign cleared (float types; NaN ranks above Inf, -0 equals
 * +0) or |x| (int8, -128 ranks highest); on equal magnitude the lower
 * position wins.  Kept values are copied bit for bit.  An A that is already
 * 2:4 is therefore compressed losslessly.
 *
 *   A       in:  M x K elements of `dtype`.
 *   A_vals  out: sp24_values_bytes(M, K, dtype, layout) bytes.
 *   meta    out: sp24_meta_bytes(M, K, dtype, layout) bytes.
 *   M, K    0 <= M, K <= 2^31 - 1, K % 32 == 0.  M == 0 or K == 0 enqueues
 *           nothing.
 *   layout  SP24_LAYOUT_ROW or SP24_LAYOUT_KBLOCK.
 * Errors: INVALID_VALUE (shape, null pointer with nonzero size, A overlapping
 * an output), UNSUPPORTED (unknown dtype or layout), MISALIGNED (pointer not
 * 16-byte aligned), LAUNCH.
 */
int sp24_prune_compress(const void* A, void* A_vals, uint32_t* meta, int64_t M, int64_t K, int dtype, int layout,
                        void* stream);

/*
 * sp24_gemm -- D = alpha * expand(A_vals, meta) * B + beta * C, D written
 * over C.
 *
 * The hardware form is the sparse matrix-core instruction: each compressed A
 * value is multiplied with the row of B its position code selects, and the
 * products accumulate into D ("CDNA and CDNA2 sparse MFMA builtins", section
 * "Structured sparsity (4:2 pattern)"; the ISA page for
 * v_smfmac_f32_32x32x32_bf8_bf8, section "Semantics").  Accumulation is
 * fp32 (exact int32 for int8).  Measured behaviour of the matrix units on
 * gfx950, which the parity tests pin:
 *   - every single product of two fp16, bf16, fp8 or bf8 values (subnormals
 *     included) is formed exactly and rounded to fp32 once; overflow gives
 *     +-Inf, NaN inputs give NaN;
 *   - fp32 results below 2^-126 (reachable from bf16 inputs only) land on
 *     the denormal grid within one step (2^-149) of the exact value;
 *   - for 8-bit float inputs, the products of each aligned run of 8
 *     compressed elements (16 dense columns) are summed on a grid set by
 *     the largest of them: with e the binary exponent of that largest
 *     |product|, bits below 2^(e-13) are dropped.  On the N(0,1)-like data
 *     of the configured workloads the product stays within
 *     1e-4 * sum|a*b| + 1e-6 of the exact value; inputs whose products in
 *     one run differ by 2^14 or more in magnitude can exceed that by up to
 *     7 * 2^-13 of the run's largest product.  16-bit inputs meet the
 *     1e-4 bound on any finite inputs whose exact sums stay in fp32 range.
 *
 *   A_vals, meta  compressed A in `layout`, as produced by
 *                 sp24_prune_compress (or any caller-built data in the same
 *                 layout; codes are trusted -- a group whose two codes are
 *                 not strictly increasing gives unspecified results).
 *   a_type        element type of A_vals; b_type element type of B.
 *   B             K x N elements of b_type (SP24_B_KN) or its transpose,
 *                 N x K (SP24_B_NK), as `b_layout` says.
 *   C             in/out: M x N float32 (int32 for int8 x int8).  Not read
 *                 when beta == 0 (NaN there does not propagate).
 *   M, N, K       0 <= M, N, K <= 2^31 - 1, K % 32 == 0, N % 8 == 0 (and,
 *                 for 8-bit B stored K x N with N > 64, N % 16 == 0),
 *                 N * sizeof(b_type) <= 16 MiB - 2 (so 128 rows of B stay
 *                 below 2 GiB), for SP24_B_NK 256 * K * sizeof(b_type) <
 *                 2 GiB and, for the ROW layout, 256 * K/2 * sizeof(a_type)
 *                 < 2 GiB (K <= 8388606 for 16-bit types); for K > 0 and
 *                 N > 64, fewer than 2^23 output tiles of 256 x 256
 *                 (always so for an output that fits in device memory).
 *                 M == 0 or N == 0: nothing is enqueued.  K == 0: D = beta*C.
 *   alpha, beta   float scalars.  For int8: alpha must be 1, beta 0 or 1.
 *   workspace     may be NULL when sp24_gemm_workspace_bytes() == 0.
 * Errors: INVALID_VALUE (shape, null pointer, C overlapping an input,
 * workspace too small), UNSUPPORTED (type pair, int8 alpha/beta, N not a
 * multiple of 8 (of 16 for 8-bit B stored K x N with N > 64), N or K past
 * the limits above, unknown layout or b_layout), MISALIGNED, LAUNCH.
 */
int sp24_gemm(const void* A_vals, const uint32_t* meta, int a_type, int layout, const void* B, int b_type,
              int b_layout, void* C, int64_t M, int64_t N, int64_t K, float alpha, float beta, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * sp24_gemm_ex -- sp24_gemm with a choice of output type and a bias:
 *   D[i][j] = round_c_type(alpha * (expand(A_vals, meta) * B)[i][j]
 *                          + beta * C[i][j] + bias[j]),
 * D written over C.  The product accumulates in fp32 (exact int32 for int8)
 * exactly as in sp24_gemm; the sum with beta*C and the bias is formed in
 * fp32 and rounded once, to nearest even, into c_type.  (The pages' RDNA4
 * builtins accumulate into FP16 or BF16 directly ("RDNA4 sparse WMMA
 * builtins", sections "FP16-accumulate builtins" and "BF16-accumulate
 * builtins"); the CDNA sparse instructions accumulate in FP32 only, so a
 * 16-bit result is produced here by one rounding at the end.  The bias is
 * the linear-layer epilogue this library adds.)
 *
 *   c_type   SP24_F32, SP24_F16 or SP24_BF16 for floating inputs;
 *            SP24_I32 for int8 x int8.  C and D are M x N elements of c_type.
 *            C (when beta != 0) is read in c_type and widened to fp32.
 *   bias     NULL, or N float32 values (device pointer, 16-byte aligned)
 *            added to every row.  Floating inputs only.
 *   Everything else as for sp24_gemm; sp24_gemm(...) is sp24_gemm_ex with
 *   c_type = SP24_F32 (SP24_I32 for int8) and bias = NULL.
 * Errors: as sp24_gemm, plus UNSUPPORTED (c_type not allowed for the input
 * types, a bias with int8 inputs), MISALIGNED (bias), INVALID_VALUE (C
 * overlapping the bias).
 */
int sp24_gemm_ex(const void* A_vals, const uint32_t* meta, int a_type, int layout, const void* B, int b_type,
                 int b_layout, void* C, int c_type, const float* bias, int64_t M, int64_t N, int64_t K, float alpha,
                 float beta, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sp24_decompress -- (A_vals, meta) -> dense A, the inverse of compression:
 * in every group of 4 the two stored values go to the positions their codes
 * name and the other two elements become +0 (all-zero bits) ("CDNA and CDNA2
 * sparse MFMA builtins", section "Structured sparsity (4:2 pattern)").  If
 * both codes of a group name one position (metadata compression never
 * produces), the group's second value is left there.
 *
 *   A_vals, meta  in: compressed A in `layout` (sizes as for
 *                 sp24_prune_compress).
 *   A             out: M x K elements of `dtype`, row-major.
 *   M, K          as for sp24_prune_compress.
 * Errors: INVALID_VALUE (shape, null pointer, A overlapping an input),
 * UNSUPPORTED (dtype or layout), MISALIGNED, LAUNCH.
 */
int sp24_decompress(const void* A_vals, const uint32_t* meta, void* A, int64_t M, int64_t K, int dtype, int layout,
                    void* stream);

/*
 * sp24_validate_meta -- counts the groups whose two codes are not strictly
 * increasing (p0 >= p1).  sp24_prune_compress never produces such groups;
 * sp24_gemm gives unspecified results for them, so callers that build
 * metadata themselves can check it here first.  Only the M rows and the K
 * columns are examined (not the K-blocked padding).
 *
 *   meta        in: metadata of an M x K matrix of `dtype` in `layout`.
 *   bad_groups  out: DEVICE pointer to one uint64 (8-byte aligned), set to
 *               the count when the stream reaches this call (the library
 *               clears it with a kernel of its own, no memset).
 * Errors: INVALID_VALUE (shape, null pointer, overlap), UNSUPPORTED,
 * MISALIGNED (meta not 16-byte or bad_groups not 8-byte aligned), LAUNCH.
 */
int sp24_validate_meta(const uint32_t* meta, int64_t M, int64_t K, int dtype, int layout, uint64_t* bad_groups,
                       void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* sp24_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int sp24_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SP24_H */
