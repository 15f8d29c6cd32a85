// Host side of the C ABI declared in include/sp24.h: argument checks,
// kernel selection and launch on the caller's stream.
#include <stdint.h>

#include "sp24_internal.hpp"

namespace sp24 {
hipError_t launch_prune_compress(const void* A, void* vals, uint32_t* meta, int64_t M, int64_t K, int dtype,
                                 int layout, hipStream_t stream);
hipError_t launch_gemm(int op, int layout, int b_layout, const void* A_vals, const uint32_t* meta, const void* B,
                       void* C, int M, int N, int K, float alpha, float beta, const float* bias, int out,
                       hipStream_t stream);
hipError_t launch_decompress(const void* vals, const uint32_t* meta, void* A, int64_t M, int64_t K, int dtype,
                             int layout, hipStream_t stream);
hipError_t launch_validate(const uint32_t* meta, int64_t M, int64_t K, int dtype, int layout, uint64_t* bad,
                           hipStream_t stream);
}  // namespace sp24

namespace {

int esize(int dtype) {
  switch (dtype) {
    case SP24_F16: case SP24_BF16: return 2;
    case SP24_I8: case SP24_FP8_E4M3: case SP24_BF8_E5M2: return 1;
    default: return 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) share a byte.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

using sp24::op_for;

constexpr int64_t kMaxDim = 0x7FFFFFFF;
constexpr uint64_t kTileBytesMax = 0x7FFFFF00ull;

bool layout_ok(int layout) { return layout == SP24_LAYOUT_ROW || layout == SP24_LAYOUT_KBLOCK; }

// K-blocks of the GEMM-ready layout: 64 dense columns (16-bit) or 128 (8-bit).
int64_t kblocks(int64_t K, int es) {
  const int64_t kb = es == 2 ? 64 : 128;
  return (K + kb - 1) / kb;
}

}  // namespace

extern "C" {

size_t sp24_values_bytes(int64_t M, int64_t K, int dtype, int layout) {
  const int es = esize(dtype);
  if (es == 0 || M < 0 || K < 0 || !layout_ok(layout)) return 0;
  if (layout == SP24_LAYOUT_KBLOCK) return (size_t)kblocks(K, es) * (size_t)M * 64u;
  return (size_t)M * (size_t)(K / 2) * (size_t)es;
}

size_t sp24_meta_bytes(int64_t M, int64_t K, int dtype, int layout) {
  const int es = esize(dtype);
  if (es == 0 || M < 0 || K < 0 || !layout_ok(layout)) return 0;
  if (layout == SP24_LAYOUT_KBLOCK) return (size_t)kblocks(K, es) * (size_t)((M + 127) / 128 * 128) * (es == 2 ? 8u : 16u);
  return (size_t)M * (size_t)(K / 32) * 4u;
}

size_t sp24_gemm_workspace_bytes(int64_t, int64_t, int64_t, int, int) { return 0; }

int sp24_prune_compress(const void* A, void* A_vals, uint32_t* meta, int64_t M, int64_t K, int dtype, int layout,
                        void* stream) {
  const int es = esize(dtype);
  if (es == 0 || !layout_ok(layout)) return SP24_ERR_UNSUPPORTED;
  if (M < 0 || K < 0 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return SP24_ERR_INVALID_VALUE;
  if (M == 0 || K == 0) return SP24_OK;
  if (!A || !A_vals || !meta) return SP24_ERR_INVALID_VALUE;
  if (!aligned16(A) || !aligned16(A_vals) || !aligned16(meta)) return SP24_ERR_MISALIGNED;
  const uint64_t a_bytes = (uint64_t)M * K * es;
  const uint64_t v_bytes = sp24_values_bytes(M, K, dtype, layout), m_bytes = sp24_meta_bytes(M, K, dtype, layout);
  if (overlap(A, a_bytes, A_vals, v_bytes) || overlap(A, a_bytes, meta, m_bytes) ||
      overlap(A_vals, v_bytes, meta, m_bytes))
    return SP24_ERR_INVALID_VALUE;
  const hipError_t e =
      sp24::launch_prune_compress(A, A_vals, meta, M, K, dtype, layout, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}

int sp24_gemm_ex(const void* A_vals, const uint32_t* meta, int a_type, int layout, const void* B, int b_type,
                 int b_layout, void* C, int c_type, const float* bias, int64_t M, int64_t N, int64_t K, float alpha,
                 float beta, void* workspace, size_t workspace_bytes, void* stream) {
  const int op = op_for(a_type, b_type);
  if (op < 0 || !layout_ok(layout) || (b_layout != SP24_B_KN && b_layout != SP24_B_NK)) return SP24_ERR_UNSUPPORTED;
  // output type: int32 for int8 inputs (no bias), fp32 / fp16 / bf16 otherwise
  int out;
  if (op == sp24::OP_I8) {
    if (c_type != SP24_I32 || bias) return SP24_ERR_UNSUPPORTED;
    out = sp24::OUT_32;
  } else if (c_type == SP24_F32) {
    out = sp24::OUT_32;
  } else if (c_type == SP24_F16) {
    out = sp24::OUT_F16;
  } else if (c_type == SP24_BF16) {
    out = sp24::OUT_BF16;
  } else {
    return SP24_ERR_UNSUPPORTED;
  }
  const int ec = out == sp24::OUT_32 ? 4 : 2;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return SP24_ERR_INVALID_VALUE;
  const int ea = esize(a_type), eb = esize(b_type);
  // N % 8: 16-byte rows of a 16-bit output and of 16-bit B.  8-bit B stored
  // K x N also needs 16-byte rows where the large-tile kernel (N > 64)
  // stages it; the small-N kernel loads each k-step's rows of B as one
  // contiguous run (128 * N bytes, a whole number of KiB).
  if (N % 8 != 0) return SP24_ERR_UNSUPPORTED;
  if (eb == 1 && b_layout == SP24_B_KN && N > 64 && N % 16 != 0) return SP24_ERR_UNSUPPORTED;
  // The kernels address one k-step of B (<= 128 rows) and, in the ROW layout,
  // the compressed rows of one 256-row tile with 32-bit offsets inside
  // buffer ranges below 2 GiB.
  if ((uint64_t)N * eb * 128 > kTileBytesMax) return SP24_ERR_UNSUPPORTED;
  if (layout == SP24_LAYOUT_ROW && (uint64_t)(K / 2) * ea * 256 > kTileBytesMax) return SP24_ERR_UNSUPPORTED;
  if (b_layout == SP24_B_NK && (uint64_t)K * eb * 256 > kTileBytesMax) return SP24_ERR_UNSUPPORTED;
  // one workgroup of 512 threads per 256 x 256 output tile, in one grid
  // dimension of fewer than 2^32 work-items (an output of over 2^39 elements)
  if (K > 0 && N > 64 && ((M + 255) / 256) * ((N + 255) / 256) >= (1ll << 23)) return SP24_ERR_UNSUPPORTED;
  if (op == sp24::OP_I8 && (alpha != 1.0f || (beta != 0.0f && beta != 1.0f))) return SP24_ERR_UNSUPPORTED;
  if (workspace_bytes < sp24_gemm_workspace_bytes(M, N, K, a_type, b_type)) return SP24_ERR_INVALID_VALUE;
  (void)workspace;
  if (M == 0 || N == 0) return SP24_OK;
  if (!C) return SP24_ERR_INVALID_VALUE;
  if (K > 0 && (!A_vals || !meta || !B)) return SP24_ERR_INVALID_VALUE;
  if (!aligned16(C) || (K > 0 && (!aligned16(A_vals) || !aligned16(meta) || !aligned16(B))) ||
      (bias && !aligned16(bias)))
    return SP24_ERR_MISALIGNED;
  const uint64_t c_bytes = (uint64_t)M * N * ec;
  if (K > 0 && (overlap(C, c_bytes, A_vals, sp24_values_bytes(M, K, a_type, layout)) ||
                overlap(C, c_bytes, meta, sp24_meta_bytes(M, K, a_type, layout)) ||
                overlap(C, c_bytes, B, (uint64_t)K * N * eb)))
    return SP24_ERR_INVALID_VALUE;
  if (bias && overlap(C, c_bytes, bias, (uint64_t)N * 4)) return SP24_ERR_INVALID_VALUE;
  const hipError_t e = sp24::launch_gemm(op, layout, b_layout, A_vals, meta, B, C, (int)M, (int)N, (int)K, alpha,
                                         beta, bias, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}

int sp24_gemm(const void* A_vals, const uint32_t* meta, int a_type, int layout, const void* B, int b_type,
              int b_layout, void* C, int64_t M, int64_t N, int64_t K, float alpha, float beta, void* workspace,
              size_t workspace_bytes, void* stream) {
  const int c_type = op_for(a_type, b_type) == sp24::OP_I8 ? SP24_I32 : SP24_F32;
  return sp24_gemm_ex(A_vals, meta, a_type, layout, B, b_type, b_layout, C, c_type, nullptr, M, N, K, alpha, beta,
                      workspace, workspace_bytes, stream);
}

int sp24_decompress(const void* A_vals, const uint32_t* meta, void* A, int64_t M, int64_t K, int dtype, int layout,
                    void* stream) {
  const int es = esize(dtype);
  if (es == 0 || !layout_ok(layout)) return SP24_ERR_UNSUPPORTED;
  if (M < 0 || K < 0 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return SP24_ERR_INVALID_VALUE;
  if (M == 0 || K == 0) return SP24_OK;
  if (!A || !A_vals || !meta) return SP24_ERR_INVALID_VALUE;
  if (!aligned16(A) || !aligned16(A_vals) || !aligned16(meta)) return SP24_ERR_MISALIGNED;
  const uint64_t a_bytes = (uint64_t)M * K * es;
  const uint64_t v_bytes = sp24_values_bytes(M, K, dtype, layout), m_bytes = sp24_meta_bytes(M, K, dtype, layout);
  if (overlap(A, a_bytes, A_vals, v_bytes) || overlap(A, a_bytes, meta, m_bytes)) return SP24_ERR_INVALID_VALUE;
  const hipError_t e = sp24::launch_decompress(A_vals, meta, A, M, K, dtype, layout, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}

int sp24_validate_meta(const uint32_t* meta, int64_t M, int64_t K, int dtype, int layout, uint64_t* bad_groups,
                       void* stream) {
  const int es = esize(dtype);
  if (es == 0 || !layout_ok(layout)) return SP24_ERR_UNSUPPORTED;
  if (M < 0 || K < 0 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return SP24_ERR_INVALID_VALUE;
  if (!bad_groups || (M > 0 && K > 0 && !meta)) return SP24_ERR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(bad_groups) & 7u) != 0 || (meta && !aligned16(meta))) return SP24_ERR_MISALIGNED;
  if (meta && overlap(bad_groups, 8, meta, sp24_meta_bytes(M, K, dtype, layout))) return SP24_ERR_INVALID_VALUE;
  const hipError_t e =
      sp24::launch_validate(meta, M, K, dtype, layout, bad_groups, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}

const char* sp24_status_string(int status) {
  switch (status) {
    case SP24_OK: return "SP24_OK";
    case SP24_ERR_INVALID_VALUE: return "SP24_ERR_INVALID_VALUE";
    case SP24_ERR_UNSUPPORTED: return "SP24_ERR_UNSUPPORTED";
    case SP24_ERR_MISALIGNED: return "SP24_ERR_MISALIGNED";
    case SP24_ERR_LAUNCH: return "SP24_ERR_LAUNCH";
    default: return "SP24_ERR_UNKNOWN";
  }
}

int sp24_version(void) { return 400; }

}  // extern "C"
