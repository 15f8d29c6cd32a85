// Internal helpers shared by the libsp24 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sp24.h"

namespace sp24 {

#define SP24_LDS __attribute__((address_space(3)))

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Sparse-MFMA operation, one per supported (A type, B type) pair.
enum Op { OP_F16 = 0, OP_BF16, OP_I8, OP_FP8_FP8, OP_FP8_BF8, OP_BF8_FP8, OP_BF8_BF8, OP_COUNT };

__host__ __device__ constexpr bool op_is_8bit(int op) { return op >= OP_I8; }
__host__ __device__ constexpr bool op_is_int(int op) { return op == OP_I8; }
// Dense K consumed by one 16x16 sparse instruction: 64 for 16-bit inputs, 128 for 8-bit.
__host__ __device__ constexpr int op_kstep(int op) { return op_is_8bit(op) ? 128 : 64; }
__host__ __device__ constexpr int op_esize(int op) { return op_is_8bit(op) ? 1 : 2; }

// Sparse-MFMA operation for an (A, B) element-type pair, or -1.
inline int op_for(int a, int b) {
  if (a == SP24_F16 && b == SP24_F16) return OP_F16;
  if (a == SP24_BF16 && b == SP24_BF16) return OP_BF16;
  if (a == SP24_I8 && b == SP24_I8) return OP_I8;
  if (a == SP24_FP8_E4M3 && b == SP24_FP8_E4M3) return OP_FP8_FP8;
  if (a == SP24_FP8_E4M3 && b == SP24_BF8_E5M2) return OP_FP8_BF8;
  if (a == SP24_BF8_E5M2 && b == SP24_FP8_E4M3) return OP_BF8_FP8;
  if (a == SP24_BF8_E5M2 && b == SP24_BF8_E5M2) return OP_BF8_BF8;
  return -1;
}

// One 16x16 sparse MFMA step.  Per lane: `a` = 16 bytes of compressed A
// (8 values for 16-bit types, 16 for 8-bit), `b` = 32 bytes of dense B,
// `idx` = this lane's 2-bit position codes (bits 2e.. for its element e; for
// 16-bit types ABID picks the 16-bit half of idx).  Accumulator is 4 x fp32
// (or int32 for int8) in the 16x16 layout lane = 16*(i/4) + j, reg = i%4.
template <int OP, int ABID = 0>
__device__ __forceinline__ i32x4 smfmac16(i32x4 acc, i32x4 a, i32x8 b, int idx) {
  if constexpr (OP == OP_F16) {
    f32x4 c = __builtin_bit_cast(f32x4, acc);
    c = __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), c,
                                                   idx, 0, ABID);
    return __builtin_bit_cast(i32x4, c);
  } else if constexpr (OP == OP_BF16) {
    f32x4 c = __builtin_bit_cast(f32x4, acc);
    c = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, b), c,
                                                    idx, 0, ABID);
    return __builtin_bit_cast(i32x4, c);
  } else if constexpr (OP == OP_I8) {
    return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc, idx, 0, 0);
  } else {
    f32x4 c = __builtin_bit_cast(f32x4, acc);
    if constexpr (OP == OP_FP8_FP8) c = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c, idx, 0, 0);
    else if constexpr (OP == OP_FP8_BF8) c = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_bf8(a, b, c, idx, 0, 0);
    else if constexpr (OP == OP_BF8_FP8) c = __builtin_amdgcn_smfmac_f32_16x16x128_bf8_fp8(a, b, c, idx, 0, 0);
    else c = __builtin_amdgcn_smfmac_f32_16x16x128_bf8_bf8(a, b, c, idx, 0, 0);
    return __builtin_bit_cast(i32x4, c);
  }
}

// A dispatch counts its work-items in 32 bits per grid dimension, so a grid
// of 512-thread workgroups must stay below 2^23 of them.  Kernels whose
// workgroup count grows with the problem are launched in pieces of at most
// this many workgroups; each piece passes the index of its first workgroup.
static constexpr uint32_t kMaxLaunchWorkgroups = 1u << 18;

// ---- buffer resources: raw byte-addressed, hardware range-checked ----------
// Reads at offsets >= num_records return zeros, which is how ragged edges and
// the K tail are handled without branches.
#define SP24_RSRC_WORD3 0x00020000
static constexpr uint32_t kOOB = 0x7FFFFFF0u;          // offset used for masked lanes
static constexpr uint64_t kMaxRecords = 0x7FFFFF00ull;  // keep every range below kOOB

// Direct-to-LDS buffer loads, issued through inline assembly.  The compiler
// then does not see an LDS write, so it inserts no waits of its own for them
// (with the compiler-visible builtin, its alias tracking for these loads was
// lost across branches and the loop back-edge, which made it wait for every
// freshly issued load); callers wait with explicit s_waitcnt vmcnt and order
// LDS reads with barriers that carry a memory clobber.  The buffer resource
// is a plain SGPR quad; the LDS address is m0 + the lane's 16 (or 4) bytes.
__device__ __forceinline__ i32x4 make_rsrc4(const void* base, uint64_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t n = (uint32_t)(bytes < kMaxRecords ? bytes : kMaxRecords);
  return i32x4{(int)(uint32_t)b, (int)((b >> 32) & 0xFFFFu), (int)n, SP24_RSRC_WORD3};
}
__device__ __forceinline__ uint32_t lds_addr(const SP24_LDS void* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ void dma16_asm(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds));
}
__device__ __forceinline__ void dma4_asm(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds));
}

// s_waitcnt with only vmcnt (and lgkmcnt) constrained (gfx9 encoding).
template <int VM, int LGKM = 15>
__device__ __forceinline__ void waitcnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Epilogue of the product: D = round_out(alpha * acc + beta * C + bias[col]).
// OUT_32 writes float32 (int32 for int8 inputs, where only beta in {0, 1}
// and no bias are allowed); OUT_F16 / OUT_BF16 round the fp32 sum once, to
// nearest even, and C is read in the same 16-bit type.
enum OutType { OUT_32 = 0, OUT_F16 = 1, OUT_BF16 = 2 };
struct Epilogue {
  float alpha, beta;
  const float* bias;  // N values or nullptr
  int out;            // OutType
};

// The product's output stores (CACHED is a compile-time choice: with a
// run-time one the compiler merges the two stores of the same value and
// keeps the ordinary one).  Streaming by default: while other tiles are still
// reading A and B, letting the output allocate in the caches evicts them.
// When every tile runs at once nothing is read after the epilogues, and
// ordinary stores let the caches absorb the burst of all outputs.
template <bool CACHED, typename T>
__device__ __forceinline__ void put(T v, T* p) {
  if constexpr (CACHED) *p = v;
  else __builtin_nontemporal_store(v, p);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Four consecutive outputs of one row at element offset o, column col
// (col % 4 == 0, all four inside N).  v = the fp32 accumulators.
template <bool INT, bool CACHED>
__device__ __forceinline__ void store_out4(void* C, int64_t o, int col, f32x4 v, const Epilogue& ep) {
  if constexpr (INT) {
    i32x4 d = __builtin_bit_cast(i32x4, v);
    if (ep.beta != 0.0f) d += __builtin_nontemporal_load((const i32x4*)((const int*)C + o));
    put<CACHED>(d, (i32x4*)((int*)C + o));
  } else {
    f32x4 d = v * ep.alpha;
    if (ep.out == OUT_32) {
      if (ep.beta != 0.0f) d += ep.beta * __builtin_nontemporal_load((const f32x4*)((const float*)C + o));
      if (ep.bias) d += *(const f32x4*)(ep.bias + col);
      put<CACHED>(d, (f32x4*)((float*)C + o));
    } else if (ep.out == OUT_F16) {
      f16x4* p = (f16x4*)((_Float16*)C + o);
      if (ep.beta != 0.0f) d += ep.beta * __builtin_convertvector(__builtin_nontemporal_load(p), f32x4);
      if (ep.bias) d += *(const f32x4*)(ep.bias + col);
      put<CACHED>(__builtin_convertvector(d, f16x4), p);
    } else {
      bf16x4* p = (bf16x4*)((__bf16*)C + o);
      if (ep.beta != 0.0f) d += ep.beta * __builtin_convertvector(__builtin_nontemporal_load(p), f32x4);
      if (ep.bias) d += *(const f32x4*)(ep.bias + col);
      put<CACHED>(__builtin_convertvector(d, bf16x4), p);
    }
  }
}

// store_out4 for a 32-bit output with beta != 0, with the four C values
// (their bits) already read: the same arithmetic.
template <bool INT, bool CACHED>
__device__ __forceinline__ void store_out4_c(void* C, int64_t o, int col, f32x4 v, i32x4 c, const Epilogue& ep) {
  if constexpr (INT) {
    put<CACHED>(__builtin_bit_cast(i32x4, v) + c, (i32x4*)((int*)C + o));
  } else {
    f32x4 d = v * ep.alpha;
    d += ep.beta * __builtin_bit_cast(f32x4, c);
    if (ep.bias) d += *(const f32x4*)(ep.bias + col);
    put<CACHED>(d, (f32x4*)((float*)C + o));
  }
}

// store_out4 for a 16-bit output (BF: bfloat16, else fp16) with beta != 0,
// with the four C values (their bits) already read: the same arithmetic.
template <bool BF, bool CACHED>
__device__ __forceinline__ void store_out4_c16(void* C, int64_t o, int col, f32x4 v, i32x2 c, const Epilogue& ep) {
  f32x4 d = v * ep.alpha;
  if constexpr (BF) {
    d += ep.beta * __builtin_convertvector(__builtin_bit_cast(bf16x4, c), f32x4);
    if (ep.bias) d += *(const f32x4*)(ep.bias + col);
    put<CACHED>(__builtin_convertvector(d, bf16x4), (bf16x4*)((__bf16*)C + o));
  } else {
    d += ep.beta * __builtin_convertvector(__builtin_bit_cast(f16x4, c), f32x4);
    if (ep.bias) d += *(const f32x4*)(ep.bias + col);
    put<CACHED>(__builtin_convertvector(d, f16x4), (f16x4*)((_Float16*)C + o));
  }
}

// One output element (same arithmetic as store_out4).
template <bool INT>
__device__ __forceinline__ void store_out1(void* C, int64_t o, int col, float v, const Epilogue& ep) {
  if constexpr (INT) {
    int d = __float_as_int(v);
    int* p = (int*)C + o;
    *p = ep.beta != 0.0f ? d + *p : d;
  } else {
    float d = v * ep.alpha;
    if (ep.out == OUT_32) {
      float* p = (float*)C + o;
      if (ep.beta != 0.0f) d += ep.beta * *p;
      if (ep.bias) d += ep.bias[col];
      *p = d;
    } else if (ep.out == OUT_F16) {
      _Float16* p = (_Float16*)C + o;
      if (ep.beta != 0.0f) d += ep.beta * (float)*p;
      if (ep.bias) d += ep.bias[col];
      *p = (_Float16)d;
    } else {
      __bf16* p = (__bf16*)C + o;
      if (ep.beta != 0.0f) d += ep.beta * (float)*p;
      if (ep.bias) d += ep.bias[col];
      *p = (__bf16)d;
    }
  }
}

}  // namespace sp24
