// Measurement aids, not steps of the 2:4 method:
//   sp24_calib_stream: a plain HBM stream (read, and copy a prefix of what
//     was read), the measured floor of the library's bandwidth-bound kernels
//     for the same bytes and launch shape;
//   sp24_calib_mfma / sp24_calib_mfma_ex: the product's sparse-MFMA
//     instruction stream with its operands held in registers, the measured
//     ceiling of the matrix cores on the workload's own operand values; also
//     with the product's direct-to-LDS loads issued between the
//     instructions, and with the 32x32 instruction shape.
#include "../../include/sp24_calib.h"
#include "sp24_internal.hpp"

namespace sp24 {

constexpr int kCalibUnroll = 4;

// Pieces are 16 bytes.  Each thread handles pieces base + u*stride_u for
// u < kCalibUnroll per iteration of a grid-stride loop, so the four loads of
// an iteration are in flight together and consecutive lanes read
// consecutive pieces.  Loads are non-temporal (the data is not reused),
// stores ordinary, as in the compress kernel.
__global__ void calib_stream_kernel(const i32x4* __restrict__ src, int64_t nread, i32x4* __restrict__ dst,
                                    int64_t nwrite, uint32_t* __restrict__ sink) {
  const int64_t stride_u = (int64_t)gridDim.x * blockDim.x;
  const int64_t step = stride_u * kCalibUnroll;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < nread; base += step) {
    i32x4 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const int64_t q = base + u * stride_u;
      v[u] = q < nread ? __builtin_nontemporal_load(src + q) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const int64_t q = base + u * stride_u;
      if (q < nwrite) dst[q] = v[u];
      acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
  }
  // one value per workgroup (a vector atomic xor; no scalar-cache stores)
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

// One pass: each thread loads kOnceUnroll pieces at a stride of the block
// size, all in flight together, then stores its share of the written prefix
// (the shape of the library's compress kernels).
constexpr int kOnceUnroll = 8;
__global__ void calib_stream_once_kernel(const i32x4* __restrict__ src, int64_t nread, i32x4* __restrict__ dst,
                                         int64_t nwrite, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * blockDim.x * kOnceUnroll + threadIdx.x;
  i32x4 v[kOnceUnroll];
#pragma unroll
  for (int u = 0; u < kOnceUnroll; ++u) {
    const int64_t q = base + (int64_t)u * blockDim.x;
    v[u] = q < nread ? __builtin_nontemporal_load(src + q) : i32x4{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kOnceUnroll; ++u) {
    const int64_t q = base + (int64_t)u * blockDim.x;
    if (q < nwrite) dst[q] = v[u];
    acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

// The product's matrix-core work with the memory side taken away.  Each
// wave holds one k-step's operands of a 128 x 64 wave tile (8 A fragments
// with their codes, 4 B fragments), loaded once, and then issues `rounds`
// times the instructions of a k-step in the product's order (each B
// fragment against the A fragments), into the wave tile's accumulators.
// Eight waves per workgroup, two per SIMD, as in the product; here both
// waves of a SIMD issue instructions all the time.
//   SHAPE 16: 32 instructions of 16x16 per round (the product's);
//   SHAPE 32: 16 instructions of 32x32 per round, the same operand
//             registers read as 32x32 fragments (4 row tiles x 2 column
//             tiles x 2 halves of the k-step), the same work per round.
//   LOADS:    after each of the first L of the round's 8 instruction groups
//             the wave issues one 1 KiB direct-to-LDS load in the product's
//             form (LDS base in M0 and a per-lane offset, both set for each
//             load), L = the product's loads per wave and k-step (7 for
//             16-bit types, 8 for 8-bit), from consecutive 1 KiB blocks of
//             the load source, into a 16 KiB ring of LDS per wave; one wait
//             per round leaves a round's loads in flight.  The loads write
//             only LDS, which nothing reads, so the accumulators do not
//             depend on them.
constexpr int kCalibWaves = 8;
constexpr uint64_t kCalibAUnit = 8 * 1024, kCalibBUnit = 4 * 2048, kCalibCUnit = 8 * 64 * 4;
constexpr int kCalibRing = 16384;  // LDS bytes per wave for the loads

typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One 32x32 sparse instruction: 16 bytes of compressed A and 32 bytes of B
// per lane, as smfmac16 (32x32x32 for 16-bit types, 32x32x64 for 8-bit).
template <int OP>
__device__ __forceinline__ i32x16 smfmac32(i32x16 acc, i32x4 a, i32x8 b, int idx) {
  if constexpr (OP == OP_I8) {
    return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, acc, idx, 0, 0);
  } else {
    f32x16 c = __builtin_bit_cast(f32x16, acc);
    if constexpr (OP == OP_F16)
      c = __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), c,
                                                     idx, 0, 0);
    else if constexpr (OP == OP_BF16)
      c = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, b), c,
                                                      idx, 0, 0);
    else if constexpr (OP == OP_FP8_FP8) c = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c, idx, 0, 0);
    else if constexpr (OP == OP_FP8_BF8) c = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_bf8(a, b, c, idx, 0, 0);
    else if constexpr (OP == OP_BF8_FP8) c = __builtin_amdgcn_smfmac_f32_32x32x64_bf8_fp8(a, b, c, idx, 0, 0);
    else c = __builtin_amdgcn_smfmac_f32_32x32x64_bf8_bf8(a, b, c, idx, 0, 0);
    return __builtin_bit_cast(i32x16, c);
  }
}

template <int OP, int SHAPE, bool LOADS>
__global__ __launch_bounds__(kCalibWaves * 64) void calib_mfma_kernel(const char* __restrict__ a, uint64_t na,
                                                                      const char* __restrict__ codes, uint64_t nc,
                                                                      const char* __restrict__ b, uint64_t nb,
                                                                      int rounds, const char* __restrict__ lsrc,
                                                                      uint32_t lmask, uint32_t* __restrict__ sink) {
  constexpr int L = op_esize(OP) == 2 ? 7 : 8;
  __shared__ __attribute__((aligned(1024))) char ring[LOADS ? kCalibWaves * kCalibRing : 16];
  const int l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint64_t gw = (uint64_t)blockIdx.x * kCalibWaves + w;  // this wave's fragment set
  const char* pa = a + (gw % na) * kCalibAUnit + 16 * l;
  const char* pc = codes + (gw % nc) * kCalibCUnit + 4 * l;
  const char* pb = b + (gw % nb) * kCalibBUnit + 32 * l;
  i32x4 fa[8];
  int idx[8];
  i32x8 fb[4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    fa[t] = *(const i32x4*)(pa + t * 1024);
    idx[t] = *(const int*)(pc + t * 256);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) fb[t] = *(const i32x8*)(pb + t * 2048);
  // The operands are in registers before the loop starts: the compiler's
  // own waits for these loads would otherwise sit inside the loop, where
  // they would also wait for the direct-to-LDS loads it does not see.
#pragma unroll
  for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(fa[t]), "+v"(idx[t]));
#pragma unroll
  for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(fb[t]));
  const i32x4 rs = make_rsrc4(lsrc, (uint64_t)lmask + 1);
  const uint32_t lbase = lds_addr((const SP24_LDS char*)ring) + (LOADS ? w * kCalibRing : 0);
  const uint32_t wstart = (uint32_t)(gw * 131u) * 1024u;
  auto load = [&](int r, int q) {
    if constexpr (LOADS) {
      const uint32_t j = (uint32_t)(r * L + q);
      dma16_asm(rs, lbase + (j & 15u) * 1024u, ((wstart + j * 1024u) & lmask) + 16u * (uint32_t)l, 0u);
    }
  };
  uint32_t x = 0;
  if constexpr (SHAPE == 16) {
    i32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int tm = 4 * (q & 1) + h, tn = q >> 1;
          acc[tm][tn] = smfmac16<OP>(acc[tm][tn], fa[tm], fb[tn], idx[tm]);
        }
        if constexpr (LOADS) {
          __builtin_amdgcn_sched_barrier(0);
          if (q < L) load(r, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (LOADS) {
        waitcnt<L>();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) x ^= (uint32_t)(acc[i][j][0] ^ acc[i][j][1] ^ acc[i][j][2] ^ acc[i][j][3]);
  } else {
    i32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tm = 2 * (q & 1) + h, ks = (q >> 1) & 1, tn = q >> 2;
          acc[tm][tn] = smfmac32<OP>(acc[tm][tn], fa[2 * tm + ks], fb[2 * tn + ks], idx[2 * tm + ks]);
        }
        if constexpr (LOADS) {
          __builtin_amdgcn_sched_barrier(0);
          if (q < L) load(r, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (LOADS) {
        waitcnt<L>();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) x ^= (uint32_t)acc[i][j][e];
  }
  if constexpr (LOADS) waitcnt<0>();
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if (l == 0) atomicXor(sink + blockIdx.x, x);
}

}  // namespace sp24

namespace {
template <int OP>
void launch_calib_mfma(int shape, bool loads, dim3 grid, dim3 block, hipStream_t st, const char* pa, uint64_t na,
                       const char* pc, uint64_t nc, const char* pb, uint64_t nb, int rounds, const char* ls,
                       uint32_t lmask, uint32_t* sink) {
  using namespace sp24;
  if (shape == 16 && !loads)
    hipLaunchKernelGGL((calib_mfma_kernel<OP, 16, false>), grid, block, 0, st, pa, na, pc, nc, pb, nb, rounds, ls, lmask,
                       sink);
  else if (shape == 16)
    hipLaunchKernelGGL((calib_mfma_kernel<OP, 16, true>), grid, block, 0, st, pa, na, pc, nc, pb, nb, rounds, ls, lmask,
                       sink);
  else if (!loads)
    hipLaunchKernelGGL((calib_mfma_kernel<OP, 32, false>), grid, block, 0, st, pa, na, pc, nc, pb, nb, rounds, ls, lmask,
                       sink);
  else
    hipLaunchKernelGGL((calib_mfma_kernel<OP, 32, true>), grid, block, 0, st, pa, na, pc, nc, pb, nb, rounds, ls, lmask,
                       sink);
}
}  // namespace

extern "C" int sp24_calib_mfma_ex(const void* a_vals, uint64_t a_bytes, const uint32_t* codes, uint64_t code_bytes,
                                  const void* b, uint64_t b_bytes, int a_type, int b_type, int rounds,
                                  int workgroups, int shape, const void* load_src, uint64_t load_src_bytes,
                                  uint32_t* sink, void* stream) {
  const int op = sp24::op_for(a_type, b_type);
  if (op < 0) return SP24_ERR_UNSUPPORTED;
  if (!a_vals || !codes || !b || !sink || rounds < 1 || workgroups < 1) return SP24_ERR_INVALID_VALUE;
  if (shape != 16 && shape != 32) return SP24_ERR_INVALID_VALUE;
  const bool loads = load_src != nullptr;
  if (loads && load_src_bytes < 1024) return SP24_ERR_INVALID_VALUE;
  const uint64_t na = a_bytes / sp24::kCalibAUnit, nc = code_bytes / sp24::kCalibCUnit,
                 nb = b_bytes / sp24::kCalibBUnit;
  if (na == 0 || nc == 0 || nb == 0) return SP24_ERR_INVALID_VALUE;
  if (((uintptr_t)a_vals | (uintptr_t)codes | (uintptr_t)b | (uintptr_t)load_src) & 15u) return SP24_ERR_MISALIGNED;
  // the largest power of two <= load_src_bytes, at most 1 GiB (a 32-bit mask)
  uint64_t span = 1024;
  while (loads && span * 2 <= load_src_bytes && span < (1ull << 30)) span *= 2;
  const uint32_t lmask = loads ? (uint32_t)(span - 1) : 0u;
  const char* pa = static_cast<const char*>(a_vals);
  const char* pc = reinterpret_cast<const char*>(codes);
  const char* pb = static_cast<const char*>(b);
  const char* ls = loads ? static_cast<const char*>(load_src) : pb;
  const dim3 grid((unsigned)workgroups), block(sp24::kCalibWaves * 64);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (op) {
#define SP24_CALIB_CASE(O)                                                                                  \
  case sp24::O:                                                                                             \
    launch_calib_mfma<sp24::O>(shape, loads, grid, block, st, pa, na, pc, nc, pb, nb, rounds, ls, lmask, sink); \
    break;
    SP24_CALIB_CASE(OP_F16)
    SP24_CALIB_CASE(OP_BF16)
    SP24_CALIB_CASE(OP_I8)
    SP24_CALIB_CASE(OP_FP8_FP8)
    SP24_CALIB_CASE(OP_FP8_BF8)
    SP24_CALIB_CASE(OP_BF8_FP8)
    SP24_CALIB_CASE(OP_BF8_BF8)
#undef SP24_CALIB_CASE
    default: return SP24_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}

extern "C" int sp24_calib_mfma(const void* a_vals, uint64_t a_bytes, const uint32_t* codes, uint64_t code_bytes,
                               const void* b, uint64_t b_bytes, int a_type, int b_type, int rounds, int workgroups,
                               uint32_t* sink, void* stream) {
  return sp24_calib_mfma_ex(a_vals, a_bytes, codes, code_bytes, b, b_bytes, a_type, b_type, rounds, workgroups, 16,
                            nullptr, 0, sink, stream);
}

extern "C" int sp24_calib_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                                 uint32_t* sink, int workgroups, int threads, void* stream) {
  if (!src || !sink || (write_bytes && !dst) || write_bytes > read_bytes) return SP24_ERR_INVALID_VALUE;
  if ((read_bytes | write_bytes) & 15u) return SP24_ERR_INVALID_VALUE;
  if (workgroups < 0 || threads < 64 || threads > 1024 || threads % 64) return SP24_ERR_INVALID_VALUE;
  if (((uintptr_t)src | (uintptr_t)dst) & 15u) return SP24_ERR_MISALIGNED;
  if (read_bytes == 0) return SP24_OK;
  const int64_t pieces = (int64_t)(read_bytes / 16);
  if (workgroups == 0) {
    const int64_t grid = (pieces + (int64_t)threads * sp24::kOnceUnroll - 1) / ((int64_t)threads * sp24::kOnceUnroll);
    if (grid > 0x7FFFFFFFll) return SP24_ERR_INVALID_VALUE;
    hipLaunchKernelGGL(sp24::calib_stream_once_kernel, dim3((unsigned)grid), dim3((unsigned)threads), 0,
                       (hipStream_t)stream, static_cast<const sp24::i32x4*>(src), pieces,
                       static_cast<sp24::i32x4*>(dst), (int64_t)(write_bytes / 16), sink);
  } else {
    hipLaunchKernelGGL(sp24::calib_stream_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), 0,
                       (hipStream_t)stream, static_cast<const sp24::i32x4*>(src), pieces,
                       static_cast<sp24::i32x4*>(dst), (int64_t)(write_bytes / 16), sink);
  }
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}
