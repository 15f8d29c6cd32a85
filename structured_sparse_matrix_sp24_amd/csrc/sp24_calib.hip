// sp24_calib_stream: a plain HBM stream (read, and copy a prefix of what was
// read), used by the benchmark as the measured floor of the library's
// bandwidth-bound kernels for the same bytes and launch shape.  Not part of
// the 2:4 method.
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

}  // namespace sp24

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
