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

}  // namespace sp24

extern "C" int sp24_calib_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                                 uint32_t* sink, int workgroups, int threads, void* stream) {
  if (!src || !sink || (write_bytes && !dst) || write_bytes > read_bytes) return SP24_ERR_INVALID_VALUE;
  if ((read_bytes | write_bytes) & 15u) return SP24_ERR_INVALID_VALUE;
  if (workgroups < 1 || threads < 64 || threads > 1024 || threads % 64) return SP24_ERR_INVALID_VALUE;
  if (((uintptr_t)src | (uintptr_t)dst) & 15u) return SP24_ERR_MISALIGNED;
  if (read_bytes == 0) return SP24_OK;
  hipLaunchKernelGGL(sp24::calib_stream_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), 0,
                     (hipStream_t)stream, static_cast<const sp24::i32x4*>(src), (int64_t)(read_bytes / 16),
                     static_cast<sp24::i32x4*>(dst), (int64_t)(write_bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH;
}
