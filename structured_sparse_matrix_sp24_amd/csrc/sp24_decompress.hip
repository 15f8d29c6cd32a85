// sp24_decompress / sp24_validate_meta: the inverse of compression and a
// check of compressed metadata, both bound by HBM bandwidth (no MFMA, no LDS).
//
// Decompression restores the dense row from its kept values and their 2-bit
// positions: each group of four gets its two values at the positions its
// codes name, the other two elements are +0 ("CDNA and CDNA2 sparse MFMA
// builtins", section "Structured sparsity (4:2 pattern)").  Codes that name
// the same position twice (never produced by compression) leave the second
// value there.
//
// Validation counts the groups whose two codes are not strictly increasing:
// compression never produces them, and the matrix-core product leaves them
// undefined, so a caller can check metadata built by other means.
#include "sp24_internal.hpp"

namespace sp24 {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;
constexpr int kDecKbThreads = 512;  // K-blocked kernel

// One group of four 16-bit values from its two kept values and 4-bit code
// (p0 in bits 0-1, p1 in bits 2-3); the second value wins a shared slot.
__device__ __forceinline__ uint64_t expand16(uint32_t pair, uint32_t nib) {
  const uint32_t p0 = nib & 3u, p1 = (nib >> 2) & 3u;
  uint64_t w = (uint64_t)(pair & 0xFFFFu) << (16 * p0);
  w &= ~(0xFFFFull << (16 * p1));
  return w | ((uint64_t)(pair >> 16) << (16 * p1));
}
// The same for four 8-bit values.
__device__ __forceinline__ uint32_t expand8(uint32_t pair, uint32_t nib) {
  const uint32_t p0 = nib & 3u, p1 = (nib >> 2) & 3u;
  uint32_t w = (pair & 0xFFu) << (8 * p0);
  w &= ~(0xFFu << (8 * p1));
  return w | (((pair >> 8) & 0xFFu) << (8 * p1));
}

// 8 bytes of values + the chunk's codes -> one 16-byte chunk of dense A.
template <int ES>
__device__ __forceinline__ i32x4 expand_chunk(i32x2 v, uint32_t code) {
  i32x4 out;
  if constexpr (ES == 2) {
    const uint64_t g0 = expand16((uint32_t)v[0], code & 0xFu);
    const uint64_t g1 = expand16((uint32_t)v[1], (code >> 4) & 0xFu);
    out = i32x4{(int)(uint32_t)g0, (int)(uint32_t)(g0 >> 32), (int)(uint32_t)g1, (int)(uint32_t)(g1 >> 32)};
  } else {
    out = i32x4{(int)expand8((uint32_t)v[0] & 0xFFFFu, code & 0xFu),
                (int)expand8((uint32_t)v[0] >> 16, (code >> 4) & 0xFu),
                (int)expand8((uint32_t)v[1] & 0xFFFFu, (code >> 8) & 0xFu),
                (int)expand8((uint32_t)v[1] >> 16, (code >> 12) & 0xFu)};
  }
  return out;
}

// Row-major layout: chunk q of A (16 bytes) <- 8 bytes of values at q and the
// codes at metadata byte q (16-bit) or bytes 2q, 2q+1 (8-bit), independent of
// M and K because K % 32 == 0.
template <int ES>
__global__ __launch_bounds__(kDecThreads) void decompress_row_kernel(const i32x2* __restrict__ vals,
                                                                       const uint8_t* __restrict__ meta,
                                                                       i32x4* __restrict__ A, int64_t nchunks) {
  const int64_t base = (int64_t)blockIdx.x * (kDecThreads * kDecUnroll) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kDecUnroll; ++u) {
    const int64_t q = base + (int64_t)u * kDecThreads;
    if (q >= nchunks) break;
    const i32x2 v = __builtin_nontemporal_load(vals + q);
    const uint32_t code = ES == 2 ? (uint32_t)meta[q] : (uint32_t)reinterpret_cast<const uint16_t*>(meta)[q];
    __builtin_nontemporal_store(expand_chunk<ES>(v, code), A + q);
  }
}

// K-blocked layout: workgroup (row tile rt, block group) of T threads covers
// rows rt*128 .. +128 of NB consecutive blocks; thread t handles chunk
// t % (8*NB) of rows rt*128 + t/(8*NB) + (T/(8*NB))*u, with one base address
// per thread advanced by a uniform stride per round; the codes are read from
// their interleaved position in the row's 128-row group.  (An earlier form
// that recomputed each round's 64-bit addresses from the row index gave
// different outputs from run to run on 8192 x 8192 inputs while passing on
// small ones; this form gave the same, oracle-exact output in every run.)
template <int ES, int NB, int T>
__global__ __launch_bounds__(T) void decompress_kblock_kernel(const char* __restrict__ vals,
                                                               const char* __restrict__ meta,
                                                               char* __restrict__ A, int64_t M, int64_t K,
                                                               uint32_t nblk, uint32_t wg0) {
  constexpr int MB = ES == 2 ? 8 : 16, CE = 16 / ES;
  constexpr int CPR = 8 * NB, RPR = T / CPR, NR = 128 / RPR;
  const uint32_t nwb = (nblk + NB - 1) / NB;
  const uint32_t g = wg0 + blockIdx.x;  // workgroup index over all pieces of the launch
  const int64_t b = (int64_t)(g % nwb) * NB + (threadIdx.x % CPR) / 8;
  const uint32_t rt = g / nwb;
  const int64_t Mp = (M + 127) / 128 * 128;
  const int c = threadIdx.x & 7;
  const int64_t kcol = b * (8 * CE) + (int64_t)c * CE;
  if (kcol >= K) return;
  const char* mgroup = meta + (b * Mp + (int64_t)rt * 128) * MB;
  const int64_t row0 = (int64_t)rt * 128;
  const int rows_here = (int)min<int64_t>(M - row0, 128);
  const int r_first = threadIdx.x / CPR;
  const char* src = vals + (b * M + row0 + r_first) * 64 + c * 8;
  char* dst = A + (row0 + r_first) * K * ES + kcol * ES;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int rr = r_first + RPR * u;
    if (rr >= rows_here) break;
    const int t = rr >> 4, r = rr & 15;
    const i32x2 v = __builtin_nontemporal_load(reinterpret_cast<const i32x2*>(src + RPR * 64 * u));
    uint32_t code;
    if constexpr (ES == 2)
      code = *reinterpret_cast<const uint8_t*>(mgroup + (((r * 4 + c / 2) * 4 + t / 2) * 2 + (t & 1)) * 2 + (c & 1));
    else
      code = *reinterpret_cast<const uint16_t*>(mgroup + ((r * 4 + c / 2) * 8 + t) * 4 + (c & 1) * 2);
    __builtin_nontemporal_store(expand_chunk<ES>(v, code),
                                reinterpret_cast<i32x4*>(dst + (int64_t)(RPR * u) * K * ES));
  }
}

// ---- validation ---------------------------------------------------------------
// Groups of a 32-bit code word (eight 4-bit codes p0 | p1 << 2) whose codes
// are not strictly increasing (p0 >= p1), among those whose nibbles `mask`
// covers; all eight at once.  Per nibble, (p0 | 4) - p1 lies in
// 1..7, so nothing borrows across nibbles, and its bit 2 is set exactly when
// p0 >= p1.
__device__ __forceinline__ int bad_groups_masked(uint32_t w, uint32_t mask) {
  const uint32_t d = ((w & 0x33333333u) | 0x44444444u) - ((w >> 2) & 0x33333333u);
  return __builtin_popcount(d & 0x44444444u & mask);
}

// Sum over the wave, then one 64-bit vector atomic per wave.
__device__ __forceinline__ void add_wave_count(int n, unsigned long long* out) {
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
  if (lane_id() == 0 && n != 0) atomicAdd(out, (unsigned long long)n);
}

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }

// Row-major layout: four 32-bit words (32 groups) per thread and load,
// grid-stride; the last nwords % 4 words one by one.
__global__ __launch_bounds__(256) void validate_row_kernel(const uint32_t* __restrict__ meta, int64_t nwords,
                                                            unsigned long long* out) {
  int bad = 0;
  const int64_t nq = nwords / 4, stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t q = t0; q < nq; q += stride) {
    const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(meta) + q);
#pragma unroll
    for (int e = 0; e < 4; ++e) bad += bad_groups_masked((uint32_t)v[e], 0xFFFFFFFFu);
  }
  for (int64_t q = 4 * nq + t0; q < nwords; q += stride) bad += bad_groups_masked(meta[q], 0xFFFFFFFFu);
  add_wave_count(bad, out);
}

// K-blocked layout: one 16-byte piece of one block's metadata per thread and
// load (block b over grid y, pieces over grid x, both grid-stride).  In a
// 128-row group, code word x (16-bit units for 16-bit types, 32-bit for 8-bit
// ones) belongs to row 16t + r and word g of the row's block, with t = x & 7,
// g = (x >> 3) & 3, r = (x >> 5) & 15, so a piece holds 8 (or 4) consecutive
// t of one (g, r).  Only groups inside K of rows below M are counted (the
// tail of a partial last block and the padding rows hold zero codes).
template <int ES>
__global__ __launch_bounds__(256) void validate_kblock_kernel(const char* __restrict__ meta, int64_t M, int64_t K,
                                                               int64_t nblk, unsigned long long* out) {
  constexpr int MB = ES == 2 ? 8 : 16, KB = ES == 2 ? 64 : 128, GPW = KB / 16;  // groups per word
  constexpr int WPP = ES == 2 ? 8 : 4;                                             // words per 16-byte piece
  constexpr int PPG = 128 * MB / 16;                                               // pieces per 128-row group
  const int64_t Mp = (M + 127) / 128 * 128;
  const int64_t ppb = Mp * MB / 16;                                                // pieces per block
  int bad = 0;
  for (int64_t b = blockIdx.y; b < nblk; b += gridDim.y) {
    const i32x4* blk = reinterpret_cast<const i32x4*>(meta + b * Mp * MB);
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < ppb; c += (int64_t)gridDim.x * blockDim.x) {
      const i32x4 v = __builtin_nontemporal_load(blk + c);
      const int x0 = (int)(c % PPG) * WPP;             // first word of the piece in its group
      const int64_t row0 = (c / PPG) * 128 + (x0 >> 5 & 15);  // row of t = 0
      const int g = (x0 >> 3) & 3, t0 = x0 & 7;
      const int64_t inside = (K - (b * KB + (int64_t)g * (KB / 4))) / 4;  // groups of word g inside K
      const int ng = inside >= GPW ? GPW : (inside > 0 ? (int)inside : 0);
      const uint32_t wmask = ng == 8 ? 0xFFFFFFFFu : (1u << (4 * ng)) - 1u;  // nibbles of one word inside K
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // one 32-bit element: two 16-bit words (rows t, t+1) or one 32-bit word
        uint32_t mask;
        if constexpr (ES == 2)
          mask = (row0 + 16 * (t0 + 2 * e) < M ? wmask : 0u) | (row0 + 16 * (t0 + 2 * e + 1) < M ? wmask << 16 : 0u);
        else
          mask = row0 + 16 * (t0 + e) < M ? wmask : 0u;
        bad += bad_groups_masked((uint32_t)v[e], mask);
      }
    }
  }
  add_wave_count(bad, out);
}

// ---- host launchers (arguments already validated) ------------------------------
hipError_t launch_decompress(const void* vals, const uint32_t* meta, void* A, int64_t M, int64_t K, int dtype,
                             int layout, hipStream_t stream) {
  const int es = (dtype == SP24_F16 || dtype == SP24_BF16) ? 2 : 1;
  if (M == 0 || K == 0) return hipSuccess;
  const dim3 block(kDecThreads);
  if (layout == SP24_LAYOUT_KBLOCK) {
    const int64_t kb = es == 2 ? 64 : 128;
    const int64_t nblk = (K + kb - 1) / kb, row_tiles = (M + 127) / 128;
    // 16-bit types: two blocks (256 contiguous bytes of a dense row) per
    // workgroup while that leaves at least 1024 workgroups; 512 threads
    const int nb = es == 2 && row_tiles * ((nblk + 1) / 2) >= 1024 ? 2 : 1;
    const int64_t nwb = (nblk + nb - 1) / nb;
    const int64_t total = row_tiles * nwb;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const dim3 blk(kDecKbThreads);
    const char* v = static_cast<const char*>(vals);
    const char* m = reinterpret_cast<const char*>(meta);
    char* a = static_cast<char*>(A);
    const uint32_t n = (uint32_t)nblk;
    for (int64_t first = 0; first < total; first += kMaxLaunchWorkgroups) {
      const dim3 grid((unsigned)(total - first < kMaxLaunchWorkgroups ? total - first : kMaxLaunchWorkgroups));
      const uint32_t g0 = (uint32_t)first;
      if (es == 2 && nb == 2)
        hipLaunchKernelGGL((decompress_kblock_kernel<2, 2, kDecKbThreads>), grid, blk, 0, stream, v, m, a, M, K, n,
                           g0);
      else if (es == 2)
        hipLaunchKernelGGL((decompress_kblock_kernel<2, 1, kDecKbThreads>), grid, blk, 0, stream, v, m, a, M, K, n,
                           g0);
      else
        hipLaunchKernelGGL((decompress_kblock_kernel<1, 1, kDecKbThreads>), grid, blk, 0, stream, v, m, a, M, K, n,
                           g0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int64_t nchunks = M * K * es / 16;
  const int64_t blocks = (nchunks + kDecThreads * kDecUnroll - 1) / (kDecThreads * kDecUnroll);
  if (blocks * kDecThreads > 0xFFFFFFFFll) return hipErrorInvalidValue;  // A > 256 GiB
  const i32x2* v = static_cast<const i32x2*>(vals);
  const uint8_t* m = reinterpret_cast<const uint8_t*>(meta);
  i32x4* a = static_cast<i32x4*>(A);
  if (es == 2) hipLaunchKernelGGL((decompress_row_kernel<2>), dim3((unsigned)blocks), block, 0, stream, v, m, a, nchunks);
  else hipLaunchKernelGGL((decompress_row_kernel<1>), dim3((unsigned)blocks), block, 0, stream, v, m, a, nchunks);
  return hipGetLastError();
}

hipError_t launch_validate(const uint32_t* meta, int64_t M, int64_t K, int dtype, int layout, uint64_t* bad,
                           hipStream_t stream) {
  const int es = (dtype == SP24_F16 || dtype == SP24_BF16) ? 2 : 1;
  unsigned long long* out = reinterpret_cast<unsigned long long*>(bad);
  // cleared by a kernel (not a memset), so the call can be captured in a graph
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, stream, out);
  if (M == 0 || K == 0) return hipGetLastError();
  if (layout == SP24_LAYOUT_KBLOCK) {
    const int64_t kb = es == 2 ? 64 : 128;
    const int64_t nblk = (K + kb - 1) / kb;
    const int64_t ppb = (M + 127) / 128 * 128 * (es == 2 ? 8 : 16) / 16;  // 16-byte pieces per block
    const dim3 grid((unsigned)((ppb + 255) / 256 < 64 ? (ppb + 255) / 256 : 64), (unsigned)(nblk < 1024 ? nblk : 1024));
    const char* m = reinterpret_cast<const char*>(meta);
    if (es == 2) hipLaunchKernelGGL((validate_kblock_kernel<2>), grid, dim3(256), 0, stream, m, M, K, nblk, out);
    else hipLaunchKernelGGL((validate_kblock_kernel<1>), grid, dim3(256), 0, stream, m, M, K, nblk, out);
    return hipGetLastError();
  }
  const int64_t nwords = M * (K / 32);
  const unsigned grid = (unsigned)((nwords / 4 + 255) / 256 < 2048 ? (nwords / 4 + 255) / 256 + 1 : 2048);
  hipLaunchKernelGGL(validate_row_kernel, dim3(grid), dim3(256), 0, stream, meta, nwords, out);
  return hipGetLastError();
}

}  // namespace sp24
