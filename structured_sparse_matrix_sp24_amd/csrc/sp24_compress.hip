// sp24_prune_compress: dense A -> 2:4 compressed values + 2-bit position codes.
//
// Compression as the pages state it ("CDNA and CDNA2 sparse MFMA builtins",
// section "Structured sparsity (4:2 pattern)"): walk K in groups of four,
// keep two positions, store the kept values one after the other, and record
// each kept value's position (0..3) as a 2-bit code.  Which two to keep is
// the library's reading (the pages leave pruning to an offline pass): the
// two largest magnitudes, the lower position winning a tie.
//
// Design: the whole problem is a flat stream.  Because K % 32 == 0, every
// 16-byte chunk of A (8 fp16/bf16 = 2 groups, or 16 8-bit values = 4 groups)
// maps to exactly 8 bytes of A_vals and 1 (16-bit) or 2 (8-bit) bytes of
// metadata at the same chunk index, independent of M and K.  Each lane reads
// whole 16-byte chunks with consecutive lanes on consecutive chunks, so every
// wave instruction (load and store) is one contiguous span.  No MFMA, no LDS:
// the kernel is bound by HBM bandwidth.  A is read with non-temporal loads
// (it is not reused); the outputs are written with ordinary stores, which
// measured about 5 % faster than non-temporal ones for the 8192^2 fp16 A.
//
// The K-blocked output layout (one k-step of the GEMM = KB dense columns per
// block, all M rows of a block stored together) uses a 2-D mapping instead:
// a lane owns one 16-byte chunk of one row's block (8 chunks per block), so
// eight consecutive lanes read one row's 128 contiguous bytes and a wave
// writes eight consecutive rows of a block, i.e. one contiguous 512-byte run
// of values and one 64- or 128-byte run of metadata.
#include "sp24_internal.hpp"

namespace sp24 {

// Keep mask of one group of 4 magnitude keys: bit i set iff element i is among
// the two largest keys, ties going to the lower index.  rank_i counts the
// elements that beat i; i is kept iff rank_i < 2 (the ranks are a permutation
// of 0..3, so exactly two bits are set).
__device__ __forceinline__ uint32_t keep_mask(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  const uint32_t b01 = k1 > k0, b02 = k2 > k0, b03 = k3 > k0;
  const uint32_t b12 = k2 > k1, b13 = k3 > k1, b23 = k3 > k2;
  const uint32_t r0 = b01 + b02 + b03;
  const uint32_t r1 = (1u - b01) + b12 + b13;
  const uint32_t r2 = (1u - b02) + (1u - b12) + b23;
  const uint32_t r3 = (1u - b03) + (1u - b13) + (1u - b23);
  return (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) | ((uint32_t)(r3 < 2) << 3);
}

// One group of four 16-bit values packed in a 64-bit word (element p in bits
// 16p..16p+15).  Returns the two kept values (low half = lower position) and
// writes the 4-bit code p0 | p1 << 2.
__device__ __forceinline__ uint32_t group16(uint64_t w, uint32_t& nib) {
  const uint32_t e0 = (uint32_t)w & 0xFFFFu, e1 = (uint32_t)(w >> 16) & 0xFFFFu;
  const uint32_t e2 = (uint32_t)(w >> 32) & 0xFFFFu, e3 = (uint32_t)(w >> 48) & 0xFFFFu;
  const uint32_t m = keep_mask(e0 & 0x7FFFu, e1 & 0x7FFFu, e2 & 0x7FFFu, e3 & 0x7FFFu);
  const uint32_t p0 = __builtin_ctz(m), p1 = 31u - __builtin_clz(m);
  nib = p0 | (p1 << 2);
  const uint32_t v0 = (uint32_t)(w >> (16 * p0)) & 0xFFFFu;
  const uint32_t v1 = (uint32_t)(w >> (16 * p1)) & 0xFFFFu;
  return v0 | (v1 << 16);
}

// One group of four 8-bit values in a 32-bit word.  INT selects |x| keys
// (int8) instead of sign-cleared bit patterns (fp8 / bf8).
template <bool INT>
__device__ __forceinline__ uint32_t group8(uint32_t w, uint32_t& nib) {
  uint32_t k[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t b = (w >> (8 * p)) & 0xFFu;
    if constexpr (INT) {
      const int v = (int)(int8_t)b;
      k[p] = (uint32_t)(v < 0 ? -v : v);
    } else {
      k[p] = b & 0x7Fu;
    }
  }
  const uint32_t m = keep_mask(k[0], k[1], k[2], k[3]);
  const uint32_t p0 = __builtin_ctz(m), p1 = 31u - __builtin_clz(m);
  nib = p0 | (p1 << 2);
  return ((w >> (8 * p0)) & 0xFFu) | (((w >> (8 * p1)) & 0xFFu) << 8);
}

constexpr int kCompressThreads = 256;
constexpr int kCompressUnroll = 4;

// ES = element size in bytes; INT = int8 keys.  Chunk q of A -> vals[q] (8 B)
// and meta bytes [q*ES .. q*ES + ES) (the byte order of the uint32 words is
// little-endian, so byte q of the meta array holds codes of groups 2q, 2q+1
// for 16-bit data, and bytes 2q, 2q+1 hold groups 4q..4q+3 for 8-bit data).
template <int ES, bool INT>
__global__ __launch_bounds__(kCompressThreads) void prune_compress_kernel(const i32x4* __restrict__ A,
                                                                            i32x2* __restrict__ vals,
                                                                            uint8_t* __restrict__ meta,
                                                                            int64_t nchunks) {
  const int64_t base = (int64_t)blockIdx.x * (kCompressThreads * kCompressUnroll) + threadIdx.x;
  i32x4 in[kCompressUnroll];
#pragma unroll
  for (int u = 0; u < kCompressUnroll; ++u) {
    const int64_t q = base + (int64_t)u * kCompressThreads;
    if (q < nchunks) in[u] = __builtin_nontemporal_load(A + q);
  }
#pragma unroll
  for (int u = 0; u < kCompressUnroll; ++u) {
    const int64_t q = base + (int64_t)u * kCompressThreads;
    if (q >= nchunks) break;
    const uint32_t d0 = (uint32_t)in[u][0], d1 = (uint32_t)in[u][1];
    const uint32_t d2 = (uint32_t)in[u][2], d3 = (uint32_t)in[u][3];
    i32x2 out;
    if constexpr (ES == 2) {
      uint32_t n0, n1;
      out[0] = (int)group16((uint64_t)d0 | ((uint64_t)d1 << 32), n0);
      out[1] = (int)group16((uint64_t)d2 | ((uint64_t)d3 << 32), n1);
      vals[q] = out;
      meta[q] = (uint8_t)(n0 | (n1 << 4));
    } else {
      uint32_t n0, n1, n2, n3;
      const uint32_t v0 = group8<INT>(d0, n0), v1 = group8<INT>(d1, n1);
      const uint32_t v2 = group8<INT>(d2, n2), v3 = group8<INT>(d3, n3);
      out[0] = (int)(v0 | (v1 << 16));
      out[1] = (int)(v2 | (v3 << 16));
      vals[q] = out;
      reinterpret_cast<uint16_t*>(meta)[q] = (uint16_t)(n0 | (n1 << 4) | (n2 << 8) | (n3 << 12));
    }
  }
}

// K-blocked layout.  Workgroup (row tile rt, block group) covers rows
// rt*128 .. +128 of NB consecutive blocks; thread t handles chunk t % (8*NB)
// of rows rt*128 + t/(8*NB) + (256/(8*NB))*u.  Consecutive workgroups take
// consecutive block groups of the same row tile, so the workgroups in
// flight read one contiguous band of A (DRAM-page friendly); each writes
// one 8 KiB run of values per block.  Chunks past K (the tail of a partial
// last block) are written as zero values with zero codes, and rows past M
// up to the 128-row group boundary get zero codes (the metadata is padded
// to whole groups).
//
// A chunk's codes are half of a code word: chunk c of a row
// holds half c%2 of the row's word g = c/2 (bytes for 16-bit types, 16-bit
// halves for 8-bit types).  In the 128-row group, word g of row 16t + r sits
// at u16 index ((r*4 + g)*4 + t/2)*2 + t%2 (16-bit types) or u32 index
// (r*4 + g)*8 + t (8-bit types).  That interleaving scatters a thread's
// codes, so they are collected in LDS and each block's group of codes
// (1 or 2 KiB, contiguous) is written with 16-byte stores.
constexpr int kKbRowsPerTile = 128;

// Blocks per workgroup (NB): 16-bit types take 4 (each row's 512 contiguous
// bytes are read by 32 lanes) when that still gives at least 1024
// workgroups, else 1 (a 4096 x 4096 A then compresses in 14.5 us instead of
// 16.6 us); 8-bit types always 1 (their metadata is twice as large and the
// staging writes collide in LDS with more blocks).
constexpr int64_t kKbMinWorkgroups = 1024;

template <int ES, bool INT, int NB>
__global__ __launch_bounds__(kCompressThreads) void prune_compress_kblock_kernel(const char* __restrict__ A,
                                                                                   char* __restrict__ vals,
                                                                                   char* __restrict__ meta,
                                                                                   int64_t M, int64_t K,
                                                                                   uint32_t nblk) {
  constexpr int MB = ES == 2 ? 8 : 16;         // metadata bytes per row per block
  constexpr int CE = 16 / ES;                   // dense elements per chunk
  constexpr int GB = 128 * MB;                  // metadata bytes of one 128-row group per block
  constexpr int CPR = 8 * NB;                   // chunks per row in the tile
  constexpr int RPR = kCompressThreads / CPR;   // rows per load round
  constexpr int NR = 128 / RPR;                 // load rounds
  __shared__ __attribute__((aligned(16))) char lmeta[NB * GB];
  const uint32_t nwb = (nblk + NB - 1) / NB;
  const int64_t b0 = (int64_t)(blockIdx.x % nwb) * NB;
  const uint32_t rt = blockIdx.x / nwb;
  const int64_t Mp = (M + 127) / 128 * 128;
  const int cc = threadIdx.x % CPR;             // chunk in the tile row
  const int bi = cc / 8, c = cc % 8;            // block in the tile, chunk in the block
  const int64_t b = b0 + bi;
  const int64_t kcol = b * (8 * CE) + (int64_t)c * CE;
  const bool inside = kcol < K;
  const int64_t rowbytes = K * ES;
  i32x4 in[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int64_t row = (int64_t)rt * kKbRowsPerTile + threadIdx.x / CPR + RPR * u;
    in[u] = i32x4{0, 0, 0, 0};
    if (row < M && inside)
      in[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(A + row * rowbytes + kcol * ES));
  }
  char* lm = lmeta + bi * GB;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int rr = threadIdx.x / CPR + RPR * u;  // row inside the 128-row group
    const int64_t row = (int64_t)rt * kKbRowsPerTile + rr;
    const int t = rr >> 4, r = rr & 15;
    const uint32_t d0 = (uint32_t)in[u][0], d1 = (uint32_t)in[u][1];
    const uint32_t d2 = (uint32_t)in[u][2], d3 = (uint32_t)in[u][3];
    i32x2 out = {0, 0};
    const bool live = row < M && inside;  // padding rows and chunks past K: zero codes
    if constexpr (ES == 2) {
      uint8_t code = 0;
      if (live) {
        uint32_t n0, n1;
        out[0] = (int)group16((uint64_t)d0 | ((uint64_t)d1 << 32), n0);
        out[1] = (int)group16((uint64_t)d2 | ((uint64_t)d3 << 32), n1);
        code = (uint8_t)(n0 | (n1 << 4));
      }
      lm[(((r * 4 + c / 2) * 4 + t / 2) * 2 + (t & 1)) * 2 + (c & 1)] = (char)code;
    } else {
      uint16_t code = 0;
      if (live) {
        uint32_t n0, n1, n2, n3;
        const uint32_t v0 = group8<INT>(d0, n0), v1 = group8<INT>(d1, n1);
        const uint32_t v2 = group8<INT>(d2, n2), v3 = group8<INT>(d3, n3);
        out[0] = (int)(v0 | (v1 << 16));
        out[1] = (int)(v2 | (v3 << 16));
        code = (uint16_t)(n0 | (n1 << 4) | (n2 << 8) | (n3 << 12));
      }
      *reinterpret_cast<uint16_t*>(lm + ((r * 4 + c / 2) * 8 + t) * 4 + (c & 1) * 2) = code;
    }
    if (row < M && b < (int64_t)nblk) *reinterpret_cast<i32x2*>(vals + (b * M + row) * 64 + c * 8) = out;
  }
  __syncthreads();
  // each block's group metadata, 16 bytes per thread
#pragma unroll
  for (int q = threadIdx.x; q < NB * GB / 16; q += kCompressThreads) {
    const int bq = q / (GB / 16), w = q % (GB / 16);
    if (b0 + bq < (int64_t)nblk)
      reinterpret_cast<i32x4*>(meta + ((b0 + bq) * Mp + (int64_t)rt * 128) * MB)[w] =
          *reinterpret_cast<const i32x4*>(lmeta + 16 * q);
  }
}

// Host launcher (arguments already validated).
hipError_t launch_prune_compress(const void* A, void* vals, uint32_t* meta, int64_t M, int64_t K, int dtype,
                                 int layout, hipStream_t stream) {
  const int es = (dtype == SP24_F16 || dtype == SP24_BF16) ? 2 : 1;
  const bool is_int = dtype == SP24_I8;
  if (M == 0 || K == 0) return hipSuccess;
  const dim3 block(kCompressThreads);
  if (layout == SP24_LAYOUT_KBLOCK) {
    const int64_t kb = es == 2 ? 64 : 128;
    const int64_t nblk = (K + kb - 1) / kb;
    const int64_t row_tiles = (M + kKbRowsPerTile - 1) / kKbRowsPerTile;
    const int nb_per_wg = (es == 2 && row_tiles * ((nblk + 3) / 4) >= kKbMinWorkgroups) ? 4 : 1;
    const int64_t nwb = (nblk + nb_per_wg - 1) / nb_per_wg;
    if (row_tiles * nwb > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(row_tiles * nwb));
    const char* a = static_cast<const char*>(A);
    char* v = static_cast<char*>(vals);
    char* m = reinterpret_cast<char*>(meta);
    const uint32_t nb = (uint32_t)nblk;
    if (es == 2 && nb_per_wg == 4)
      hipLaunchKernelGGL((prune_compress_kblock_kernel<2, false, 4>), grid, block, 0, stream, a, v, m, M, K, nb);
    else if (es == 2)
      hipLaunchKernelGGL((prune_compress_kblock_kernel<2, false, 1>), grid, block, 0, stream, a, v, m, M, K, nb);
    else if (is_int)
      hipLaunchKernelGGL((prune_compress_kblock_kernel<1, true, 1>), grid, block, 0, stream, a, v, m, M, K, nb);
    else
      hipLaunchKernelGGL((prune_compress_kblock_kernel<1, false, 1>), grid, block, 0, stream, a, v, m, M, K, nb);
    return hipGetLastError();
  }
  const int64_t nchunks = M * K * es / 16;
  const int64_t per_block = (int64_t)kCompressThreads * kCompressUnroll;
  const int64_t blocks = (nchunks + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  const i32x4* a = static_cast<const i32x4*>(A);
  i32x2* v = static_cast<i32x2*>(vals);
  uint8_t* m = reinterpret_cast<uint8_t*>(meta);
  if (es == 2) hipLaunchKernelGGL((prune_compress_kernel<2, false>), grid, block, 0, stream, a, v, m, nchunks);
  else if (is_int) hipLaunchKernelGGL((prune_compress_kernel<1, true>), grid, block, 0, stream, a, v, m, nchunks);
  else hipLaunchKernelGGL((prune_compress_kernel<1, false>), grid, block, 0, stream, a, v, m, nchunks);
  return hipGetLastError();
}

}  // namespace sp24
