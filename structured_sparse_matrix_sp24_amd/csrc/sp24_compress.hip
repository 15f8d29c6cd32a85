// sp24_prune_compress: dense A -> 2:4 compressed values + 2-bit position codes.
//
// Compression as the pages state it ("CDNA and CDNA2 sparse MFMA builtins",
// section "Structured sparsity (4:2 pattern)"): walk K in groups of four,
// keep two positions, store the kept values one after the other, and record
// each kept value's position (0..3) as a 2-bit code.  Which two to keep is
// the library's reading (the pages leave pruning to an offline pass): the
// two largest magnitudes, the lower position winning a tie.
//
// Design: the whole problem is a flat stream bound by HBM bandwidth (no
// MFMA).  Because K % 32 == 0, every 16-byte chunk of A (8 fp16/bf16 = 2
// groups, or 16 8-bit values = 4 groups) maps to exactly 8 bytes of A_vals and
// 1 (16-bit) or 2 (8-bit) bytes of metadata at the same chunk index,
// independent of M and K.  In the row-major layout each lane reads whole
// 16-byte chunks with consecutive lanes on consecutive chunks, so every wave
// instruction (load and store) is one contiguous span.  A is read with
// non-temporal loads (it is not reused); the outputs are written with
// ordinary stores, which measured about 5 % faster than non-temporal ones for
// the 8192^2 fp16 A.  The selection itself is kept short (byte permutes and
// three-input max / median), since with pairwise rank counting the 8-bit
// kernels were bound by the vector ALU rather than by HBM.
//
// The K-blocked output layout (one k-step of the GEMM = KB dense columns per
// block, all M rows of a block stored together) uses a 2-D mapping instead:
// a lane owns one 16-byte chunk of one row's block, so 8 * NB consecutive
// lanes read 128 * NB contiguous bytes of a row, and the values of the
// workgroup's 128 rows go out as one 8 KiB run per block.  The metadata of a
// 128-row group is interleaved for the product's fragment reads, so it is
// gathered in LDS and written as one contiguous 1 or 2 KiB run per block.
#include "sp24_internal.hpp"

namespace sp24 {

// Median of three (the compiler forms max3 from max(max()) itself, but not
// the median).
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Top two of one group of four.  Each element gets a tagged key: its
// magnitude key shifted up by one byte, with 3 - position in the low byte.
// The tagged keys are distinct, a larger magnitude ranks higher, and between
// equal magnitudes the lower position ranks higher, so the two largest tagged
// keys are the two elements kept.  They are found with a three-input maximum
// and median of the first three and one compare-exchange with the fourth:
//   first  = max(max3(t0, t1, t2), t3)
//   second = max(med3(t0, t1, t2), min(max3(t0, t1, t2), t3)).
// Returns the tags of the two kept elements as hi = larger tag (lower
// position p0 = 3 - hi) and lo (p1 = 3 - lo).  About 25 vector instructions
// per group with the key and value byte permutes below, against about 70 for
// pairwise rank counting, which left the 8-bit kernels bound by the ALU.
__device__ __forceinline__ void top2_tags(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3, uint32_t& hi,
                                          uint32_t& lo) {
  const uint32_t m3 = max(max(t0, t1), t2), d3 = med3_u32(t0, t1, t2);
  const uint32_t first = max(m3, t3), second = max(d3, min(m3, t3));
  const uint32_t ta = first & 3u, tb = second & 3u;
  hi = max(ta, tb);
  lo = min(ta, tb);
}
// 4-bit code p0 | p1 << 2 of a group from its kept tags.
__device__ __forceinline__ uint32_t code_of(uint32_t hi, uint32_t lo) { return 15u - (hi + (lo << 2)); }

// Byte permutes build the tagged keys: the key's bytes move up by one and
// byte 0 takes the tag 3 - p from the constant word below (its byte p is
// 3 - p); selector 12 gives a zero byte.
constexpr uint32_t kTagBytes = 0x00010203u;

// One group of four 16-bit values in two words (element p in bits
// 16(p%2).. of word p/2).  Returns the two kept values (low half = lower
// position) and writes the 4-bit code.  The values are picked with a byte
// permute: selector bytes 2p0, 2p0+1, 2p1, 2p1+1 of the 8 bytes lo:hi.
__device__ __forceinline__ uint32_t group16(uint32_t lo_w, uint32_t hi_w, uint32_t& nib) {
  const uint32_t a = lo_w & 0x7FFF7FFFu, b = hi_w & 0x7FFF7FFFu;  // magnitude keys
  const uint32_t t0 = __builtin_amdgcn_perm(kTagBytes, a, 0x0C010004u);
  const uint32_t t1 = __builtin_amdgcn_perm(kTagBytes, a, 0x0C030205u);
  const uint32_t t2 = __builtin_amdgcn_perm(kTagBytes, b, 0x0C010006u);
  const uint32_t t3 = __builtin_amdgcn_perm(kTagBytes, b, 0x0C030207u);
  uint32_t hi, lo;
  top2_tags(t0, t1, t2, t3, hi, lo);
  nib = code_of(hi, lo);
  // p0 = 3 - hi, p1 = 3 - lo: selector 0x01000100 + p0*0x0202 + p1*0x02020000
  // (each 16-bit half of hi | lo << 16 is at most 3, so one 24-bit multiply
  // by 0x0202 doubles and copies both into their two selector bytes)
  const uint32_t sel = 0x07060706u - __umul24(hi | (lo << 16), 0x0202u);
  return __builtin_amdgcn_perm(hi_w, lo_w, sel);
}

// Tagged keys of the four 8-bit values of one word (byte p = position p).
// INT selects |x| keys (int8: |-128| = 128) instead of sign-cleared bit
// patterns (fp8 / bf8).  The byte-wise |x| needs no carries across bytes:
// for a negative byte, (x ^ 0xFF) + 1 = -x <= 128.
template <bool INT>
__device__ __forceinline__ void tags8(uint32_t w, uint32_t t[4]) {
  uint32_t k;
  if constexpr (INT) {
    const uint32_t m = w & 0x80808080u, s = m >> 7;  // sign bit, and 1, of each negative byte
    k = (w ^ (m | (m - s))) + s;                      // m | (m - s): 0xFF in each negative byte
  } else {
    k = w & 0x7F7F7F7Fu;
  }
  t[0] = __builtin_amdgcn_perm(kTagBytes, k, 0x0C0C0004u);
  t[1] = __builtin_amdgcn_perm(kTagBytes, k, 0x0C0C0105u);
  t[2] = __builtin_amdgcn_perm(kTagBytes, k, 0x0C0C0206u);
  t[3] = __builtin_amdgcn_perm(kTagBytes, k, 0x0C0C0307u);
}
// Two groups of four 8-bit values (words a, b) -> their four kept bytes
// (a's p0, p1, then b's) and the two 4-bit codes.
template <bool INT>
__device__ __forceinline__ uint32_t group8x2(uint32_t a, uint32_t b, uint32_t& na, uint32_t& nb) {
  uint32_t ta[4], tb[4], ha, la, hb, lb;
  tags8<INT>(a, ta);
  tags8<INT>(b, tb);
  top2_tags(ta[0], ta[1], ta[2], ta[3], ha, la);
  top2_tags(tb[0], tb[1], tb[2], tb[3], hb, lb);
  na = code_of(ha, la);
  nb = code_of(hb, lb);
  // selector bytes p0a, p1a, 4 + p0b, 4 + p1b with p = 3 - tag
  const uint32_t sel = 0x07070303u - (ha + (la << 8) + (hb << 16) + (lb << 24));
  return __builtin_amdgcn_perm(b, a, sel);
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
      out[0] = (int)group16(d0, d1, n0);
      out[1] = (int)group16(d2, d3, n1);
      vals[q] = out;
      meta[q] = (uint8_t)(n0 | (n1 << 4));
    } else {
      uint32_t n0, n1, n2, n3;
      out[0] = (int)group8x2<INT>(d0, d1, n0, n1);
      out[1] = (int)group8x2<INT>(d2, d3, n2, n3);
      vals[q] = out;
      reinterpret_cast<uint16_t*>(meta)[q] = (uint16_t)(n0 | (n1 << 4) | (n2 << 8) | (n3 << 12));
    }
  }
}

// K-blocked layout.  Workgroup (row tile rt, block group) of T threads
// covers rows rt*128 .. +128 of NB consecutive blocks; thread t handles
// chunk t % (8*NB) of rows rt*128 + t/(8*NB) + (T/(8*NB))*u.  Consecutive workgroups take
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

// Launch shape, measured on cold data over 2048..16384-row, 4096..16384-
// column A: 16-bit types take NB = 2 blocks per workgroup (each row's 256
// contiguous bytes read by 16 lanes) with 512 threads when that still gives
// at least 1024 workgroups, else NB = 1; 8-bit types take NB = 1 with 512
// threads.  Cold inputs, back to back: fp16 8192 x 8192 40 us (41.5 us with
// 256 threads), fp16 4096 x 4096 10.6 us (11.1), int8 8192 x 8192 24 us.
// Measured and not kept: NB = 4 or 8 (with the values staged in LDS so they
// still leave as 8 KiB runs: 40.8 and 43.8 us); consecutive workgroups on
// consecutive row tiles of one block group instead of consecutive block
// groups of one row tile (47 to 52 us); one workgroup per row segment,
// reading rows linearly and scattering values and codes (57 us).  The
// row-major layout's kernel, whose reads and writes are both one linear
// stream, takes 36.3 us for the same A.
constexpr int64_t kKbMinWorkgroups = 1024;
constexpr int kKbBlocks16 = 2, kKbThreads16 = 512, kKbThreads8 = 512;

template <int ES, bool INT, int NB, int T>
__global__ __launch_bounds__(T) void prune_compress_kblock_kernel(const char* __restrict__ A, char* __restrict__ vals,
                                                                  char* __restrict__ meta, int64_t M, int64_t K,
                                                                  uint32_t nblk, uint32_t wg0) {
  constexpr int MB = ES == 2 ? 8 : 16;         // metadata bytes per row per block
  constexpr int CE = 16 / ES;                   // dense elements per chunk
  constexpr int GB = 128 * MB;                  // metadata bytes of one 128-row group per block
  constexpr int CPR = 8 * NB;                   // chunks per row in the tile
  constexpr int RPR = T / CPR;                  // rows per load round
  constexpr int NR = 128 / RPR;                 // load rounds
  __shared__ __attribute__((aligned(16))) char lmeta[NB * GB];
  const uint32_t nwb = (nblk + NB - 1) / NB;
  const uint32_t g = wg0 + blockIdx.x;  // workgroup index over all pieces of the launch
  const int64_t b0 = (int64_t)(g % nwb) * NB;
  const uint32_t rt = g / nwb;
  const int64_t Mp = (M + 127) / 128 * 128;
  const int cc = threadIdx.x % CPR;             // chunk in the tile row
  const int bi = cc / 8, c = cc % 8;            // block in the tile, chunk in the block
  const int64_t b = b0 + bi;
  const int64_t kcol = b * (8 * CE) + (int64_t)c * CE;
  const bool inside = kcol < K;
  const int64_t rowbytes = K * ES;
  // Row rr of the tile (rr = r_first + RPR*u) is row row0 + rr of A; the
  // addresses advance by a uniform stride per round, and the bounds checks
  // are 32-bit compares against the rows this tile has inside M.
  const int64_t row0 = (int64_t)rt * kKbRowsPerTile;
  const int rows_here = (int)min<int64_t>(M - row0, (int64_t)kKbRowsPerTile);
  const int r_first = threadIdx.x / CPR;
  const char* src = A + (row0 + r_first) * rowbytes + kcol * ES;
  char* dst = vals + (b * M + row0 + r_first) * 64 + c * 8;
  i32x4 in[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    in[u] = i32x4{0, 0, 0, 0};
    if (r_first + RPR * u < rows_here && inside)
      in[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(src + (int64_t)(RPR * u) * rowbytes));
  }
  char* lm = lmeta + bi * GB;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int rr = r_first + RPR * u;  // row inside the 128-row group
    const int t = rr >> 4, r = rr & 15;
    const uint32_t d0 = (uint32_t)in[u][0], d1 = (uint32_t)in[u][1];
    const uint32_t d2 = (uint32_t)in[u][2], d3 = (uint32_t)in[u][3];
    i32x2 out = {0, 0};
    const bool live = rr < rows_here && inside;  // padding rows and chunks past K: zero codes
    if constexpr (ES == 2) {
      uint8_t code = 0;
      if (live) {
        uint32_t n0, n1;
        out[0] = (int)group16(d0, d1, n0);
        out[1] = (int)group16(d2, d3, n1);
        code = (uint8_t)(n0 | (n1 << 4));
      }
      lm[(((r * 4 + c / 2) * 4 + t / 2) * 2 + (t & 1)) * 2 + (c & 1)] = (char)code;
    } else {
      uint16_t code = 0;
      if (live) {
        uint32_t n0, n1, n2, n3;
        out[0] = (int)group8x2<INT>(d0, d1, n0, n1);
        out[1] = (int)group8x2<INT>(d2, d3, n2, n3);
        code = (uint16_t)(n0 | (n1 << 4) | (n2 << 8) | (n3 << 12));
      }
      *reinterpret_cast<uint16_t*>(lm + ((r * 4 + c / 2) * 8 + t) * 4 + (c & 1) * 2) = code;
    }
    if (rr < rows_here && b < (int64_t)nblk) *reinterpret_cast<i32x2*>(dst + RPR * 64 * u) = out;
  }
  __syncthreads();
  // each block's group metadata, 16 bytes per thread
#pragma unroll
  for (int q = threadIdx.x; q < NB * GB / 16; q += T) {
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
    const dim3 block(es == 2 ? kKbThreads16 : kKbThreads8);
    const int64_t kb = es == 2 ? 64 : 128;
    const int64_t nblk = (K + kb - 1) / kb;
    const int64_t row_tiles = (M + kKbRowsPerTile - 1) / kKbRowsPerTile;
    const int nb_per_wg =
        (es == 2 && row_tiles * ((nblk + kKbBlocks16 - 1) / kKbBlocks16) >= kKbMinWorkgroups) ? kKbBlocks16 : 1;
    const int64_t nwb = (nblk + nb_per_wg - 1) / nb_per_wg;
    const int64_t total = row_tiles * nwb;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const char* a = static_cast<const char*>(A);
    char* v = static_cast<char*>(vals);
    char* m = reinterpret_cast<char*>(meta);
    const uint32_t nb = (uint32_t)nblk;
    for (int64_t first = 0; first < total; first += kMaxLaunchWorkgroups) {
      const dim3 grid((unsigned)(total - first < kMaxLaunchWorkgroups ? total - first : kMaxLaunchWorkgroups));
      const uint32_t g0 = (uint32_t)first;
      if (es == 2 && nb_per_wg == kKbBlocks16)
        hipLaunchKernelGGL((prune_compress_kblock_kernel<2, false, kKbBlocks16, kKbThreads16>), grid, block, 0,
                           stream, a, v, m, M, K, nb, g0);
      else if (es == 2)
        hipLaunchKernelGGL((prune_compress_kblock_kernel<2, false, 1, kKbThreads16>), grid, block, 0, stream, a, v,
                           m, M, K, nb, g0);
      else if (is_int)
        hipLaunchKernelGGL((prune_compress_kblock_kernel<1, true, 1, kKbThreads8>), grid, block, 0, stream, a, v, m,
                           M, K, nb, g0);
      else
        hipLaunchKernelGGL((prune_compress_kblock_kernel<1, false, 1, kKbThreads8>), grid, block, 0, stream, a, v,
                           m, M, K, nb, g0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int64_t nchunks = M * K * es / 16;
  const int64_t per_block = (int64_t)kCompressThreads * kCompressUnroll;
  const int64_t blocks = (nchunks + per_block - 1) / per_block;
  if (blocks * kCompressThreads > 0xFFFFFFFFll) return hipErrorInvalidValue;  // A > 256 GiB
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
