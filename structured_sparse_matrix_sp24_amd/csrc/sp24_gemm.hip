// sp24_gemm: D = alpha * expand(A_vals, meta) * B + beta * C on the gfx950
// sparse matrix cores (v_smfmac_*_16x16x64 for 16-bit inputs, *_16x16x128 for
// 8-bit inputs).
//
// What the instruction computes ("CDNA and CDNA2 sparse MFMA builtins",
// builtin reference and section "Structured sparsity"; ISA page for
// v_smfmac_f32_32x32x32_bf8_bf8, section "Semantics"): one 16x16 tile
// D += expand(A, idx) * B with A held compressed.  The register layouts used
// here were pinned on gfx950 with probe kernels (the pages print only the
// older CDNA shapes):
//   A   lane l holds row l%16; its 16 bytes are 4 (16-bit) or 8 (8-bit)
//       groups of K; lane group ga = l/16.
//   B   lane l holds column l%16; 32 bytes; lane group gb = l/16.
//   idx each lane's own register: code of its compressed element e at bits
//       2e (+16 if ABID is odd, for 16-bit inputs).
//   D   lane l, register r = element (4*(l/16) + r, l%16)  (the pages'
//       16x16 accumulator layout).
//   Group q of A lane group ga meets B lane group gb = 2*(ga%2) + q/H at its
//   group slot t = H*(ga/2) + q%H, where H = groups per A lane / 2.
//
// K mapping chosen from that pairing (per k-step of KS dense columns): A lane
// group ga reads its 16 contiguous compressed bytes [16*ga, 16*ga + 16), so a
// B lane group gb needs two runs of K:
//   16-bit:  k in [8gb, 8gb+8)  and [32+8gb, 32+8gb+8)      (KS = 64)
//   8-bit:   k in [16gb, 16gb+16) and [64+16gb, 64+16gb+16) (KS = 128)
// which the LDS transpose reads (ds_read_b64_tr_b16 / _b8) deliver 4 or 8 k
// at a time from a row-major (k, n) tile.
#include "sp24_internal.hpp"

namespace sp24 {

// ----------------------------------------------------------------------------
// Large-tile kernel: 256 x 256 output tile per workgroup, 4 waves in 2 x 2,
// each wave 128 x 128 = 8 x 8 instruction tiles (256 accumulator registers,
// one wave per SIMD).  Per k-step the workgroup stages A_vals (256 rows x
// 64 B), meta (256 rows x 8 or 16 B) and B (KS rows x 512 or 256 B) into LDS
// with buffer loads that write LDS directly; three stages are in flight.
//
// Each k-step is split into two halves of four column tiles.  The barrier
// that publishes the next stage sits between the halves, and the next
// stage's fragment reads are issued right after it, so the second half's
// MFMAs cover the LDS latency.  All per-lane addresses are computed once;
// inside the loop a stage costs a handful of scalar ops plus immediates.
// ----------------------------------------------------------------------------
constexpr int kBM = 256, kBN = 256, kThreads = 256;
constexpr int kLdsA = kBM * 64;    // 16 KiB
constexpr int kLdsB = 32768;       // KS * BN * esize = 32 KiB for both families
constexpr int kLdsM = kBM * 16;    // 4 KiB (16-bit inputs use half)

// A tile: row r, 16-byte chunk c stored at chunk c ^ swzA(r) (conflict-free
// for 16 lanes reading 16 consecutive rows at one chunk).
__device__ __forceinline__ int swzA(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }
// B tile, 16-bit: row k holds 256 columns = 16 pairs of chunks; pair p stored
// at p ^ swzB16(k).  8-bit: 16 chunks per row; chunk c stored at c ^ swzB8(k).
// For the rows one transpose read touches these depend only on the lane, so
// a lane's read address is a per-lane constant plus immediates.
__device__ __forceinline__ int swzB16(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }
__device__ __forceinline__ int swzB8(int k) { return (k & 7) | (((k >> 4) & 1) << 3); }

struct Stage {
  SP24_LDS char* a;
  SP24_LDS char* b;
  SP24_LDS char* m;
};
constexpr int kLdsStage = kLdsA + kLdsB + kLdsM;  // 52 KiB; three stages = 156 KiB
__device__ __forceinline__ Stage stage_of(SP24_LDS char* base) { return Stage{base, base + kLdsA, base + kLdsA + kLdsB}; }

// Per-lane constants, computed once per workgroup.
struct LaneConsts {
  uint32_t voA[4];  // DMA byte offsets of this lane's A chunks (k-step 0)
  uint32_t voB[8];  // DMA byte offsets of this lane's B chunks within a k-step slice
  uint32_t voM[2];  // DMA byte offsets of this lane's metadata (k-step 0)
  int ldsA;         // LDS offset of this lane's A fragment for tm = 0
  int ldsM;         // LDS offset of this lane's index half-word / word for tm = 0
  int ldsB[8];      // LDS offset of this lane's transpose read for column tile tn (r = 0)
};

struct Frags {
  i32x4 a[8];
  int idx[8];
};
struct BHalf {
  i32x8 b[4];
};

template <int OP>
__device__ __forceinline__ LaneConsts make_lane_consts(int w, int l, int64_t rowA, int64_t rowM, int ldb) {
  constexpr int ES = op_esize(OP);
  LaneConsts c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (w * 4 + i) * 16 + (l >> 2);
    c.voA[i] = (uint32_t)(row * rowA + 16 * ((l & 3) ^ swzA(row)));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = w * 8 + i;
    int row, ch;
    if constexpr (ES == 2) {
      row = j * 2 + (l >> 5);
      const int p = l & 31;
      ch = (((p >> 1) ^ swzB16(row)) << 1) | (p & 1);
    } else {
      row = j * 4 + (l >> 4);
      ch = (l & 15) ^ swzB8(row);
    }
    c.voB[i] = (uint32_t)(row * ldb + 16 * ch);
  }
  if constexpr (ES == 2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) c.voM[i] = (uint32_t)(((w * 2 + i) * 32 + (l >> 1)) * rowM + 4 * (l & 1));
  } else {
    c.voM[0] = (uint32_t)((w * 64 + l) * rowM);
    c.voM[1] = 0;
  }
  const int wm = w >> 1, wn = w & 1, ga = l >> 4, r16 = l & 15;
  c.ldsA = (wm * 128 + r16) * 64 + 16 * (ga ^ swzA(r16));
  c.ldsM = ES == 2 ? (wm * 128 + r16) * 8 + 2 * ga : (wm * 128 + r16) * 16 + 4 * ga;
  const int gb = l >> 4, s = l & 15;
#pragma unroll
  for (int tn = 0; tn < 8; ++tn) {
    const int ct = wn * 8 + tn;
    if constexpr (ES == 2) {
      const int k0 = 8 * gb + (s >> 2);
      c.ldsB[tn] = k0 * 512 + ((ct ^ swzB16(k0)) << 5) + (s & 3) * 8;
    } else {
      const int k0 = 16 * gb + (s >> 1);
      c.ldsB[tn] = k0 * 256 + ((ct ^ swzB8(k0)) << 4) + (s & 1) * 8;
    }
  }
  return c;
}

// Issue the DMA of one k-step into a stage.  `full` = the k-step lies wholly
// inside K (every step but possibly the last); the last step of a K that is
// not a multiple of KS masks the A chunks past the row end.
template <int OP>
__device__ __forceinline__ void issue_stage(const Stage& st, const LaneConsts& lc, i32x4 rA, i32x4 rM, const char* B,
                                            int64_t btotal, int n0, int N, int64_t rowA, int w, int ks, bool full) {
  constexpr int KS = op_kstep(OP), ES = op_esize(OP);
  const int l = lane_id();
  if (full) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16_asm(rA, lds_addr(st.a + (w * 4 + i) * 1024), (uint32_t)((int)lc.voA[i]), (uint32_t)(ks * 64));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (w * 4 + i) * 16 + (l >> 2);
      const int64_t col = (int64_t)ks * 64 + 16 * ((l & 3) ^ swzA(row));
      const uint32_t off = col < rowA ? lc.voA[i] + (uint32_t)(ks * 64) : kOOB;
      dma16_asm(rA, lds_addr(st.a + (w * 4 + i) * 1024), (uint32_t)((int)off), (uint32_t)(0));
    }
  }
  const int64_t start = ((int64_t)ks * KS * N + n0) * ES;
  const i32x4 rB = make_rsrc4(B + start, btotal - start);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    dma16_asm(rB, lds_addr(st.b + (w * 8 + i) * 1024), (uint32_t)((int)lc.voB[i]), (uint32_t)(0));
  if constexpr (ES == 2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (full) {
        dma4_asm(rM, lds_addr(st.m + (w * 2 + i) * 256), (uint32_t)((int)lc.voM[i]), (uint32_t)(ks * 8));
      } else {
        dma4_asm(rM, lds_addr(st.m + (w * 2 + i) * 256), (uint32_t)((int)(lc.voM[i] + ks * 8)), (uint32_t)(0));
      }
    }
  } else {
    if (full) dma16_asm(rM, lds_addr(st.m + w * 1024), (uint32_t)((int)lc.voM[0]), (uint32_t)(ks * 16));
    else dma16_asm(rM, lds_addr(st.m + w * 1024), (uint32_t)((int)(lc.voM[0] + ks * 16)), (uint32_t)(0));
  }
}

// Loads issued per wave per stage (vmcnt budget).
template <int OP>
constexpr int loads_per_stage() { return op_esize(OP) == 2 ? 4 + 8 + 2 : 4 + 8 + 1; }

template <int OP>
__device__ __forceinline__ void read_a(const Stage& st, const LaneConsts& lc, Frags& f) {
  constexpr int ES = op_esize(OP);
#pragma unroll
  for (int tm = 0; tm < 8; ++tm) {
    f.a[tm] = *(const SP24_LDS i32x4*)(st.a + lc.ldsA + tm * 1024);
    if constexpr (ES == 2) f.idx[tm] = *(const SP24_LDS unsigned short*)(st.m + lc.ldsM + tm * 128);
    else f.idx[tm] = *(const SP24_LDS int*)(st.m + lc.ldsM + tm * 256);
  }
}

// B fragments of column tiles 4H .. 4H+3: four transpose reads each, at row
// offsets +0, +4 (or +8), +32 (or +64) and +36 (or +72) from the lane's base,
// which are byte offsets 0, 2048, 16384, 18432 for both element sizes.
template <int OP, int H>
__device__ __forceinline__ void read_b(const Stage& st, const LaneConsts& lc, BHalf& h) {
  constexpr int ES = op_esize(OP);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const SP24_LDS char* p = st.b + lc.ldsB[4 * H + t];
    i32x2 q[4];
    if constexpr (ES == 2) {
      q[0] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p)));
      q[1] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p + 2048)));
      q[2] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p + 16384)));
      q[3] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p + 18432)));
    } else {
      q[0] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p));
      q[1] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p + 2048));
      q[2] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p + 16384));
      q[3] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p + 18432));
    }
    h.b[t] = i32x8{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
  }
}

template <int OP, int H>
__device__ __forceinline__ void mma_half(i32x4 (&acc)[8][8], const Frags& f, const BHalf& h) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int tm = 0; tm < 8; ++tm) acc[tm][4 * H + t] = smfmac16<OP>(acc[tm][4 * H + t], f.a[tm], h.b[t], f.idx[tm]);
}

// Workgroup barrier that the compiler may not move memory operations across
// (the data behind it was written by other waves' direct-to-LDS loads).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int OP>
__global__ __launch_bounds__(kThreads, 1) void gemm_large_kernel(const char* __restrict__ A_vals,
                                                                  const char* __restrict__ meta,
                                                                  const char* __restrict__ B, void* C, int M, int N,
                                                                  int K, float alpha, float beta, int tiles_m,
                                                                  int tiles_n) {
  // One LDS object per stage (A | B | meta): the compiler's wait insertion
  // tells direct-to-LDS loads apart only by the object they write, and it
  // tracks only a few such objects.
  __shared__ __attribute__((aligned(1024))) char lS0[kLdsStage], lS1[kLdsStage], lS2[kLdsStage];
  const Stage s0 = stage_of((SP24_LDS char*)lS0);
  const Stage s1 = stage_of((SP24_LDS char*)lS1);
  const Stage s2 = stage_of((SP24_LDS char*)lS2);
  constexpr int KS = op_kstep(OP), ES = op_esize(OP);

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of tiles so neighbouring tiles share its L2, then walk
  // that range in groups of 8 tile-rows.
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GM = 8;
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = t - group * GM * tiles_n;
  const int m0 = (first_m + in_group % gsize) * kBM;
  const int n0 = (in_group / gsize) * kBN;

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = lane_id();
  const int64_t rowA = (int64_t)K / 2 * ES;  // bytes per compressed row
  const int64_t rowM = (int64_t)K / 8;       // bytes per metadata row
  const int ldb = N * ES;
  const LaneConsts lc = make_lane_consts<OP>(w, l, rowA, rowM, ldb);
  const i32x4 rA = make_rsrc4(A_vals + (int64_t)m0 * rowA, (int64_t)(M - m0) * rowA);
  const i32x4 rM = make_rsrc4(meta + (int64_t)m0 * rowM, (int64_t)(M - m0) * rowM);
  const int64_t btotal = (int64_t)K * N * ES;
  const int nsteps = (K + KS - 1) / KS;
  const int nfull = K / KS;  // steps that lie wholly inside K

  i32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  constexpr int LPS = loads_per_stage<OP>();
  auto issue = [&](const Stage& st, int ks) {
    issue_stage<OP>(st, lc, rA, rM, B, btotal, n0, N, rowA, w, ks, ks < nfull);
  };
  // Two register sets (X, Y) for the fragments of consecutive steps and
  // three LDS stages: the roles repeat every 6 steps, so the loop is unrolled
  // 6 times and no fragment is ever copied between registers.
  Frags fX, fY;
  BHalf b1X, b1Y, b2;
  if (nsteps > 0) {
    issue(s0, 0);
    if (nsteps > 1) issue(s1, 1);
    if (nsteps > 1) waitcnt<LPS, 0>();
    else waitcnt<0, 0>();
    stage_barrier();
    if (nsteps > 2) issue(s2, 2);
    read_a<OP>(s0, lc, fX);
    read_b<OP, 0>(s0, lc, b1X);
  }
  // One k-step on stage `cur` with fragments (fc, b1c); step ks+1 lives in
  // stage `nxt` and its fragments go to (fn, b1n).  The DMA of step ks+3
  // reuses `cur` once every wave has passed the barrier (all reads of `cur`
  // have completed by then).
  auto step = [&](const Stage& cur, const Stage& nxt, int ks, Frags& fc, BHalf& b1c, Frags& fn, BHalf& b1n) {
    read_b<OP, 1>(cur, lc, b2);
    mma_half<OP, 0>(acc, fc, b1c);
    if (ks + 1 < nsteps) {
      if (ks + 2 < nsteps) waitcnt<LPS, 0>();
      else waitcnt<0, 0>();
      stage_barrier();
      if (ks + 3 < nsteps) issue(cur, ks + 3);
      read_a<OP>(nxt, lc, fn);
      read_b<OP, 0>(nxt, lc, b1n);
    }
    mma_half<OP, 1>(acc, fc, b2);
  };
  // Whole rounds of six steps, then up to five more (a single loop with early
  // exits gives the register allocator several live states at once and it
  // spills).
  int ks = 0;
  for (; ks + 6 <= nsteps; ks += 6) {
    step(s0, s1, ks + 0, fX, b1X, fY, b1Y);
    step(s1, s2, ks + 1, fY, b1Y, fX, b1X);
    step(s2, s0, ks + 2, fX, b1X, fY, b1Y);
    step(s0, s1, ks + 3, fY, b1Y, fX, b1X);
    step(s1, s2, ks + 4, fX, b1X, fY, b1Y);
    step(s2, s0, ks + 5, fY, b1Y, fX, b1X);
  }
  if (ks + 0 < nsteps) step(s0, s1, ks + 0, fX, b1X, fY, b1Y);
  if (ks + 1 < nsteps) step(s1, s2, ks + 1, fY, b1Y, fX, b1X);
  if (ks + 2 < nsteps) step(s2, s0, ks + 2, fX, b1X, fY, b1Y);
  if (ks + 3 < nsteps) step(s0, s1, ks + 3, fY, b1Y, fX, b1X);
  if (ks + 4 < nsteps) step(s1, s2, ks + 4, fX, b1X, fY, b1Y);

  // ---- epilogue: D = alpha * acc + beta * C  (int8: acc + C when beta == 1)
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int tm = 0; tm < 8; ++tm) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 128 + tm * 16 + 4 * (l >> 4) + r;
      if (row >= M) continue;
#pragma unroll
      for (int tn = 0; tn < 8; ++tn) {
        const int col = n0 + wn * 128 + tn * 16 + (l & 15);
        if (col >= N) continue;
        const int64_t o = (int64_t)row * N + col;
        if constexpr (op_is_int(OP)) {
          int* D = static_cast<int*>(C);
          const int v = acc[tm][tn][r];
          D[o] = beta != 0.0f ? v + D[o] : v;
        } else {
          // cast the whole vector: a bit cast of one vector element is not safe here
          const f32x4 fv = __builtin_bit_cast(f32x4, acc[tm][tn]);
          float* D = static_cast<float*>(C);
          const float v = fv[r] * alpha;
          D[o] = beta != 0.0f ? v + beta * D[o] : v;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// 8-wave variant of the large-tile kernel: the same 256 x 256 tile and A / B
// LDS layout, but 8 waves (two per SIMD) in 2 x 4, each owning 128 x 64 =
// 8 x 4 instruction tiles (128 accumulators).  With two waves per SIMD one
// wave's LDS reads and barrier waits overlap the other wave's MFMAs.
//
// Global -> LDS staging:
//   A, B   one k-step per stage, three stages (48 KiB each) in flight;
//   meta   two k-steps per load (16 or 32 contiguous bytes per row instead
//          of 8 or 16 -- the per-row pieces are what the loads pay for), in
//          its own double buffer, issued together with the A / B data of the
//          group's first step.
// ----------------------------------------------------------------------------
constexpr int kThreads8 = 512;
constexpr int kLdsAB = kLdsA + kLdsB;        // 48 KiB per stage
constexpr int kLdsMeta = kBM * 32;           // one metadata group, 8 KiB (16-bit inputs use half)

struct LaneConsts8 {
  uint32_t voA[2];
  uint32_t voB[4];
  uint32_t voM[2];
  int ldsA;
  int ldsM;
  int ldsB[4];
};

// Metadata group: 2 k-steps.  LDS layout [row][group bytes]: 16 B per row for
// 16-bit inputs (k-step j of the group at byte 8j), 32 B for 8-bit (16j).
template <int OP>
__host__ __device__ constexpr int meta_group_bytes() { return op_esize(OP) == 2 ? 16 : 32; }
// DMA loads per wave per group: 16-bit inputs 2 x (16 rows x 16 B, 4 B per
// lane); 8-bit inputs 1 x (32 rows x 32 B, 16 B per lane).
template <int OP>
__host__ __device__ constexpr int meta_loads8() { return op_esize(OP) == 2 ? 2 : 1; }

template <int OP>
__device__ __forceinline__ LaneConsts8 make_lane_consts8(int w, int l, int64_t rowA, int64_t rowM, int ldb) {
  constexpr int ES = op_esize(OP);
  LaneConsts8 c;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (w * 2 + i) * 16 + (l >> 2);
    c.voA[i] = (uint32_t)(row * rowA + 16 * ((l & 3) ^ swzA(row)));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = w * 4 + i;
    int row, ch;
    if constexpr (ES == 2) {
      row = j * 2 + (l >> 5);
      const int p = l & 31;
      ch = (((p >> 1) ^ swzB16(row)) << 1) | (p & 1);
    } else {
      row = j * 4 + (l >> 4);
      ch = (l & 15) ^ swzB8(row);
    }
    c.voB[i] = (uint32_t)(row * ldb + 16 * ch);
  }
  if constexpr (ES == 2) {
    // 256 rows x 16 B = 4 KiB: two 4-byte loads per lane per wave (16 rows each)
#pragma unroll
    for (int i = 0; i < 2; ++i) c.voM[i] = (uint32_t)(((w * 2 + i) * 16 + (l >> 2)) * rowM + 4 * (l & 3));
  } else {
    // 256 rows x 32 B = 8 KiB: one 16-byte load per lane per wave (32 rows)
    c.voM[0] = (uint32_t)((w * 32 + (l >> 1)) * rowM + 16 * (l & 1));
    c.voM[1] = 0;
  }
  const int wm = w >> 2, wn = w & 3, ga = l >> 4, r16 = l & 15;
  c.ldsA = (wm * 128 + r16) * 64 + 16 * (ga ^ swzA(r16));
  c.ldsM = (wm * 128 + r16) * meta_group_bytes<OP>() + (ES == 2 ? 2 * ga : 4 * ga);
  const int gb = l >> 4, s = l & 15;
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const int ct = wn * 4 + tn;
    if constexpr (ES == 2) {
      const int k0 = 8 * gb + (s >> 2);
      c.ldsB[tn] = k0 * 512 + ((ct ^ swzB16(k0)) << 5) + (s & 3) * 8;
    } else {
      const int k0 = 16 * gb + (s >> 1);
      c.ldsB[tn] = k0 * 256 + ((ct ^ swzB8(k0)) << 4) + (s & 1) * 8;
    }
  }
  return c;
}

constexpr int kLoadsAB8 = 2 + 4;  // A + B loads per wave per k-step

// A and B of k-step ks into a stage.  `full`: the step lies wholly inside K
// (the last step of a K that is not a multiple of KS masks A past the row end).
template <int OP>
__device__ __forceinline__ void issue_ab8(SP24_LDS char* st, const LaneConsts8& lc, i32x4 rA, const char* B,
                                          int64_t btotal, int n0, int N, int64_t rowA, int w, int ks, bool full) {
  constexpr int KS = op_kstep(OP), ES = op_esize(OP);
  const int l = lane_id();
  const uint32_t la = lds_addr(st);
  if (full) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_asm(rA, la + (w * 2 + i) * 1024, lc.voA[i], (uint32_t)(ks * 64));
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (w * 2 + i) * 16 + (l >> 2);
      const int64_t col = (int64_t)ks * 64 + 16 * ((l & 3) ^ swzA(row));
      const uint32_t off = col < rowA ? lc.voA[i] + (uint32_t)(ks * 64) : kOOB;
      dma16_asm(rA, la + (w * 2 + i) * 1024, off, 0u);
    }
  }
  const int64_t start = ((int64_t)ks * KS * N + n0) * ES;
  const i32x4 rB = make_rsrc4(B + start, btotal - start);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16_asm(rB, la + kLdsA + (w * 4 + i) * 1024, lc.voB[i], 0u);
}

// Metadata group g (k-steps 2g, 2g+1) into a metadata buffer.  Rows past M and
// bytes past the row end read as zero (range-checked loads; the zero codes
// meet zero A values).
template <int OP>
__device__ __forceinline__ void issue_meta8(SP24_LDS char* mb, const LaneConsts8& lc, i32x4 rM, int64_t rowM, int w,
                                            int g) {
  constexpr int GB = meta_group_bytes<OP>();
  const int l = lane_id();
  const uint32_t la = lds_addr(mb);
  if constexpr (op_esize(OP) == 2) {
    const int64_t col = (int64_t)g * GB + 4 * (l & 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = col < rowM ? lc.voM[i] + (uint32_t)(g * GB) : kOOB;
      dma4_asm(rM, la + (w * 2 + i) * 256, off, 0u);
    }
  } else {
    const int64_t col = (int64_t)g * GB + 16 * (l & 1);
    const uint32_t off = col < rowM ? lc.voM[0] + (uint32_t)(g * GB) : kOOB;
    dma16_asm(rM, la + w * 1024, off, 0u);
  }
}

template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() { waitcnt<VM, 0>(); }

template <int OP>
__global__ __launch_bounds__(kThreads8) void gemm_large8_kernel(const char* __restrict__ A_vals,
                                                                 const char* __restrict__ meta,
                                                                 const char* __restrict__ B, void* C, int M, int N,
                                                                 int K, float alpha, float beta, int tiles_m,
                                                                 int tiles_n) {
  // One LDS object per buffer.
  __shared__ __attribute__((aligned(1024))) char lS0[kLdsAB], lS1[kLdsAB], lS2[kLdsAB];
  __shared__ __attribute__((aligned(1024))) char lM0[kLdsMeta], lM1[kLdsMeta];
  // (uniform selects; an array of LDS pointers would become a table in memory)
  auto st = [&](int i) -> SP24_LDS char* {
    return i == 0 ? (SP24_LDS char*)lS0 : (i == 1 ? (SP24_LDS char*)lS1 : (SP24_LDS char*)lS2);
  };
  auto mb = [&](int i) -> SP24_LDS char* { return i == 0 ? (SP24_LDS char*)lM0 : (SP24_LDS char*)lM1; };
  constexpr int KS = op_kstep(OP), ES = op_esize(OP);
  constexpr int LM = meta_loads8<OP>();

  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GM = 8;
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = t - group * GM * tiles_n;
  const int m0 = (first_m + in_group % gsize) * kBM;
  const int n0 = (in_group / gsize) * kBN;

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = lane_id();
  const int64_t rowA = (int64_t)K / 2 * ES;
  const int64_t rowM = (int64_t)K / 8;
  const int ldb = N * ES;
  const LaneConsts8 lc = make_lane_consts8<OP>(w, l, rowA, rowM, ldb);
  const i32x4 rA = make_rsrc4(A_vals + (int64_t)m0 * rowA, (int64_t)(M - m0) * rowA);
  const i32x4 rM = make_rsrc4(meta + (int64_t)m0 * rowM, (int64_t)(M - m0) * rowM);
  const int64_t btotal = (int64_t)K * N * ES;
  const int nsteps = (K + KS - 1) / KS;
  const int nfull = K / KS;

  i32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  // DMA of step j: its metadata group first when j starts a group.
  auto issue = [&](int j) {
    if ((j & 1) == 0) issue_meta8<OP>(mb((j >> 1) & 1), lc, rM, rowM, w, j >> 1);
    issue_ab8<OP>(st(j % 3), lc, rA, B, btotal, n0, N, rowA, w, j, j < nfull);
  };
  if (nsteps > 0) issue(0);
  if (nsteps > 1) issue(1);
  for (int ks = 0; ks < nsteps; ++ks) {
    // Step ks's data is complete once only the loads of step ks+1 remain.
    if (ks + 1 < nsteps) {
      if (((ks + 1) & 1) == 0) wait_vm_lgkm0<kLoadsAB8 + LM>();
      else wait_vm_lgkm0<kLoadsAB8>();
    } else {
      wait_vm_lgkm0<0>();
    }
    stage_barrier();
    if (ks + 2 < nsteps) issue(ks + 2);
    const SP24_LDS char* cur = st(ks % 3);
    const SP24_LDS char* cm = mb((ks >> 1) & 1) + (ks & 1) * (meta_group_bytes<OP>() / 2);
    i32x8 b[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const SP24_LDS char* p = cur + kLdsA + lc.ldsB[tn];
      i32x2 q[4];
      if constexpr (ES == 2) {
        q[0] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p)));
        q[1] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p + 2048)));
        q[2] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p + 16384)));
        q[3] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(p + 18432)));
      } else {
        q[0] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p));
        q[1] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p + 2048));
        q[2] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p + 16384));
        q[3] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(p + 18432));
      }
      b[tn] = i32x8{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
    }
#pragma unroll
    for (int tm = 0; tm < 8; ++tm) {
      const i32x4 a = *(const SP24_LDS i32x4*)(cur + lc.ldsA + tm * 1024);
      int idx;
      if constexpr (ES == 2) idx = *(const SP24_LDS unsigned short*)(cm + lc.ldsM + tm * 16 * 16);
      else idx = *(const SP24_LDS int*)(cm + lc.ldsM + tm * 16 * 32);
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = smfmac16<OP>(acc[tm][tn], a, b[tn], idx);
    }
  }

  const int wm = w >> 2, wn = w & 3;
#pragma unroll
  for (int tm = 0; tm < 8; ++tm) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 128 + tm * 16 + 4 * (l >> 4) + r;
      if (row >= M) continue;
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int col = n0 + wn * 64 + tn * 16 + (l & 15);
        if (col >= N) continue;
        const int64_t o = (int64_t)row * N + col;
        if constexpr (op_is_int(OP)) {
          int* D = static_cast<int*>(C);
          const int v = acc[tm][tn][r];
          D[o] = beta != 0.0f ? v + D[o] : v;
        } else {
          const f32x4 fv = __builtin_bit_cast(f32x4, acc[tm][tn]);
          float* D = static_cast<float*>(C);
          const float v = fv[r] * alpha;
          D[o] = beta != 0.0f ? v + beta * D[o] : v;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Small-N kernel (N <= 64): A is read from HBM exactly once.  A workgroup of
// 8 waves owns one 16-row tile and all N columns; the waves split the
// k-steps round-robin, each staging its own B slice (KS x N) through LDS for
// the transpose reads, and the 8 partial tiles are summed on chip in a fixed
// order (deterministic).
// ----------------------------------------------------------------------------
constexpr int kSmallWaves = 8;
constexpr int kSmallBSlice = 64 * 64 * 2;  // KS * N * esize bytes, N <= 64

template <int OP>
__global__ __launch_bounds__(kSmallWaves * 64) void gemm_smalln_kernel(const char* __restrict__ A_vals,
                                                                        const char* __restrict__ meta,
                                                                        const char* __restrict__ B, void* C, int M,
                                                                        int N, int K, float alpha, float beta) {
  constexpr int KS = op_kstep(OP), ES = op_esize(OP);
  __shared__ __attribute__((aligned(1024))) char lB[kSmallWaves][2][kSmallBSlice];
  const int w = threadIdx.x >> 6, l = lane_id();
  const int m0 = blockIdx.x * 16;
  const int ga = l >> 4, gb = l >> 4, s = l & 15;
  const int nt = (N + 15) >> 4;
  const int nsteps = (K + KS - 1) / KS;
  const int64_t rowA = (int64_t)K / 2 * ES, rowM = (int64_t)K / 8;
  const int ldb = N * ES;                 // bytes per B row (multiple of 16)
  const int chunks_per_row = ldb >> 4;
  const int slice_instr = (KS * ldb) >> 10;  // 1 KiB per DMA instruction (KS*ldb is a multiple of 1 KiB)
  const int row = m0 + (l & 15);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A_vals + (int64_t)m0 * rowA, (int64_t)(M - m0) * rowA);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(meta + (int64_t)m0 * rowM, (int64_t)(M - m0) * rowM);
  const int64_t btotal = (int64_t)K * ldb;

  i32x4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  // Register prefetch of A and idx, LDS double buffer of the B slice.
  auto fetch = [&](int ks, int buf, i32x4& a, int& idx) {
    const int64_t col = (int64_t)ks * 64 + 16 * ga;
    const uint32_t offa = col < rowA ? (uint32_t)((l & 15) * rowA + col) : kOOB;
    a = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)offa, 0, 0);
    if constexpr (ES == 2) idx = (int)__builtin_amdgcn_raw_buffer_load_b16(rm, (int)((l & 15) * rowM + ks * 8 + 2 * ga), 0, 0);
    else idx = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, (int)((l & 15) * rowM + ks * 16 + 4 * ga), 0, 0);
    const int64_t start = (int64_t)ks * KS * ldb;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + start, btotal - start);
    for (int j = 0; j < slice_instr; ++j) {
      const int q = j * 64 + l;  // chunk index inside the slice
      const int brow = q / chunks_per_row, bc = q - brow * chunks_per_row;
      dma16(rb, (SP24_LDS char*)lB[w][buf] + j * 1024, (uint32_t)(brow * ldb + 16 * bc));
    }
  };
  i32x4 a_cur, a_nxt;
  int i_cur = 0, i_nxt = 0;
  int ks = w, buf = 0;
  if (ks < nsteps) fetch(ks, 0, a_cur, i_cur);
  for (; ks < nsteps; ks += kSmallWaves) {
    const int ksn = ks + kSmallWaves;
    if (ksn < nsteps) fetch(ksn, buf ^ 1, a_nxt, i_nxt);
    // wait for everything except the prefetch just issued
    if (ksn < nsteps) {
      switch (slice_instr) {  // the prefetch is 2 + slice_instr loads
        case 1: waitcnt<3>(); break;
        case 2: waitcnt<4>(); break;
        case 3: waitcnt<5>(); break;
        case 4: waitcnt<6>(); break;
        case 5: waitcnt<7>(); break;
        case 6: waitcnt<8>(); break;
        case 7: waitcnt<9>(); break;
        default: waitcnt<10>(); break;
      }
    } else {
      waitcnt<0>();
    }
    const SP24_LDS char* sb = (const SP24_LDS char*)lB[w][buf];
    for (int tn = 0; tn < nt; ++tn) {
      i32x2 p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (ES == 2) {
          const int k = 8 * gb + 4 * (r & 1) + 32 * (r >> 1) + (s >> 2);
          const int addr = k * ldb + tn * 32 + (s & 3) * 8;
          p[r] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((SP24_LDS i16x4*)(sb + addr)));
        } else {
          const int k = 16 * gb + 8 * (r & 1) + 64 * (r >> 1) + (s >> 1);
          const int addr = k * ldb + tn * 16 + (s & 1) * 8;
          p[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SP24_LDS i32x2*)(sb + addr));
        }
      }
      const i32x8 b = {p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
      acc[tn] = smfmac16<OP>(acc[tn], a_cur, b, i_cur);
    }
    a_cur = a_nxt;
    i_cur = i_nxt;
    buf ^= 1;
  }
  // ---- reduce the 8 partial tiles in LDS (fixed order), then epilogue
  waitcnt<0, 0>();
  __syncthreads();
  int* red = (int*)&lB[0][0][0];  // 8 waves x 4 tiles x 64 lanes x 4 regs x 4 B = 32 KiB
  for (int tn = 0; tn < nt; ++tn)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((w * 4 + tn) * 4 + r) * 64 + l] = acc[tn][r];
  __syncthreads();
  // thread t handles output element (i, j) = (t / 64 .. ) of the 16 x N tile
  for (int e = threadIdx.x; e < 16 * nt * 16; e += kSmallWaves * 64) {
    const int tn = e >> 8, within = e & 255;
    const int i = within >> 4, j = within & 15;
    const int lane = 16 * (i >> 2) + j, r = i & 3;
    const int grow = m0 + i, gcol = tn * 16 + j;
    if (grow >= M || gcol >= N) continue;
    const int64_t o = (int64_t)grow * N + gcol;
    if constexpr (op_is_int(OP)) {
      int sum = 0;
      for (int ww = 0; ww < kSmallWaves; ++ww) sum += red[((ww * 4 + tn) * 4 + r) * 64 + lane];
      int* D = static_cast<int*>(C);
      D[o] = beta != 0.0f ? sum + D[o] : sum;
    } else {
      float sum = 0.0f;
      for (int ww = 0; ww < kSmallWaves; ++ww) sum += __int_as_float(red[((ww * 4 + tn) * 4 + r) * 64 + lane]);
      float* D = static_cast<float*>(C);
      const float v = alpha * sum;
      D[o] = beta != 0.0f ? v + beta * D[o] : v;
    }
  }
}

// ---- K == 0: D = beta * C ---------------------------------------------------
template <bool INT>
__global__ void scale_c_kernel(void* C, int64_t n, float beta) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if constexpr (INT) {
    int* D = static_cast<int*>(C);
    D[i] = beta != 0.0f ? D[i] : 0;
  } else {
    float* D = static_cast<float*>(C);
    D[i] = beta != 0.0f ? beta * D[i] : 0.0f;
  }
}

template <int OP>
static hipError_t launch_op(const void* A_vals, const uint32_t* meta, const void* B, void* C, int M, int N, int K,
                            float alpha, float beta, hipStream_t stream) {
  const char* a = static_cast<const char*>(A_vals);
  const char* m = reinterpret_cast<const char*>(meta);
  const char* b = static_cast<const char*>(B);
  if (K == 0) {
    const int64_t n = (int64_t)M * N;
    hipLaunchKernelGGL((scale_c_kernel<op_is_int(OP)>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, C, n,
                       beta);
    return hipGetLastError();
  }
  if (N <= 64) {
    hipLaunchKernelGGL((gemm_smalln_kernel<OP>), dim3((unsigned)((M + 15) / 16)), dim3(kSmallWaves * 64), 0, stream,
                       a, m, b, C, M, N, K, alpha, beta);
    return hipGetLastError();
  }
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
#ifdef SP24_LARGE4
  hipLaunchKernelGGL((gemm_large_kernel<OP>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0, stream, a, m, b,
                     C, M, N, K, alpha, beta, tiles_m, tiles_n);
#else
  hipLaunchKernelGGL((gemm_large8_kernel<OP>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads8), 0, stream, a, m,
                     b, C, M, N, K, alpha, beta, tiles_m, tiles_n);
#endif
  return hipGetLastError();
}

hipError_t launch_gemm(int op, const void* A_vals, const uint32_t* meta, const void* B, void* C, int M, int N, int K,
                       float alpha, float beta, hipStream_t stream) {
  switch (op) {
    case OP_F16: return launch_op<OP_F16>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    case OP_BF16: return launch_op<OP_BF16>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    case OP_I8: return launch_op<OP_I8>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    case OP_FP8_FP8: return launch_op<OP_FP8_FP8>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    case OP_FP8_BF8: return launch_op<OP_FP8_BF8>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    case OP_BF8_FP8: return launch_op<OP_BF8_FP8>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    case OP_BF8_BF8: return launch_op<OP_BF8_BF8>(A_vals, meta, B, C, M, N, K, alpha, beta, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sp24
