// Device-side building blocks of the flash-CCE head for gfx950 (CDNA4).
//
// One GEMM core serves every contraction of the head.  Both operands are
// row-major with K contiguous ("NT"): C[i][j] = sum_k A[i][k] * B[j][k].
//
//   workgroup tile   256 (A rows) x 256 (B rows), 256 threads = 4 waves
//   wave tile        128 x 128 = 4 x 4 MFMA tiles of 32x32, fp32 accumulators
//   MFMA             v_mfma_f32_32x32x16_bf16 (8 bf16 of K per lane)
//   K pipeline       32 bf16 per stage, a ring of 4 LDS stages filled by
//                    direct-to-LDS buffer loads issued 3 stages ahead
//   LDS              64-byte rows, 16-byte chunks XOR-swizzled by row so that
//                    the fragment reads of 8 consecutive rows hit distinct banks
//
// Accumulator layout of one 32x32 MFMA tile (lane l, register r):
//   i = 8*(r/4) + 4*(l/32) + (r%4),   j = l%32
// so a lane owns one B row (j) and 16 A rows.  The forward puts vocabulary
// rows in A and token rows in B: each lane then holds 16 logits of ONE token,
// and the per-token max / sum-exp runs almost entirely inside the lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int TILE = 256;
constexpr int BK = 32;                           // K elements per LDS stage
constexpr int NSTAGE = 4;                        // LDS ring depth
constexpr int HALF_BYTES = TILE * BK * 2;        // one operand of one stage: 16 KB
constexpr int STAGE_BYTES = 2 * HALF_BYTES;      // A then B: 32 KB
constexpr int NT = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

// The operand ring (4 x 32 KB) and, after the K loop, epilogue staging of up
// to 256 x 264 bf16.
struct __align__(16) Smem {
  unsigned char raw[NSTAGE * STAGE_BYTES > TILE * (TILE + 8) * 2 ? NSTAGE * STAGE_BYTES
                                                                 : TILE * (TILE + 8) * 2];
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(unsigned, b);
}
__device__ __forceinline__ u16 to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(u16, b);
}

// Merge two (max, sum-exp) states of the online softmax.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == NEG_INF) return;
  s = s * fast_exp2((m - mn) * LOG2E) + s2 * fast_exp2((m2 - mn) * LOG2E);
  m = mn;
}

// Launch index -> (ta, tb) tile of an nA x nB tile grid.  Workgroups are dealt
// to the 8 XCDs round-robin by launch index, so the launch index is first
// remapped so that each XCD receives a contiguous run of logical tiles; the
// logical order is a grouped raster (GA 'a' tiles, then the next 'b') so the
// workgroups sharing one XCD's L2 share both A and B tiles.  The launch grid
// is padded to a multiple of 8; extra workgroups return false.
// Logical tile index L -> (ta, tb) in the grouped raster described above.
__device__ __forceinline__ void raster_tile(int L, int nA, int nB, int GA, int& ta, int& tb) {
  const int ga = GA < nA ? GA : nA;
  const int group = L / (ga * nB);
  const int first = group * ga;
  const int gsize = (nA - first) < ga ? (nA - first) : ga;
  const int idx = L - group * ga * nB;
  ta = first + idx % gsize;
  tb = idx / gsize;
}

__device__ __forceinline__ bool map_tile(int bid, int nlaunch, int nA, int nB, int GA,
                                         int& ta, int& tb) {
  const int n = nA * nB;
  const int per = nlaunch >> 3;
  const int L = (bid & 7) * per + (bid >> 3);
  if (L >= n) return false;
  const int ga = GA < nA ? GA : nA;
  const int group = L / (ga * nB);
  const int first = group * ga;
  const int gsize = (nA - first) < ga ? (nA - first) : ga;
  const int idx = L - group * ga * nB;
  ta = first + idx % gsize;
  tb = idx / gsize;
  return true;
}

// Buffer resource over [base, base + bytes): loads whose (range-checked) VGPR
// offset falls past the end return zero.  The scalar offset is always 0.
// base and bytes are workgroup-uniform (kernel arguments and blockIdx only);
// readfirstlane states that, so the descriptor lives in SGPRs and the loads
// need no per-lane waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  void* pu = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// ---------------------------------------------------------------------------
// LDS layout of one operand of one stage: 256 rows x 64 bytes (32 bf16 of K).
// Row r's 16-byte chunk c (K elements 8c .. 8c+7) sits at position
// c ^ swz(r) of the row, with
//   swz(r) = ((r1 ^ r2) | (r2 ^ r3) << 1)   (r1, r2, r3: bits 1..3 of r).
// For one chunk index, 8 consecutive rows (from a multiple of 8) land in 8
// distinct 16-byte bank groups of 32 banks, and 16 consecutive rows (from a
// multiple of 16) in 16 distinct groups of 64 banks, so the fragment reads are
// conflict-free whether the LDS serves 8 or 16 lanes of a 16-byte read per
// clock.  swz depends only on row bits 1..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) ^ (row >> 2)) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ lds_ptr_t to_lds(void* p) { return (lds_ptr_t)(p); }

// Direct-to-LDS loads of one 256 x 32 K-slice of an operand.  Wave w moves
// rows 64w .. 64w+63 with 4 instructions of 16 rows; in each, lane L fills LDS
// bytes 16L .. 16L+15 (row 16p + L/4 of the instruction, position L%4), so it
// fetches global chunk (L%4) ^ swz(row).
//
// Row-major operand (leading dimension ld): the buffer resource ends at row
// rows_valid, so rows past it read as zero, and so does a chunk at k >= K
// (K tail, K % 8 == 0), which is pointed past the resource.
//
// BLOCKED operand: the tile is stored as K/32 consecutive 16 KB blocks, block b
// holding rows 0..255 x K elements 32b .. 32b+31 row-major (64 bytes a row),
// so each K-slice is one contiguous 16 KB read.  Every row is valid and
// K % 32 == 0 (the workspace matrices the library writes itself).
template <bool KTAIL, bool BLOCKED = false>
struct DmaOperand {
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;     // byte offset of this lane's chunk for instruction 0 at k = 0
  int pstride;  // bytes between instructions (16 rows)
  int c8;       // this lane's chunk index * 8 (K elements)
  int K;

  __device__ __forceinline__ void init(const u16* base, int ld, int rows, int K_, int lane, int w) {
    // row bits 0..3 are lane bits 2..5, so swz(row) = swz(lane >> 2) for every instruction
    const int c = (lane & 3) ^ swz(lane >> 2);
    const int row0 = 64 * w + (lane >> 2);
    if (BLOCKED) {
      rsrc = make_rsrc(base, (unsigned)(K_ >> 5) * 16384u);
      voff = row0 * 64 + c * 16;
      pstride = 16 * 64;
    } else {
      rsrc = make_rsrc(base, (unsigned)(rows > 0 ? rows : 0) * (unsigned)ld * 2u);
      voff = row0 * ld * 2 + c * 16;
      pstride = 16 * ld * 2;
    }
    c8 = c * 8;
    K = K_;
  }

  // Issue the 4 loads of K-slice k0 into the operand region `dst` of a stage.
  __device__ __forceinline__ void issue(int k0, unsigned char* dst, int w) const {
    const bool kv = BLOCKED || !KTAIL || k0 + c8 < K;
    const int kb = BLOCKED ? k0 * 512 : k0 * 2;  // bytes to slice k0 (a 16 KB block per 32 of K)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int off = kv ? voff + p * pstride + kb : 0x7ffffff0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, to_lds(dst + (64 * w + 16 * p) * 64), 16, off,
                                               0, 0, 0);
    }
  }
};

// Element-by-element loads of one K-slice into the same swizzled layout (the
// path for odd D or 16-byte-misaligned operands; not pipelined).
__device__ __forceinline__ void slow_slice(const u16* __restrict__ base, int ld, int rows_valid,
                                           int K, int k0, unsigned char* dst, int tid) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = tid + 256 * p;  // 1024 chunks: row idx/4, chunk idx%4
    const int row = idx >> 2, c = idx & 3;
    const int k = k0 + c * 8;
    unsigned e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      e[q] = (row < rows_valid && k + q < K) ? base[(size_t)row * ld + k + q] : 0u;
    *reinterpret_cast<u32x4*>(dst + row * 64 + ((c ^ swz(row)) << 4)) =
        u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
  }
}

// Fragments of one 16-wide K sub-step: 4 A tiles and 4 B tiles of 32 rows.
struct Frags {
  bf16x8 a[4], b[4];
};

// Per-lane byte offsets of the fragment rows inside a stage.
struct FragAddr {
  int a, b;    // row part of the A / B addresses (tile 0)
  int k0, k1;  // chunk part for sub-step 0 (K 0..15) and sub-step 1 (K 16..31)
  __device__ __forceinline__ void init(int lane, int wi, int wj) {
    const int r = lane & 31, half = lane >> 5;
    const int sw = swz(r);  // swz of every row this lane reads (rows r + 32 i + 128 wi)
    a = (wi * 128 + r) * 64;
    b = HALF_BYTES + (wj * 128 + r) * 64;
    k0 = (half ^ sw) << 4;
    k1 = ((2 + half) ^ sw) << 4;
  }
};

__device__ __forceinline__ void load_frags(const unsigned char* stage, const FragAddr& fa, int kpart,
                                           Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(stage + fa.a + i * 32 * 64 + kpart);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(stage + fa.b + j * 32 * 64 + kpart);
}

__device__ __forceinline__ void mma_16(const Frags& f, floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void zero_acc(floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
#define CCE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// Workgroup barrier for the operand ring: waits for this wave's LDS reads
// (lgkmcnt 0) but not for its in-flight direct-to-LDS loads; the caller has
// already waited (CCE_WAIT_VMCNT) for the loads whose data the next reads
// need.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt / expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling hints: interleave `n` instructions of class `mask` one by one
// with MFMAs, so that in-order issue never blocks the MFMA pipe behind a burst
// of memory instructions.  (mask: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read.)
#define CCE_INTERLEAVE(mask, n)                           \
  _Pragma("unroll") for (int _q = 0; _q < (n); ++_q) {    \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    \
    __builtin_amdgcn_sched_group_barrier((mask), 1, 0);   \
  }

// acc = A[0:256, 0:K] . B[0:256, 0:K]^T for the operand tiles at A and B
// (leading dimensions lda, ldb; rows beyond a_rows / b_rows are zero; with
// BLOCKED both tiles are in the blocked layout of DmaOperand and lda / ldb /
// a_rows / b_rows are unused).
// SKIP: kflags[kb * kflag_stride] == 0 marks 256-wide K block kb inactive; its
// MFMAs are skipped (its slices still stream through LDS).
//
// VEC path, iteration kt (slice kt sits in stage kt % 4):
//   issue the direct-to-LDS loads of slice kt+3 into stage (kt+3) % 4 (last
//     read in iteration kt-1, before the barrier that ended it)
//   sub-step 0: 16 MFMAs on fragments read earlier, interleaved with those
//     loads and the LDS reads of sub-step 1's fragments
//   wait until this wave's loads of slice kt+1 have landed, then barrier
//   sub-step 1: 16 MFMAs interleaved with the reads of slice kt+1's first
//     fragments
// Slices past the last one are clamped to it (their stages are no longer
// read); the loop ends by draining every load and a barrier, so LDS is free.
template <bool VEC, bool SKIP, bool KTAIL, bool BLOCKED = false>
__device__ __forceinline__ void gemm_tile(const u16* __restrict__ A, int lda, int a_rows,
                                          const u16* __restrict__ B, int ldb, int b_rows, int K,
                                          const int* __restrict__ kflags, int kflag_stride,
                                          Smem& sm, floatx16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wi = w & 1, wj = w >> 1;
  zero_acc(acc);
  FragAddr fa;
  fa.init(lane, wi, wj);
  unsigned char* ring = sm.raw;
  const int nk = (K + BK - 1) / BK;
  if (VEC) {
    DmaOperand<KTAIL, BLOCKED> da, db;
    da.init(A, lda, a_rows, K, lane, w);
    db.init(B, ldb, b_rows, K, lane, w);
    const int klast = (nk - 1) * BK;
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s) {
      const int k = min(s * BK, klast);
      da.issue(k, ring + s * STAGE_BYTES, w);
      db.issue(k, ring + s * STAGE_BYTES + HALF_BYTES, w);
    }
    CCE_WAIT_VMCNT(16);  // slice 0 landed (slices 1 and 2 may be in flight)
    ring_barrier();
    Frags f0, f1;
    load_frags(ring, fa, fa.k0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      unsigned char* cur = ring + (kt & (NSTAGE - 1)) * STAGE_BYTES;
      unsigned char* nxt = ring + ((kt + 1) & (NSTAGE - 1)) * STAGE_BYTES;
      unsigned char* far = ring + ((kt + 3) & (NSTAGE - 1)) * STAGE_BYTES;
      const bool active = !SKIP || kflags[(size_t)((kt * BK) / TILE) * kflag_stride] != 0;
      // sub-step 0
      const int kn = min((kt + 3) * BK, klast);
      da.issue(kn, far, w);
      db.issue(kn, far + HALF_BYTES, w);
      load_frags(cur, fa, fa.k1, f1);
      if (active) mma_16(f0, acc);
      CCE_INTERLEAVE(0x020, 8)
      CCE_INTERLEAVE(0x100, 8)
      CCE_WAIT_VMCNT(16);  // slice kt+1 landed (slices kt+2, kt+3 may be in flight)
      ring_barrier();
      // sub-step 1
      load_frags(nxt, fa, fa.k0, f0);
      if (active) mma_16(f1, acc);
      CCE_INTERLEAVE(0x100, 8)
    }
    CCE_WAIT_VMCNT(0);
    __syncthreads();
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const bool active = !SKIP || kflags[(size_t)((kt * BK) / TILE) * kflag_stride] != 0;
      __syncthreads();
      slow_slice(A, lda, a_rows, K, kt * BK, ring, tid);
      slow_slice(B, ldb, b_rows, K, kt * BK, ring + HALF_BYTES, tid);
      __syncthreads();
      Frags f;
      load_frags(ring, fa, fa.k0, f);
      if (active) mma_16(f, acc);
      load_frags(ring, fa, fa.k1, f);
      if (active) mma_16(f, acc);
    }
    __syncthreads();
  }
}

}  // namespace cce
