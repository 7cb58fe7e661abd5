// Device-side building blocks of the flash-CCE head for gfx950 (CDNA4).
//
// One GEMM core serves every contraction of the head.  Both operands are
// row-major with K contiguous ("NT"): C[i][j] = sum_k A[i][k] * B[j][k].
//
//   workgroup tile   256 (A rows) x 256 (B rows), 256 threads = 4 waves
//   wave tile        128 x 128 = 4 x 4 MFMA tiles of 32x32, fp32 accumulators
//   MFMA             v_mfma_f32_32x32x16_bf16 (8 bf16 of K per lane)
//   K pipeline       64 bf16 per stage, two LDS stages, global loads for
//                    stage k+2 in flight while stage k is multiplied
//   LDS              rows padded to 144 B so that the 16-byte fragment reads of
//                    32 consecutive rows hit distinct banks
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
constexpr int BK = 64;
constexpr int PITCH = BK + 8;
constexpr int NT = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

struct __align__(16) Smem {
  u16 a[2][TILE][PITCH];
  u16 b[2][TILE][PITCH];
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

// ---------------------------------------------------------------------------
// global -> register -> LDS staging of one 256 x 64 K-slice of an operand
// ---------------------------------------------------------------------------
// Thread t moves rows (t/8) + 32p, p = 0..7, bytes 16*(t%8) .. +15 of the
// slice.  Rows >= rows_valid and columns >= K read as zero.
//
// VEC (K % 8 == 0, 16-byte aligned rows): raw buffer loads over a resource
// that ends at row rows_valid, so rows past it read as zero in hardware with
// no branch (every byte offset is in the range-checked VGPR offset).  Only a K tail
// (K % 64 != 0) needs a per-chunk select.  Otherwise elements are loaded one
// by one with explicit bounds checks (a slow path for odd D).
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

template <bool VEC, bool KTAIL>
struct SliceLoader {
  const u16* base;
  int ld;
  int rows_valid;
  int K;
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;     // byte offset of this thread's first chunk at k = 0
  int rstride;  // bytes between this thread's rows (32 rows)
  u32x4 r[8];

  __device__ __forceinline__ void init(const u16* b, int ld_, int rows, int K_, int tid) {
    base = b;
    ld = ld_;
    rows_valid = rows;
    K = K_;
    if (VEC) {
      rsrc = make_rsrc(b, (unsigned)(rows > 0 ? rows : 0) * (unsigned)ld_ * 2u);
      voff = ((tid >> 3) * ld_ + (tid & 7) * 8) * 2;
      rstride = 32 * ld_ * 2;
    }
  }

  // Issues the loads of K-slice k0 (one global load per row this thread moves).
  __device__ __forceinline__ void load(int k0, int tid) {
    if (VEC) {
      // the whole offset rides in the VGPR offset (always range-checked);
      // the scalar offset stays 0.  A chunk at k >= K (K tail, K % 8 == 0) is
      // pointed past the resource so that it reads as zero.
      const bool kv = !KTAIL || k0 + (tid & 7) * 8 < K;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int off = kv ? voff + p * rstride + k0 * 2 : 0x7ffffff0;
        r[p] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      }
    } else {
      const int k = k0 + (tid & 7) * 8;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int row = (tid >> 3) + 32 * p;
        unsigned e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          e[q] = (row < rows_valid && k + q < K) ? base[(size_t)row * ld + k + q] : 0u;
        r[p] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                     e[6] | (e[7] << 16)};
      }
    }
  }

  __device__ __forceinline__ void store(u16 (*s)[PITCH], int tid) const {
    const int c = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < 8; ++p)
      *reinterpret_cast<u32x4*>(&s[(tid >> 3) + 32 * p][c]) = r[p];
  }
};

// Fragments of one 16-wide K sub-step: 4 A tiles and 4 B tiles of 32 rows.
struct Frags {
  bf16x8 a[4], b[4];
};

__device__ __forceinline__ void load_frags(const u16 (*sa)[PITCH], const u16 (*sb)[PITCH], int kk,
                                           int wi, int wj, int lane, Frags& f) {
  const int r = lane & 31;
  const int kh = (lane >> 5) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(&sa[wi * 128 + i * 32 + r][kk + kh]);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(&sb[wj * 128 + j * 32 + r][kk + kh]);
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

// Scheduling hints: interleave `n` instructions of class `mask` one by one
// with MFMAs, so that in-order issue never blocks the MFMA pipe behind a burst
// of memory instructions.  (mask: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read,
// 0x200 DS write.)
#define CCE_INTERLEAVE(mask, n)                           \
  _Pragma("unroll") for (int _q = 0; _q < (n); ++_q) {    \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    \
    __builtin_amdgcn_sched_group_barrier((mask), 1, 0);   \
  }

// acc = A[0:256, 0:K] . B[0:256, 0:K]^T for the operand tiles at A and B
// (leading dimensions lda, ldb; rows beyond a_rows / b_rows are zero).
// SKIP: kflags[kb * kflag_stride] == 0 marks 256-wide K block kb inactive; its
// MFMAs are skipped (the stage still streams through LDS).
//
// Schedule of iteration kt (stage cur = kt % 2 is multiplied):
//   sub-step 0..2: 16 MFMAs each, interleaved with the LDS reads of the next
//                  sub-step's fragments; sub-step 2 also writes K-slice kt+1
//                  (held in registers) into stage cur^1, which every wave
//                  finished reading before the previous iteration's barrier
//   barrier        (stage cur^1 now holds slice kt+1 for everyone)
//   sub-step 3:    16 MFMAs interleaved with the reads of slice kt+1's first
//                  fragments and the global loads of slice kt+2
// so each iteration is a single basic block and no LDS latency is exposed.
// Past the last slice the loads re-read the last slice and the stores write
// a stage nobody reads again; both are harmless.
template <bool VEC, bool SKIP, bool KTAIL>
__device__ __forceinline__ void gemm_tile(const u16* __restrict__ A, int lda, int a_rows,
                                          const u16* __restrict__ B, int ldb, int b_rows, int K,
                                          const int* __restrict__ kflags, int kflag_stride,
                                          Smem& sm, floatx16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wi = w & 1, wj = w >> 1;
  zero_acc(acc);
  SliceLoader<VEC, KTAIL> la, lb;
  la.init(A, lda, a_rows, K, tid);
  lb.init(B, ldb, b_rows, K, tid);
  const int nk = (K + BK - 1) / BK;
  const int klast = (nk - 1) * BK;
  la.load(0, tid);
  lb.load(0, tid);
  la.store(sm.a[0], tid);
  lb.store(sm.b[0], tid);
  la.load(min(BK, klast), tid);
  lb.load(min(BK, klast), tid);
  __syncthreads();
  Frags f0, f1;
  load_frags(sm.a[0], sm.b[0], 0, wi, wj, lane, f0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool active = !SKIP || kflags[(size_t)((kt * BK) / TILE) * kflag_stride] != 0;
    // sub-step 0
    load_frags(sm.a[cur], sm.b[cur], 16, wi, wj, lane, f1);
    if (active) mma_16(f0, acc);
    CCE_INTERLEAVE(0x100, 8)
    // sub-step 1
    load_frags(sm.a[cur], sm.b[cur], 32, wi, wj, lane, f0);
    if (active) mma_16(f1, acc);
    CCE_INTERLEAVE(0x100, 8)
    // sub-step 2 (+ slice kt+1 into the other stage)
    load_frags(sm.a[cur], sm.b[cur], 48, wi, wj, lane, f1);
    la.store(sm.a[cur ^ 1], tid);
    lb.store(sm.b[cur ^ 1], tid);
    if (active) mma_16(f0, acc);
    CCE_INTERLEAVE(0x100, 4)
    CCE_INTERLEAVE(0x300, 12)
    __syncthreads();
    // sub-step 3 (+ first fragments of slice kt+1, global loads of slice kt+2)
    load_frags(sm.a[cur ^ 1], sm.b[cur ^ 1], 0, wi, wj, lane, f0);
    const int kn = min((kt + 2) * BK, klast);
    la.load(kn, tid);
    lb.load(kn, tid);
    if (active) mma_16(f1, acc);
    CCE_INTERLEAVE(0x120, 16)
  }
}

}  // namespace cce
