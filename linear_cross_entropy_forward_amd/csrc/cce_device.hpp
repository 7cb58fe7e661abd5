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

// The operand ring (4 x 32 KB); epilogues reuse it after the K loop.
struct __align__(16) Smem {
  unsigned char raw[NSTAGE * STAGE_BYTES];
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
// The work-item index, opaque to the optimiser: values derived from it are
// computed where they are used rather than hoisted to the top of the kernel,
// where they would stay live through the K loops and be spilled.
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

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

// tanh(z / cap) for the final-logit softcap, as 1 - 2 / (e^{2z/cap} + 1) with
// k2 = 2 log2(e) / cap: one exp2 and one reciprocal, exact limits +-1 at
// +-infinity, absolute error about 1e-7 (the cancellation near 0 costs
// relative, not absolute, accuracy).
__device__ __forceinline__ float tanh_scaled(float z, float k2) {
  const float e = fast_exp2(z * k2);
  return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
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
// remapped (xcd_task) so that each XCD receives a contiguous run of logical
// tiles; the logical order is a grouped raster (GA 'a' tiles, then the next
// 'b'; raster_tile) so the workgroups sharing one XCD's L2 share both A and B
// tiles.  The launch grid is padded to a multiple of 8; extra workgroups
// return false.
__device__ __forceinline__ int xcd_task(int bid, int nlaunch) {
  return (bid & 7) * (nlaunch >> 3) + (bid >> 3);
}

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
  const int L = xcd_task(bid, nlaunch);
  if (L >= nA * nB) return false;
  raster_tile(L, nA, nB, GA, ta, tb);
  return true;
}

// Buffer descriptor over [base, base + bytes), as the 4 dwords the buffer
// instructions take: 48-bit base, stride 0 (raw buffer: offsets are bytes),
// num_records = bytes, and dword 3 = 32-bit data format (untyped loads ignore
// it).  Loads whose range-checked VGPR offset falls past the end return zero.
// base and bytes are workgroup-uniform (kernel arguments, blockIdx and loop
// counters only); readfirstlane states that, so the descriptor lives in SGPRs
// and the loads need no per-lane waterfall loop.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
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

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(void* p) {
  return (unsigned)(uintptr_t)(lds_ptr_t)(p);
}

// One direct-to-LDS load (buffer_load_dwordx4 ... lds): lane L's 16 bytes at
// buffer offset voff land at LDS byte m0 + 16 L (m0 wave-uniform).  It is
// written as assembly so that the compiler does not count it as an LDS store:
// otherwise every LDS read it cannot prove disjoint from the stage being
// filled gets a wait for ALL loads in flight, which drains the operand
// pipeline each K step.  The order between these loads and the LDS reads of
// their data is kept explicitly (CCE_WAIT_VMCNT, then a barrier).  s_nop
// covers the M0 write-to-use hazard.  soff (wave-uniform, an SGPR) is added to
// the address but takes no part in the buffer's range check, so it carries
// only offsets that keep a valid row inside its row (the K offset of a slice):
// the per-lane offsets then stay the same for every slice and stay in
// registers across the loop.
__device__ __forceinline__ void dma16(const i32x4& rsrc, int voff, unsigned m0, int soff) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(m0), "s"(soff)
               : "m0");
}

// ---------------------------------------------------------------------------
// Operand storage.  The core contracts two 256-row operand tiles over K; each
// operand is read from global memory in one of four forms:
//
//   OP_ROW   row-major [i][k] (K contiguous), leading dimension ld; rows
//            i >= rows read as zero, and so does a K tail (K % 8 == 0)
//   OP_BLK   one blocked tile: K/32 consecutive 16 KB blocks, block b holding
//            rows 0..255 x k = 32b .. 32b+31 row-major (64 bytes a row);
//            K % 32 == 0, every row valid (workspace the library writes)
//   OP_KROW  the operand transposed, row-major [k][i] with pitch ld: element
//            (i, k) at base[k * ld + i]; k >= rows or i >= cols read as zero
//   OP_KBLK  the operand is the transpose of a blocked matrix X (256 x 32
//            blocks, ld = blocks per 256-row tile of X): i runs over the 256
//            columns of one column tile of X (base points at its first block),
//            k over the rows of X
//
// Row forms land in LDS as [256 rows][64 bytes] with 16-byte chunk c of row r
// at position c ^ swz(r) (above).  K forms land as [32 k-rows][512 bytes]:
// chunk c (i = 8c .. 8c+7) of k-row kr at position c ^ kswz(kr), and their
// MFMA fragments are read with the transposing LDS read (ds_read_b64_tr_b16).
// ---------------------------------------------------------------------------
enum : int { OP_ROW = 0, OP_BLK = 1, OP_KROW = 2, OP_KBLK = 3 };

// Chunk swizzle of the K forms, by k-row modulo 4: 0, 6, 12, 10.  The
// transposing fragment read makes each 16-lane group read 4 consecutive
// k-rows x 32 bytes (and each 32 lanes 4 k-rows x 64 bytes); this XOR puts
// those pieces in distinct banks for 32 or 64 banks of 4 bytes.
__device__ __forceinline__ int kswz(int kr) { return (0xAC60 >> (4 * (kr & 3))) & 15; }

struct OpRef {
  const u16* p;
  int ld, rows, cols;
};

// Direct-to-LDS loads of one K-slice of an operand: wave w issues 4
// instructions p, each filling 1 KB of the operand's 16 KB stage region; lane
// L of instruction p writes LDS bytes (64w + 16p) * 64 + 16 L and chooses its
// global chunk so that the layouts above come out.
//   row forms: row 64w + 16p + L/4, position L%4 -> chunk (L%4) ^ swz(row)
//   K forms:   k-row 8w + 2p + L/32, position L%32 -> chunk (L%32) ^ kswz(k-row)
// Loads past a buffer resource's end read zero; an invalid chunk is pointed
// past the end.  K forms rebase their resource every slice so that no offset
// exceeds 32 bits whatever the matrix size.
//
// NRW (row forms only): operand rows per wave, 64 (a 256-row tile) or 96 (the
// 384-row A operand of the tall tile below); wave w then fills rows
// NRW w .. NRW w + NRW - 1 with NRW / 16 instructions.
template <int MODE, bool KTAIL, int NRW = 64>
struct DmaOperand {
  i32x4 rsrc;  // row forms: over the whole tile
  const u16* base;
  int ld, rows;
  int voff[2];  // byte offset of this lane's chunk (row forms: [0]; K forms: even / odd p)
  int pstride;  // bytes between instructions (row forms) or instruction pairs (K forms)
  int c8;       // row forms: this lane's chunk index * 8 (K elements)
  int K;
  unsigned ldsw;  // LDS bytes before this wave's first instruction (4 KB per wave)

  __device__ __forceinline__ void init(const OpRef& op, int K_, int lane, int w) {
    base = op.p;
    ld = op.ld;
    rows = op.rows;
    K = K_;
    ldsw = (unsigned)__builtin_amdgcn_readfirstlane(w * NRW * 64);
    if (MODE == OP_ROW || MODE == OP_BLK) {
      // row bits 0..3 are lane bits 2..5, so swz(row) = swz(lane >> 2) for every instruction
      const int c = (lane & 3) ^ swz(lane >> 2);
      const int row0 = NRW * w + (lane >> 2);
      if (MODE == OP_BLK) {
        rsrc = make_rsrc(op.p, (unsigned)(K_ >> 5) * 16384u);
        voff[0] = row0 * 64 + c * 16;
        pstride = 16 * 64;
      } else {
        rsrc = make_rsrc(op.p, (unsigned)(op.rows > 0 ? op.rows : 0) * (unsigned)op.ld * 2u);
        voff[0] = row0 * op.ld * 2 + c * 16;
        pstride = 16 * op.ld * 2;
      }
      voff[1] = 0;
      c8 = c * 8;
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kr = 8 * w + 2 * e + (lane >> 5);
        const int c = (lane & 31) ^ kswz(kr);
        if (MODE == OP_KROW)
          voff[e] = 8 * c < op.cols ? kr * op.ld * 2 + c * 16 : 0x40000000;
        else
          voff[e] = (c >> 2) * 16384 + kr * 64 + (c & 3) * 16;
      }
      pstride = MODE == OP_KROW ? 4 * op.ld * 2 : 4 * 64;  // instructions p and p+2: 4 k-rows
      c8 = 0;
    }
  }

  // Per-slice state of K-slice k0: the buffer resource the slice's loads use
  // (row forms: the tile's; K forms: rebased at the slice) and, for row
  // forms, whether this lane's chunk is inside K.
  struct Slice {
    i32x4 rs;
    int kb;  // bytes added to every address (wave-uniform: the instruction's SGPR offset)
    bool kv;
  };
  __device__ __forceinline__ Slice slice(int k0) const {
    Slice sl;
    if (MODE == OP_ROW || MODE == OP_BLK) {
      sl.rs = rsrc;
      sl.kb = __builtin_amdgcn_readfirstlane(MODE == OP_BLK ? k0 * 512 : k0 * 2);
      sl.kv = MODE == OP_BLK || !KTAIL || k0 + c8 < K;
    } else {
      const u16* sb;
      unsigned nbytes;
      if (MODE == OP_KROW) {
        const int nr = rows - k0;
        sb = base + (size_t)k0 * ld;
        nbytes = nr <= 0 ? 0u : (unsigned)(nr < BK ? nr : BK) * (unsigned)ld * 2u;
      } else {
        sb = base + (size_t)(k0 >> 8) * ld * 8192 + (size_t)(k0 & 255) * 32;
        nbytes = 8u * 16384u;
      }
      sl.rs = make_rsrc(sb, nbytes);
      sl.kb = 0;
      sl.kv = true;
    }
    return sl;
  }

  // Load instruction p (0..3) of a slice into the operand region of a stage at
  // LDS byte address dst.
  __device__ __forceinline__ void issue(const Slice& sl, unsigned dst, int p) const {
    int off;
    if (MODE == OP_ROW || MODE == OP_BLK)
      off = sl.kv ? voff[0] + p * pstride : 0x7ffffff0;
    else
      off = voff[p & 1] + (p >> 1) * pstride;
    dma16(sl.rs, off, dst + ldsw + p * 1024, sl.kb);
  }

  // All loads of K-slice k0 (4, or NRW / 16 for a row form).
  __device__ __forceinline__ void issue_all(int k0, unsigned dst) const {
    const Slice sl = slice(k0);
#pragma unroll
    for (int p = 0; p < NRW / 16; ++p) issue(sl, dst, p);
  }
};

// Element (i, k) of an operand in any of the forms (the unvectorised path).
template <int MODE>
__device__ __forceinline__ unsigned op_elem(const OpRef& op, int K, int i, int k) {
  if (MODE == OP_ROW) return (i < op.rows && k < K) ? op.p[(size_t)i * op.ld + k] : 0u;
  if (MODE == OP_BLK) return op.p[(size_t)(k >> 5) * 8192 + i * 32 + (k & 31)];
  if (MODE == OP_KROW) return (k < op.rows && i < op.cols) ? op.p[(size_t)k * op.ld + i] : 0u;
  return op.p[((size_t)(k >> 8) * op.ld + (i >> 5)) * 8192 + (k & 255) * 32 + (i & 31)];
}

// Element-by-element loads of one K-slice into the same LDS layout (the path
// for odd D or 16-byte-misaligned operands; not pipelined).
template <int MODE>
__device__ __forceinline__ void slow_slice(const OpRef& op, int K, int k0, unsigned char* dst,
                                           int tid) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = tid + 256 * p;  // 1024 chunks of 16 bytes
    unsigned e[8];
    int at;
    if (MODE == OP_ROW || MODE == OP_BLK) {
      const int row = idx >> 2, c = idx & 3;
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = op_elem<MODE>(op, K, row, k0 + 8 * c + q);
      at = row * 64 + ((c ^ swz(row)) << 4);
    } else {
      const int kr = idx >> 5, c = idx & 31;
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = op_elem<MODE>(op, K, 8 * c + q, k0 + kr);
      at = kr * 512 + ((c ^ kswz(kr)) << 4);
    }
    *reinterpret_cast<u32x4*>(dst + at) =
        u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
  }
}

// Fragments of one 16-wide K sub-step: 4 A tiles and 4 B tiles of 32 rows.
// Lane l holds row l%32 of its tile, K elements 8*(l/32) .. 8*(l/32)+7.
struct Frags {
  bf16x8 a[4], b[4];
};

// Per-lane byte offsets of the fragments inside a stage.
//   row forms: a / b = row part (tile 0); k0 / k1 = chunk part of sub-step 0 / 1
//   K forms:   a / b = address of tile 0, sub-step 0; tile t is at a ^ (t << 6)
//              (the chunk bits the tile index occupies), sub-step 1 at +8192
// K forms, transposing read: in each 16-lane group, source lane s points at
// k-row kr0 + s/4 and i = i0 + 4*(s%4); lane s then receives element
// (i0 + s, kr0 .. kr0+3).  Two reads, 4 k-rows apart, give the lane's 8 K
// elements.  Lanes 16..31 take i0 + 16, lanes 32..63 take K elements 8..15.
template <bool AK, bool BKM>
struct FragAddr {
  int a, b;
  int k0, k1;
  __device__ __forceinline__ void init(int lane, int wi, int wj) {
    const int r = lane & 31, half = lane >> 5;
    const int sw = swz(r);  // swz of every row this lane reads (rows r + 32 i + 128 wi)
    k0 = (half ^ sw) << 4;
    k1 = ((2 + half) ^ sw) << 4;
    const int s = lane & 15, gi = (lane >> 4) & 1;
    const int kr = 8 * half + (s >> 2);
    const int kbase = kr * 512 + (((2 * gi + ((s >> 1) & 1)) ^ kswz(kr)) << 4) + 8 * (s & 1);
    a = AK ? kbase + wi * 256 : (wi * 128 + r) * 64;
    b = HALF_BYTES + (BKM ? kbase + wj * 256 : (wj * 128 + r) * 64);
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 read_tr_frag(const unsigned char* p) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2048));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Fragment i of the A (B) operand for sub-step `sub` of the stage at `stage`.
template <bool AK, bool BKM>
__device__ __forceinline__ bf16x8 frag_a(const unsigned char* stage, const FragAddr<AK, BKM>& fa,
                                         int sub, int i) {
  return AK ? read_tr_frag(stage + ((fa.a ^ (i << 6)) + sub * 8192))
            : *reinterpret_cast<const bf16x8*>(stage + fa.a + i * 32 * 64 + (sub ? fa.k1 : fa.k0));
}
template <bool AK, bool BKM>
__device__ __forceinline__ bf16x8 frag_b(const unsigned char* stage, const FragAddr<AK, BKM>& fa,
                                         int sub, int j) {
  return BKM ? read_tr_frag(stage + ((fa.b ^ (j << 6)) + sub * 8192))
             : *reinterpret_cast<const bf16x8*>(stage + fa.b + j * 32 * 64 + (sub ? fa.k1 : fa.k0));
}

template <bool AK, bool BKM>
__device__ __forceinline__ void load_frags(const unsigned char* stage, const FragAddr<AK, BKM>& fa,
                                           int sub, Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = frag_a(stage, fa, sub, i);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = frag_b(stage, fa, sub, j);
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

// Wait until at most n vector-memory operations of this wave are in flight
// (n a literal).  Assembly, so that the compiler neither drops nor merges it:
// it does not see the direct-to-LDS loads this wait is for.
#define CCE_WAIT_VMCNT(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

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


// Fragment r (0..7) of a sub-step in the order the next sub-step's MFMAs
// consume them: A0, B0, B1, B2, B3, A1, A2, A3.
template <bool AK, bool BKM>
__device__ __forceinline__ void read_frag(const unsigned char* stage, const FragAddr<AK, BKM>& fa,
                                          int sub, int r, Frags& f) {
  if (r == 0) f.a[0] = frag_a(stage, fa, sub, 0);
  else if (r < 5) f.b[r - 1] = frag_b(stage, fa, sub, r - 1);
  else f.a[r - 4] = frag_a(stage, fa, sub, r - 4);
}

// One K step of the pipelined loop (slice kt in stage `cur`; `nxt` holds slice
// kt+1; `far` receives slice kt+3), in a fixed instruction order:
//   sub-step 0: 16 MFMAs (A tile i = q/4, B tile j = q%4) on fragments read
//     earlier; after MFMA q: for even q the LDS read of one of sub-step 1's
//     fragments, for q = 3, 7, 11, 15 one direct-to-LDS load of slice kt+3's
//     A half into `far` (last read in iteration kt-1, before its mid barrier)
//   wait until this wave's loads of slice kt+1 have landed (in flight may be
//     slice kt+2's 8 loads and the 4 just issued), then barrier
//   sub-step 1: 16 MFMAs; after even q the read of one of slice kt+1's first
//     fragments, after q = 3, 7, 11, 15 one load of slice kt+3's B half.
// The loads are spread one per 4 MFMAs: the CU's load path moves 64 bytes a
// clock, and the 4 waves run in step, so bunched loads stall every wave's
// issue (and crowd the LDS reads they share the LDS with).  sched_barrier
// pins the order.
template <int AMODE, int BMODE, bool KTAIL, bool AK, bool BKM>
__device__ __forceinline__ void gemm_step(const DmaOperand<AMODE, KTAIL>& da,
                                          const DmaOperand<BMODE, KTAIL>& db,
                                          const FragAddr<AK, BKM>& fa, int kn,
                                          const unsigned char* cur, const unsigned char* nxt,
                                          unsigned far, Frags& f0, Frags& f1,
                                          floatx16 (&acc)[4][4]) {
  const typename DmaOperand<AMODE, KTAIL>::Slice sa = da.slice(kn);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.a[i], f0.b[j], acc[i][j], 0, 0, 0);
    if ((q & 1) == 0) read_frag(cur, fa, 1, q >> 1, f1);
    else if ((q & 3) == 3) da.issue(sa, far, q >> 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  CCE_WAIT_VMCNT(12);  // slice kt+1 landed (slice kt+2 and half of kt+3 may be in flight)
  ring_barrier();
  const typename DmaOperand<BMODE, KTAIL>::Slice sb = db.slice(kn);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.a[i], f1.b[j], acc[i][j], 0, 0, 0);
    if ((q & 1) == 0) read_frag(nxt, fa, 0, q >> 1, f0);
    else if ((q & 3) == 3) db.issue(sb, far + HALF_BYTES, q >> 2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The pipelined K loop over the 4 ring stages at `ring` (LDS byte address
// ring_lds), unrolled by 4 so that every access names its stage statically
// (constant LDS offsets).  The order between the direct-to-LDS loads and the
// reads of their data is kept by the explicit vmcnt waits and barriers only.
// SKIP (K a multiple of 256): 256-wide K blocks flagged inactive take no
// part.  A tile with every block active takes the regular loop.  With at most
// 64 blocks the active ones form a 64-bit mask and the same pipelined loop
// walks only their slices (a scalar cursor yields the K offset of the slice
// three steps ahead), so an inactive block costs neither loads nor MFMAs.
// With more blocks, a variant streams every slice through the ring and
// branches around each sub-step's 16 MFMAs as a whole (no interleaving, no
// unrolling): control flow between interleaved MFMAs leaves the register
// allocator unable to keep the accumulators in place.
struct SliceCursor {
  unsigned long long m;  // active blocks not yet left behind (current one lowest)
  int cb, cs;            // current block, slice within it
  __device__ __forceinline__ void init(unsigned long long mask) {
    m = mask;
    cb = __builtin_ctzll(mask);
    cs = 0;
  }
  // K offset of the cursor's slice, then advance; past the last active slice
  // it keeps yielding in-range offsets of the last block (stages never read)
  __device__ __forceinline__ int next() {
    const int k = cb * TILE + cs * BK;
    if (++cs == TILE / BK) {
      cs = 0;
      m &= m - 1ull;
      if (m != 0ull) cb = __builtin_ctzll(m);
    }
    return k;
  }
};

// The regular loop over the slices of the active blocks in `mask` only.
template <int AMODE, int BMODE, bool KTAIL, bool AK, bool BKM>
__device__ __forceinline__ void gemm_loop_compact(const DmaOperand<AMODE, KTAIL>& da,
                                                  const DmaOperand<BMODE, KTAIL>& db,
                                                  const FragAddr<AK, BKM>& fa,
                                                  unsigned long long mask,
                                                  const unsigned char* ring, unsigned ring_lds,
                                                  floatx16 (&acc)[4][4]) {
  const int nsl = __builtin_popcountll(mask) * (TILE / BK);
  if (nsl == 0) {  // nothing active: acc stays 0, no load was issued
    __syncthreads();
    return;
  }
  SliceCursor cur;
  cur.init(mask);
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) {
    const int k = cur.next();
    da.issue_all(k, ring_lds + s * STAGE_BYTES);
    db.issue_all(k, ring_lds + s * STAGE_BYTES + HALF_BYTES);
  }
  CCE_WAIT_VMCNT(16);  // slice 0 landed (slices 1 and 2 may be in flight)
  ring_barrier();
  Frags f0, f1;
  load_frags(ring, fa, 0, f0);
  for (int kt0 = 0; kt0 < nsl; kt0 += NSTAGE) {
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j)
      gemm_step(da, db, fa, cur.next(), ring + j * STAGE_BYTES,
                ring + ((j + 1) & 3) * STAGE_BYTES, ring_lds + ((j + 3) & 3) * STAGE_BYTES, f0, f1,
                acc);
  }
  CCE_WAIT_VMCNT(0);
  __syncthreads();
}

template <bool SKIP, int AMODE, int BMODE, bool KTAIL, bool AK, bool BKM>
__device__ __forceinline__ void gemm_loop(const DmaOperand<AMODE, KTAIL>& da,
                                          const DmaOperand<BMODE, KTAIL>& db,
                                          const FragAddr<AK, BKM>& fa, int nk,
                                          const int* __restrict__ kflags, int kflag_stride,
                                          const unsigned char* ring, unsigned ring_lds,
                                          floatx16 (&acc)[4][4]) {
  // The LDS stage addresses are ring_lds plus constants; redefining ring_lds
  // (an empty asm) here and at every unrolled group keeps the compiler from
  // hoisting all of them out of the loops into scalar registers, which pushes
  // other values to scratch, whose reloads then wait for every load in flight.
  asm volatile("" : "+s"(ring_lds));
  bool all_active = true;
  if (SKIP) {
    // one pass over the tile's K-block flags (lanes stride over the blocks),
    // before any direct-to-LDS load is in flight
    const int nkb = (nk * BK + TILE - 1) / TILE;
    const int lane = (int)(threadIdx.x & 63);
    if (nkb <= 64) {
      const bool on = lane < nkb && kflags[(size_t)lane * kflag_stride] != 0;
      const unsigned long long mask = __ballot(on);
      if (__builtin_popcountll(mask) != nkb) {
        gemm_loop_compact(da, db, fa, mask, ring, ring_lds, acc);
        return;
      }
    } else {
      bool lane_ok = true;
      for (int kb = lane; kb < nkb; kb += 64) lane_ok &= kflags[(size_t)kb * kflag_stride] != 0;
      all_active = __ballot(!lane_ok) == 0ull;
    }
  }
  const int klast = (nk - 1) * BK;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) {
    const int k = min(s * BK, klast);
    da.issue_all(k, ring_lds + s * STAGE_BYTES);
    db.issue_all(k, ring_lds + s * STAGE_BYTES + HALF_BYTES);
  }
  CCE_WAIT_VMCNT(16);  // slice 0 landed (slices 1 and 2 may be in flight)
  ring_barrier();
  Frags f0, f1;
  load_frags(ring, fa, 0, f0);
  if (SKIP && !all_active) {
    for (int kt = 0; kt < nk; ++kt) {
      const unsigned char* cur = ring + (kt & 3) * STAGE_BYTES;
      const unsigned char* nxt = ring + ((kt + 1) & 3) * STAGE_BYTES;
      const unsigned far = ring_lds + ((kt + 3) & 3) * STAGE_BYTES;
      const bool active = kflags[(size_t)((kt * BK) / TILE) * kflag_stride] != 0;
      const int kn = min((kt + 3) * BK, klast);
      da.issue_all(kn, far);
      db.issue_all(kn, far + HALF_BYTES);
      load_frags(cur, fa, 1, f1);
      if (active) mma_16(f0, acc);
      CCE_WAIT_VMCNT(16);
      ring_barrier();
      load_frags(nxt, fa, 0, f0);
      if (active) mma_16(f1, acc);
    }
    CCE_WAIT_VMCNT(0);
    __syncthreads();
    return;
  }
  for (int kt0 = 0; kt0 < nk; kt0 += NSTAGE) {
    asm volatile("" : "+s"(ring_lds));
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j) {
      const int kt = kt0 + j;
      if (kt < nk)
        gemm_step(da, db, fa, min((kt + 3) * BK, klast), ring + j * STAGE_BYTES,
                  ring + ((j + 1) & 3) * STAGE_BYTES, ring_lds + ((j + 3) & 3) * STAGE_BYTES, f0,
                  f1, acc);
    }
  }
  CCE_WAIT_VMCNT(0);
  __syncthreads();
}

// acc = A[0:256, 0:K] . B[0:256, 0:K]^T for the operand tiles A and B, each in
// the form AMODE / BMODE (KTAIL: a row-form operand may end inside a K-slice).
// SKIP: kflags[kb * kflag_stride] == 0 marks 256-wide K block kb inactive (K
// a multiple of 256); it takes no part (see gemm_loop).
// VEC: the pipelined loop above (slice kt sits in stage kt % 4; slices past
// the last one are clamped to it, their stages no longer read); it ends by
// draining every load and a barrier, so LDS is free.  Otherwise one slice at
// a time through element loads.
template <bool VEC, bool SKIP, bool KTAIL, int AMODE = OP_ROW, int BMODE = OP_ROW>
__device__ __forceinline__ void gemm_tile(const OpRef& A, const OpRef& B, int K,
                                          const int* __restrict__ kflags, int kflag_stride,
                                          Smem& sm, floatx16 (&acc)[4][4]) {
  constexpr bool AK = AMODE >= OP_KROW, BKM = BMODE >= OP_KROW;
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wi = w & 1, wj = w >> 1;
  zero_acc(acc);
  FragAddr<AK, BKM> fa;
  fa.init(lane, wi, wj);
  unsigned char* ring = sm.raw;
  const int nk = (K + BK - 1) / BK;
  if (VEC) {
    DmaOperand<AMODE, KTAIL> da;
    DmaOperand<BMODE, KTAIL> db;
    da.init(A, K, lane, w);
    db.init(B, K, lane, w);
    gemm_loop<SKIP>(da, db, fa, nk, kflags, kflag_stride, ring, lds_addr(ring), acc);
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const bool active = !SKIP || kflags[(size_t)((kt * BK) / TILE) * kflag_stride] != 0;
      __syncthreads();
      slow_slice<AMODE>(A, K, kt * BK, ring, tid);
      slow_slice<BMODE>(B, K, kt * BK, ring + HALF_BYTES, tid);
      __syncthreads();
      Frags f;
      load_frags(ring, fa, 0, f);
      if (active) mma_16(f, acc);
      load_frags(ring, fa, 1, f);
      if (active) mma_16(f, acc);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Tall tile: A 384 rows x B 256 rows, K % 32 == 0 (TallForms below: both
// row-major for the forward and the recompute, A = vocabulary rows and B =
// token rows; A the transposed gradient buffer and B K-major for dW).
//
// The core loop above is bound by the operand stream through each CU (bytes
// per MFMA), not by the MFMAs.  A 384 x 256 tile needs 40 KB per 32-wide
// K-slice for 1.5x the MFMAs of a 256 x 256 tile (32 KB): 17 % fewer operand
// bytes per FLOP.  Each wave owns 192 x 128 = 6 x 4 MFMA tiles, 384 fp32
// accumulators a lane: A tiles 0..3 live in the 256 AGPRs (the compiler's
// MFMA form) and A tiles 4..5 in 128 VGPRs, whose MFMAs are written as
// assembly (the compiler picks one register file for all of its MFMAs).
//
// The compiler does not see inside that assembly, so the MFMA hazards that
// concern it are covered by hand: the accumulators pass through an s_nop
// statement that names them as operands after they are zeroed (VALU write ->
// MFMA read of SrcC) and after the K loop (MFMA write -> VALU read; 8-pass
// MFMA: 11 wait states, 24 given).  Within the loop an accumulator is only
// touched by its own MFMA, 24 MFMAs apart, and the A / B fragments come from
// LDS reads, which the compiler's waitcnt insertion orders before the MFMAs
// that read them (a VALU write of a fragment register would need 2 wait states
// before such an MFMA; the generated code is checked to have none).
//
// LDS: 4 stages of 40 KB (A 24 KB then B 16 KB), the whole 160 KB; the
// layouts, the swizzle and the order of the K step are those of the core loop,
// with 24 MFMAs and 10 fragment reads per sub-step, the 6 A loads of a slice in
// sub-step 0 and its 4 B loads in sub-step 1.
// ---------------------------------------------------------------------------
constexpr int TALL = 384;
constexpr int TALL_A_BYTES = TALL * BK * 2;            // 24 KB
constexpr int TALL_STAGE = TALL_A_BYTES + HALF_BYTES;  // 40 KB

struct __align__(16) SmemTall {
  unsigned char raw[NSTAGE * TALL_STAGE];
};

struct AccTall {
  floatx16 a[4][4];  // A tiles 0..3 of the wave (AGPRs)
  floatx16 v[2][4];  // A tiles 4..5 (VGPRs)
};

struct FragsTall {
  bf16x8 a[6], b[4];
};

// acc += a . b^T on one 32x32x16 MFMA with the accumulator in VGPRs.
__device__ __forceinline__ void mfma_vgpr(floatx16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// The VGPR accumulators pass through NOPS wait states here: every access
// before the statement completes before every access after it.
#define CCE_TALL_FENCE(A, NOPS)                                                               \
  asm volatile(NOPS                                                                            \
               : "+v"((A).v[0][0]), "+v"((A).v[0][1]), "+v"((A).v[0][2]), "+v"((A).v[0][3]), \
                 "+v"((A).v[1][0]), "+v"((A).v[1][1]), "+v"((A).v[1][2]), "+v"((A).v[1][3]))

// The zero comes from an assembly statement, so the compiler cannot keep a
// zero vector across the tile loop (it would spill it, and the reload before
// the first MFMA would wait for every operand load in flight).
__device__ __forceinline__ void tall_zero(AccTall& A) {
  float z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) A.a[i][j][r] = z;
#pragma unroll
      for (int i = 0; i < 2; ++i) A.v[i][j][r] = z;
    }
  CCE_TALL_FENCE(A, "s_nop 4");
}

// After the last MFMA of a tile, before any other instruction reads the VGPR
// accumulators.
__device__ __forceinline__ void tall_drain(AccTall& A) {
  CCE_TALL_FENCE(A, "s_nop 7\n\ts_nop 7\n\ts_nop 7");
}

// Per-lane fragment offsets in a tall stage (row forms; see FragAddr).
struct FragAddrTall {
  int a, b, k0, k1;
  __device__ __forceinline__ void init(int lane, int wi, int wj) {
    const int r = lane & 31, half = lane >> 5;
    const int sw = swz(r);  // rows r + 32 i + 192 wi (A) and r + 32 j + 128 wj (B)
    k0 = (half ^ sw) << 4;
    k1 = ((2 + half) ^ sw) << 4;
    a = (wi * 192 + r) * 64;
    b = TALL_A_BYTES + (wj * 128 + r) * 64;
  }
};

// Fragment r (0..9) of a sub-step in the order the next sub-step's MFMAs
// consume them: A0, B0, B1, B2, B3, A1, A2, A3, A4, A5.
__device__ __forceinline__ void tall_read_frag(const unsigned char* stage, const FragAddrTall& fa,
                                               int sub, int r, FragsTall& f) {
  const int kc = sub ? fa.k1 : fa.k0;
  if (r == 0) f.a[0] = *reinterpret_cast<const bf16x8*>(stage + fa.a + kc);
  else if (r < 5) f.b[r - 1] = *reinterpret_cast<const bf16x8*>(stage + fa.b + (r - 1) * 2048 + kc);
  else f.a[r - 4] = *reinterpret_cast<const bf16x8*>(stage + fa.a + (r - 4) * 2048 + kc);
}

__device__ __forceinline__ void tall_mfma(const FragsTall& f, int q, AccTall& acc) {
  const int i = q >> 2, j = q & 3;
  if (i < 4) acc.a[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc.a[i][j], 0, 0, 0);
  else mfma_vgpr(acc.v[i - 4][j], f.a[i], f.b[j]);
}

// Direct-to-LDS loads of one K-slice of a transposed blocked operand (OP_KBLK)
// 384 columns wide (the dW contraction's A = G^T over a tall vocabulary tile):
// the slice (32 k-rows = tokens, 12 blocks of 32 columns = vocabulary) is 12
// pieces of 2 KB, one per block (32 k-rows x 64 bytes, contiguous in G), and
// lands in LDS in the same order: block b's k-row kr at b * 2048 + kr * 64.
// Each load instruction copies 1 KB contiguous (16 k-rows of one block):
// instruction q = 6 w + p (wave w, p = 0..5) takes block q / 2, k-rows
// 16 (q % 2) .. +15.  Within a 64-byte k-row the 16-byte chunk c sits at
// position c ^ swzk(kr) (swzk(kr) = 2 ((kr >> 1) & 1)): the transposing
// fragment read takes 4 consecutive k-rows x 32 bytes per 16 lanes, and with
// this XOR those pieces fall in distinct banks for 32 or 64 banks of 4 bytes.
// Blocks at or past nvb (the tile's valid 32-column blocks) read as zero: the
// resource ends there.
__device__ __forceinline__ int swzk(int kr) { return ((kr >> 1) & 1) << 1; }

struct DmaKblkTall {
  const u16* base;
  int ld;    // blocks per 256-row tile of X
  int nvb;   // valid blocks of this tile (1..12)
  int voff;  // this lane's byte offset: its chunk of wave w's first 1 KB piece
  unsigned ldsw;
  struct Slice {
    i32x4 rs;
  };
  __device__ __forceinline__ void init(const OpRef& op, int, int lane, int w) {
    base = op.p;
    ld = op.ld;
    const int nb = (op.cols + 31) >> 5;
    nvb = nb < 12 ? nb : 12;
    ldsw = (unsigned)__builtin_amdgcn_readfirstlane(w * 6144);
    const int kr = lane >> 2;  // k-row within the 16 of one instruction (kr and kr + 16 share swzk)
    voff = 3 * w * 16384 + kr * 64 + (((lane & 3) ^ swzk(kr)) << 4);
  }
  __device__ __forceinline__ Slice slice(int k0) const {
    Slice sl;
    const u16* sb = base + (size_t)(k0 >> 8) * ld * 8192 + (size_t)(k0 & 255) * 32;
    sl.rs = make_rsrc(sb, (unsigned)nvb * 16384u);
    return sl;
  }
  // instruction p of this wave: block 3 w + p / 2, k-rows 16 (p % 2) ..
  __device__ __forceinline__ void issue(const Slice& sl, unsigned dst, int p) const {
    dma16(sl.rs, voff + (p >> 1) * 16384 + (p & 1) * 1024, dst + ldsw + p * 1024, 0);
  }
  __device__ __forceinline__ void issue_all(int k0, unsigned dst) const {
    const Slice sl = slice(k0);
#pragma unroll
    for (int p = 0; p < 6; ++p) issue(sl, dst, p);
  }
};

// Fragment offsets of the K forms in a tall stage: A (the block-major G^T slice
// of DmaKblkTall; MFMA tile t of wave wi is block 6 wi + t) and B (512-byte
// k-rows, a K-form operand of 256 columns after the A region; tile j at
// b ^ (j << 6)).  The transposing read as in FragAddr: in each 16-lane group,
// lane s points at k-row kr0 + s/4 and column i0 + 4 (s % 4); two reads 4
// k-rows apart give the lane's 8 K elements; lanes 16..31 take i0 + 16, lanes
// 32..63 K elements 8..15 (k-rows + 8).  In A the second read is 256 bytes on,
// tile t at + t * 2048, and sub-step 1 (16 k-rows further) at + 1024 (swzk is
// the same for k-rows 4, 8 and 16 apart).
struct FragAddrKTall {
  int a;  // tile 0, sub-step 0, first read
  int b;
  __device__ __forceinline__ void init(int lane, int wi, int wj) {
    const int s = lane & 15, gi = (lane >> 4) & 1, half = lane >> 5;
    const int kr = 8 * half + (s >> 2);
    const int c0 = 2 * gi + ((s >> 1) & 1);
    a = wi * 6 * 2048 + kr * 64 + ((c0 ^ swzk(kr)) << 4) + 8 * (s & 1);
    b = TALL_A_BYTES + kr * 512 + ((c0 ^ kswz(kr)) << 4) + 8 * (s & 1) + wj * 256;
  }
};

__device__ __forceinline__ bf16x8 read_tr_frag_w(const unsigned char* p, int second) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + second));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Fragment r (0..9) of a K-form tall sub-step, in the consuming order A0, B0..B3, A1..A5.
__device__ __forceinline__ void tall_read_frag(const unsigned char* stage, const FragAddrKTall& fa,
                                               int sub, int r, FragsTall& f) {
  if (r == 0) f.a[0] = read_tr_frag_w(stage + fa.a + sub * 1024, 256);
  else if (r < 5) f.b[r - 1] = read_tr_frag(stage + ((fa.b ^ ((r - 1) << 6)) + sub * 8192));
  else f.a[r - 4] = read_tr_frag_w(stage + fa.a + (r - 4) * 2048 + sub * 1024, 256);
}

// Operand forms of a tall tile: row-major A and B (the forward and the
// recompute), or A = the transpose of a blocked matrix and B K-major (dW).
template <bool KF>
struct TallForms {
  typedef DmaOperand<OP_ROW, false, 96> DA;
  typedef DmaOperand<OP_ROW, false, 64> DB;
  typedef FragAddrTall FA;
};
template <>
struct TallForms<true> {
  typedef DmaKblkTall DA;
  typedef DmaOperand<OP_KROW, false, 64> DB;
  typedef FragAddrKTall FA;
};

// One K step (slice kt in `cur`, kt+1 in `nxt`, kt+3 loaded into `far`):
//   sub-step 0: 24 MFMAs; after even q < 20 one fragment read of sub-step 1,
//     after q = 3, 7, .., 23 one of the 6 A loads of slice kt+3
//   wait for this wave's loads of slice kt+1 (in flight may be slice kt+2's 10
//   and the 6 just issued), barrier
//   sub-step 1: 24 MFMAs; after even q < 20 one read of slice kt+1's first
//     fragments, after q = 5, 11, 17, 23 one of the 4 B loads of slice kt+3.
template <bool KF>
__device__ __forceinline__ void tall_step(const typename TallForms<KF>::DA& da,
                                          const typename TallForms<KF>::DB& db,
                                          const typename TallForms<KF>::FA& fa, int kn,
                                          const unsigned char* cur, const unsigned char* nxt,
                                          unsigned far, FragsTall& f0, FragsTall& f1,
                                          AccTall& acc) {
  const typename TallForms<KF>::DA::Slice sa = da.slice(kn);
#pragma unroll
  for (int q = 0; q < 24; ++q) {
    tall_mfma(f0, q, acc);
    if ((q & 1) == 0 && q < 20) tall_read_frag(cur, fa, 1, q >> 1, f1);
    else if ((q & 3) == 3) da.issue(sa, far, q >> 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  CCE_WAIT_VMCNT(16);  // slice kt+1 landed (slice kt+2 and the A half of kt+3 may be in flight)
  ring_barrier();
  const typename TallForms<KF>::DB::Slice sb = db.slice(kn);
#pragma unroll
  for (int q = 0; q < 24; ++q) {
    tall_mfma(f1, q, acc);
    if ((q & 1) == 0 && q < 20) tall_read_frag(nxt, fa, 0, q >> 1, f0);
    else if (q % 6 == 5) db.issue(sb, far + TALL_A_BYTES, q / 6);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc = A[0:384, 0:K] . B[0:256, 0:K]^T, K % 32 == 0.  !KF: both operands
// 16-byte aligned row-major (rows past A.rows / B.rows read as zero).  KF: A is
// the transpose of a blocked matrix (OP_KBLK; A.cols = valid columns of the
// tile) and B is K-major (OP_KROW), with K a multiple of 256 (whole blocks).
// Ends with every load drained, a barrier (LDS free) and the VGPR accumulators
// readable.
template <bool KF>
__device__ __forceinline__ void gemm_tile_tall(const OpRef& A, const OpRef& B, int K, SmemTall& sm,
                                               AccTall& acc) {
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = tid >> 6;
  tall_zero(acc);
  typename TallForms<KF>::FA fa;
  fa.init(lane, w & 1, w >> 1);
  unsigned char* ring = sm.raw;
  unsigned ring_lds = lds_addr(ring);
  const int nk = K / BK;
  typename TallForms<KF>::DA da;
  typename TallForms<KF>::DB db;
  da.init(A, K, lane, w);
  db.init(B, K, lane, w);
  asm volatile("" : "+s"(ring_lds));
  const int klast = (nk - 1) * BK;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) {
    const int k = min(s * BK, klast);
    da.issue_all(k, ring_lds + s * TALL_STAGE);
    db.issue_all(k, ring_lds + s * TALL_STAGE + TALL_A_BYTES);
  }
  CCE_WAIT_VMCNT(20);  // slice 0 landed (slices 1 and 2 may be in flight)
  ring_barrier();
  FragsTall f0, f1;
#pragma unroll
  for (int r = 0; r < 10; ++r) tall_read_frag(ring, fa, 0, r, f0);
  for (int kt0 = 0; kt0 < nk; kt0 += NSTAGE) {
    asm volatile("" : "+s"(ring_lds));
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j) {
      const int kt = kt0 + j;
      if (kt < nk)
        tall_step<KF>(da, db, fa, min((kt + 3) * BK, klast), ring + j * TALL_STAGE,
                      ring + ((j + 1) & 3) * TALL_STAGE, ring_lds + ((j + 3) & 3) * TALL_STAGE, f0,
                      f1, acc);
    }
  }
  CCE_WAIT_VMCNT(0);
  __syncthreads();
  tall_drain(acc);
}

// ---------------------------------------------------------------------------
// 256 x 256 tile with 64-wide K-slices (row forms, K % 64 == 0).  A load
// instruction covers 8 rows x 128 bytes instead of 16 rows x 64 bytes: half the
// cache lines and L2 requests per byte, which the per-CU operand stream is
// bound by (measured: 8 rows x 128 bytes stream 1.6-1.7x faster than 16 rows x
// 64 bytes at equal bytes).  A stage is 512 rows x 128 bytes (64 KB); the ring
// has two.  Chunk c (16 bytes) of row r sits at position c ^ swz8(r): 8
// consecutive rows (from a multiple of 8), and the 8 rows of each parity among
// 16 consecutive ones, land in distinct 16-byte bank groups for 32 and 64
// banks.  K step (pair of 32-slices s in stage s % 2): four sub-steps of 16
// MFMAs on K 16u .. 16u + 15; during sub-step u the fragments of sub-step u + 1
// are read (u = 3: sub-step 0 of the next stage).  The loads of pair s + 1 go
// into the other stage, free once every wave has read its last fragments of
// pair s - 1: A 0..5 in sub-step 3 of step s - 1, A 6..7 and B 0..5 in
// sub-step 0 and B 6..7 in sub-step 1 of step s; one wait for all of them and a
// barrier separate sub-steps 2 and 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
constexpr int S64_A = TILE * 128;          // 32 KB
constexpr int S64_STAGE = 2 * S64_A;       // 64 KB

// Loads of one 256-row operand of a 64-wide K-slice pair: wave w fills rows
// 64 w .. 64 w + 63 with 8 instructions of 8 rows x 128 bytes; lane L takes row
// L / 8 of the instruction and position L % 8, i.e. global chunk
// (L % 8) ^ swz8(row) (swz8 of rows 64 w + 8 p + L / 8 is L / 8 ^ (p & 1)).
struct Dma128 {
  i32x4 rsrc;
  int voff[2];
  int pstride;
  unsigned ldsw;
  __device__ __forceinline__ void init(const OpRef& op, int lane, int w) {
    rsrc = make_rsrc(op.p, (unsigned)(op.rows > 0 ? op.rows : 0) * (unsigned)op.ld * 2u);
    const int r8 = lane >> 3, pos = lane & 7;
#pragma unroll
    for (int e = 0; e < 2; ++e) voff[e] = (64 * w + r8) * op.ld * 2 + ((pos ^ r8 ^ e) * 16);
    pstride = 8 * op.ld * 2;
    ldsw = (unsigned)__builtin_amdgcn_readfirstlane(w * 64 * 128);
  }
  __device__ __forceinline__ void issue(int k0, unsigned dst, int p) const {
    dma16(rsrc, voff[p & 1] + p * pstride, dst + ldsw + p * 1024,
          __builtin_amdgcn_readfirstlane(k0 * 2));
  }
};

// Per-lane fragment offsets: rows r + 32 i + 128 wi (A) and r + 32 j + 128 wj
// (B) share bits 0..3 with r, so one swizzle serves every tile; sub-step u's
// chunk 2u + half sits at (half ^ swz8(r)) ^ 2u, i.e. the offset kc0 ^ (u << 5).
struct Frag64 {
  int a, b, kc0;
  __device__ __forceinline__ void init(int lane, int wi, int wj) {
    const int r = lane & 31, half = lane >> 5;
    kc0 = (half ^ swz8(r)) << 4;  // sub-step u: kc0 ^ (u << 5)
    a = (wi * 128 + r) * 128 + kc0;
    b = S64_A + (wj * 128 + r) * 128 + kc0;
  }
};

// Fragment r (0..7: A0, B0..B3, A1..A3, the consuming order) of sub-step u.
__device__ __forceinline__ void rd64(const unsigned char* stage, const Frag64& fa, int u, int r,
                                     Frags& f) {
  const int x = u << 5;
  if (r == 0) f.a[0] = *reinterpret_cast<const bf16x8*>(stage + (fa.a ^ x));
  else if (r < 5) f.b[r - 1] = *reinterpret_cast<const bf16x8*>(stage + ((fa.b ^ x) + (r - 1) * 4096));
  else f.a[r - 4] = *reinterpret_cast<const bf16x8*>(stage + ((fa.a ^ x) + (r - 4) * 4096));
}

// 16 MFMAs on fc; after even q the next sub-step's fragment q/2 (stage rs,
// sub-step ru); after odd q load slot l0 + q/2 (A 0..7, B 8..15) of the pair at
// K offset kn into the stage at ldst, for the first nl odd q.
__device__ __forceinline__ void sub64(const Dma128& da, const Dma128& db, const Frag64& fa,
                                      const Frags& fc, Frags& fn, const unsigned char* rs, int ru,
                                      unsigned ldst, int kn, int l0, int nl,
                                      floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.a[i], fc.b[j], acc[i][j], 0, 0, 0);
    if ((q & 1) == 0) {
      rd64(rs, fa, ru, q >> 1, fn);
    } else if ((q >> 1) < nl) {
      const int l = l0 + (q >> 1);
      if (l < 8) da.issue(kn, ldst, l);
      else db.issue(kn, ldst + S64_A, l - 8);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc = A[0:256, 0:K] . B[0:256, 0:K]^T, both row-major and 16-byte aligned,
// K % 64 == 0 (rows past A.rows / B.rows read as zero), through the 128 KB ring
// at `ring`.  Ends with every load drained and a barrier (LDS free).
// The loads of a 64-wide tile's first K-slice pair, into stage 0 of a ring
// that no wave still reads: a persistent caller issues them for its next tile
// right after a tile's K loop, so that they land while it runs that tile's
// epilogue, and then calls gemm_tile64<false>.
__device__ __forceinline__ void gemm_tile64_first(const OpRef& A, const OpRef& B,
                                                  unsigned char* ring) {
  const int tid = opaque_tid(), lane = tid & 63, w = tid >> 6;
  unsigned ring_lds = lds_addr(ring);
  Dma128 da, db;
  da.init(A, lane, w);
  db.init(B, lane, w);
  asm volatile("" : "+s"(ring_lds));
#pragma unroll
  for (int p = 0; p < 8; ++p) da.issue(0, ring_lds, p);
#pragma unroll
  for (int p = 0; p < 8; ++p) db.issue(0, ring_lds + S64_A, p);
}

// FIRST: issue the first pair's loads here (else gemm_tile64_first did, and
// nothing else is in flight but them and stores).
template <bool FIRST = true>
__device__ __forceinline__ void gemm_tile64(const OpRef& A, const OpRef& B, int K, unsigned char* ring,
                                            floatx16 (&acc)[4][4]) {
  const int tid = opaque_tid(), lane = tid & 63, w = tid >> 6;
  zero_acc(acc);
  Frag64 fa;
  fa.init(lane, w & 1, w >> 1);
  unsigned ring_lds = lds_addr(ring);
  Dma128 da, db;
  da.init(A, lane, w);
  db.init(B, lane, w);
  asm volatile("" : "+s"(ring_lds));
  const int np = K / 64, klast = (np - 1) * 64;
  if (FIRST) {
#pragma unroll
    for (int p = 0; p < 8; ++p) da.issue(0, ring_lds, p);
#pragma unroll
    for (int p = 0; p < 8; ++p) db.issue(0, ring_lds + S64_A, p);
  }
  CCE_WAIT_VMCNT(0);
  ring_barrier();
  Frags f0, f1;
#pragma unroll
  for (int r = 0; r < 8; ++r) rd64(ring, fa, 0, r, f0);
  const int k1 = min(64, klast);
#pragma unroll
  for (int p = 0; p < 6; ++p) da.issue(k1, ring_lds + S64_STAGE, p);
  for (int s0 = 0; s0 < np; s0 += 2) {
    asm volatile("" : "+s"(ring_lds));
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int s = s0 + jj;
      if (s < np) {
        const unsigned char* cur = ring + jj * S64_STAGE;
        const unsigned char* nxt = ring + (jj ^ 1) * S64_STAGE;
        const unsigned lcur = ring_lds + jj * S64_STAGE, lnxt = ring_lds + (jj ^ 1) * S64_STAGE;
        const int kn = min((s + 1) * 64, klast), kn2 = min((s + 2) * 64, klast);
        sub64(da, db, fa, f0, f1, cur, 1, lnxt, kn, 6, 8, acc);   // A 6..7, B 0..5
        sub64(da, db, fa, f1, f0, cur, 2, lnxt, kn, 14, 2, acc);  // B 6..7
        sub64(da, db, fa, f0, f1, cur, 3, lnxt, kn, 0, 0, acc);
        CCE_WAIT_VMCNT(0);
        ring_barrier();
        sub64(da, db, fa, f1, f0, nxt, 0, lcur, kn2, 0, 6, acc);  // next pair: A 0..5
      }
    }
  }
  CCE_WAIT_VMCNT(0);
  __syncthreads();
}

}  // namespace cce
