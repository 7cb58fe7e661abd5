// Backward of the flash-CCE head.
//
// "Training — design (ORPO, flash-CCE head, …)" §5.1 (the analytic backward
// recomputes the logits from the saved per-row LSE and forms
// g (onehot - softmax); backward skips of near-zero softmax) and "ORPO training
// — design", lever 1 spec (backward).  With coef = -dL/dlogp:
//   G[i, v] = coef_i (softmax(i, v) - [v = y_i]),  dh = G W,  dW = G^T h.
//
// The vocabulary is walked in chunks of at most kVocabChunk entries.  Per
// chunk:
//   1. recompute z = h W[chunk]^T, G = coef (softmax - onehot) (times
//      sech^2(z / c) under a softcap c), optional filter / tile skip; G
//      written as bf16 (RNE)                                         MFMA
//   2. dh (+)= G W[chunk] and dW[chunk] = G^T h, one launch          MFMA
// All three contractions run on the same GEMM cores (256 x 256 tiles, or the
// 384 x 256 tall tiles where the operands allow); the transposed operands of
// step 2 (W[chunk] and h with K = vocab / tokens, and G^T) are read in place
// with transposing LDS reads, so nothing but G is materialised.  With tall
// tiles the two steps are pipelined over two G buffers: one launch runs chunk
// c's step 2 and chunk c+1's step 1.  dh accumulates across chunks in stream
// order, so no atomics are used and results are deterministic.  The workspace
// (G, or two of them) depends on M but not on V.
//
// G is stored BLOCKED: with Vc chunk columns, element (t, v) sits at
// ((t / 256) * (Vc / 32) + v / 32) * 8192 + (t % 256) * 32 + v % 32, so every
// 256 x 32 slice dh streams is one contiguous 16 KB block, and every 32 x 256
// slice dW streams is eight contiguous 2 KB pieces.
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <vector>

#include "cce_device.hpp"
#include "cce_launch.hpp"

namespace cce {

// The gradient entries of one recomputed tile, coef * softmax (times sech^2
// under a cap; the onehot part is not in G), straight from the accumulators
// to G: per (ii, jj, q) a lane holds 4 consecutive vocab entries of one token
// (vocab block wi*4 + ii of the tile, entries 8q + 4*half .. +3 of the row); the
// lanes l and l + 32 of a token trade halves with v_permlane32_swap so that
// each stores 8 consecutive entries (16 bytes): lane l those of q = 0 and 2,
// lane l + 32 those of q = 1 and 3.  !CAP:
// acc holds the raw logits and the softmax entry exp(z - lse) is formed here;
// CAP: acc holds t = tanh(z / c).  TGT: some token of this wave has its target
// among the wave's vocab rows (else no entry is compared with the target);
// VT: the tile runs past the chunk's last vocab row (those entries are 0).
// NI: vocab blocks of 32 in acc (4; 2 for the VGPR part of a tall tile); only
// the first nblk of them are stored (the blocks the dh contraction reads).
// RAW (with CAP): acc holds the raw logits z and t = tanh(z / c) is formed here
// (k2 = 2 log2(e) / c), so no pass rewrites the accumulators beforehand.
// LIVE: the pass also notes, per lane, whether some softmax entry it forms is
// >= lv->eps, separately for the two block parts of a tall tile: rows
// [0, lv->split) of this call's range lie in the first block, the rest in the
// second (split is a multiple of 32, so the part is fixed per ii).
struct PartLive {
  float eps;
  int split;
  bool l0, l1;
};

template <bool CAP, bool FILTER, bool TGT, bool VT, int NI = 4, bool RAW = false,
          bool LIVE = false>
__device__ __forceinline__ void store_grad_tile(const floatx16 (&acc)[NI][4],
                                                const float (&nlse)[4], const float (&cf)[4],
                                                const int (&off)[4], float c1, float filter_eps,
                                                int vl0, int vlen, int half, int wj, int lane,
                                                u16* __restrict__ gt, int nblk = NI,
                                                float k2 = 0.f, PartLive* lv = nullptr) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int tj = wj * 128 + jj * 32 + (lane & 31);
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      if (ii >= nblk) continue;
      const bool in1 = LIVE && ii * 32 >= lv->split;
      unsigned pk[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vbad = VT && (vl0 + ii * 32 + 8 * q + 4 * half + e >= vlen);
          float p, sech2 = 1.f;
          if (CAP) {
            const float t = RAW ? tanh_scaled(acc[ii][jj][4 * q + e], k2) : acc[ii][jj][4 * q + e];
            p = vbad ? 0.f : fast_exp2(fmaf(t, c1, nlse[jj]));
            sech2 = 1.f - t * t;
          } else {
            p = fast_exp2(fmaf(acc[ii][jj][4 * q + e], LOG2E, nlse[jj]));
            if (vbad) p = 0.f;
          }
          if (LIVE) {
            const bool hit = p >= lv->eps;
            lv->l0 |= hit && !in1;
            lv->l1 |= hit && in1;
          }
          // the target's entry is kept from the filter; its onehot part (-coef
          // sech^2) is applied outside these tiles, exactly
          const bool is_t = FILTER && TGT && (off[jj] == ii * 32 + 8 * q + e);
          if (FILTER && p < filter_eps && !is_t) p = 0.f;
          g[e] = cf[jj] * p * sech2;
        }
        pk[q][0] = pack_bf16x2(g[0], g[1]);
        pk[q][1] = pack_bf16x2(g[2], g[3]);
      }
#pragma unroll
      for (int qp = 0; qp < 4; qp += 2) {
        // lane l: its q = qp (entries 0..3) and lane l+32's (4..7); lane l+32:
        // lane l's q = qp+1 (entries 8..11) and its own (12..15)
        unsigned v[4];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto r = __builtin_amdgcn_permlane32_swap(pk[qp][d], pk[qp + 1][d], false, false);
          v[d] = r[0];
          v[2 + d] = r[1];
        }
        *reinterpret_cast<u32x4*>(gt + (size_t)ii * 8192 + tj * 32 + 8 * (qp + half)) =
            u32x4{v[0], v[1], v[2], v[3]};
      }
    }
  }
}

// Recompute one 256 (vocab) x 256 (token) logit tile of the chunk and write
// its gradient tile.  A = W rows of the chunk, B = h rows, so each lane owns
// one token (lse, coef, target in registers) and 16 vocab entries per MFMA
// tile.  One workgroup per tile; workgroup b takes logical tile
// (b % 8)*(n/8) + b/8 of the grouped raster (n = launch size, a multiple of
// 8), i.e. each XCD works on a contiguous run of tiles.
//
// CAP (final-logit softcap c): the accumulators keep t = tanh(z / c); the
// softmax entry is exp(c t - lse) and the chain rule through the cap adds the
// factor 1 - t^2 (sech^2(z / c)).  The tile-skip test uses the per-token
// largest t, which gives the largest softmax entry of that token.
//
// bm (the forward's saved block maximum of this chunk, tile vt of token j at
// bm[vt * M + j]; null when not given or block_eps = 0): the tile-skip test is
// taken before the recompute, from exp(bm - lse) and the targets, and a
// skipped tile is not recomputed at all.
template <bool VEC, bool FILTER, bool KTAIL, bool CAP>
__global__ __launch_bounds__(NT, 1) void k_recompute(
    const u16* __restrict__ H, const u16* __restrict__ Wc, const int* __restrict__ y,
    const float* __restrict__ lse, const float* __restrict__ coef, int M, int D, int v0,
    int vlen, int nMt, int nvt, float softcap, float filter_eps, float block_eps,
    u16* __restrict__ G, int* __restrict__ flags, int nkbV, const float* __restrict__ bm) {
  __shared__ Smem sm;
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;
  int mt, vt;
  if (!map_tile(blockIdx.x, gridDim.x, nMt, nvt, 8, mt, vt)) return;
  int* flag = flags + (size_t)mt * (nkbV / 8) + vt;
  if (bm) {
    // one token per thread: is any softmax entry of the tile >= block_eps, or
    // is the token's target among the tile's vocab rows?
    const int j = mt * TILE + tid;
    int keep = 0;
    if (j < M) {
      const float pm = fast_exp2((bm[(size_t)vt * M + j] - lse[j]) * LOG2E);
      const int o = y[j] - (v0 + vt * TILE);
      keep = (pm >= block_eps || (unsigned)o < (unsigned)TILE) ? 1 : 0;
    }
    if (!__syncthreads_or(keep)) {
      if (tid == 0) *flag = 0;
      return;
    }
  }

  floatx16 acc[4][4];
  gemm_tile<VEC, false, KTAIL>(OpRef{Wc + (size_t)vt * TILE * D, D, min(TILE, vlen - vt * TILE), D},
                               OpRef{H + (size_t)mt * TILE * D, D, min(TILE, M - mt * TILE), D}, D,
                               nullptr, 0, sm, acc);

  const int vl0 = vt * TILE + wi * 128;  // chunk-local vocab row of this wave's first A row
  float nlse[4], cf[4];
  int off[4];
  bool any_tgt_lane = false;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = mt * TILE + wj * 128 + jj * 32 + (lane & 31);
    const bool ok = j < M;
    nlse[jj] = ok ? -lse[j] * LOG2E : NEG_INF;  // padding rows: no softmax entries
    cf[jj] = ok ? coef[j] : 0.f;
    const int yy = ok ? y[j] : -1;
    off[jj] = (yy >= 0) ? yy - (v0 + vl0) - 4 * half : -1000000;
    const int o = (yy >= 0) ? yy - (v0 + vl0) : -1;
    any_tgt_lane |= (unsigned)o < 128u;
  }
  // CAP: acc becomes tanh(z / c) (rows beyond the chunk's valid vocab are
  // masked at the store).  The largest softmax entry is formed only for the
  // recompute-time skip test; otherwise the store pass forms each entry once.
  const bool vtail = vt * TILE + TILE > vlen;
  const bool skip_test = block_eps > 0.f && !bm;
  const float k2 = CAP ? 2.f * LOG2E / softcap : 0.f;
  const float c1 = CAP ? softcap * LOG2E : LOG2E;  // log2 of the softmax numerator per unit
  float pmax = 0.f;
  if (CAP) {
    float tmax[4] = {-1.f, -1.f, -1.f, -1.f};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vbad = vtail && (vl0 + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= vlen);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float t = tanh_scaled(acc[ii][jj][r], k2);
          acc[ii][jj][r] = t;
          if (!vbad) tmax[jj] = fmaxf(tmax[jj], t);
        }
      }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) pmax = fmaxf(pmax, fast_exp2(fmaf(tmax[jj], c1, nlse[jj])));
  } else if (skip_test) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vbad = vtail && (vl0 + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= vlen);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p = fast_exp2(fmaf(acc[ii][jj][r], LOG2E, nlse[jj]));
          if (!vbad) pmax = fmaxf(pmax, p);
        }
      }
  }
  if (skip_test) {
    // skip the tile if every softmax entry is below block_eps and no token of
    // the tile has its target among the tile's vocab rows
    const bool keep_lane = pmax >= block_eps || any_tgt_lane;
    const bool keep_wave = __ballot(keep_lane) != 0ull;
    if (lane == 0) red[w] = keep_wave ? 1.f : 0.f;
    __syncthreads();
    const bool keep = (red[0] + red[1] + red[2] + red[3]) > 0.f;
    if (!keep) {
      if (tid == 0) *flag = 0;
      return;
    }
  }
  if (tid == 0) *flag = 1;

  const bool wave_has_tgt = __ballot(any_tgt_lane) != 0ull;
  u16* gt = G + ((size_t)mt * nkbV + vt * 8 + wi * 4) * 8192;
#define CCE_STORE(TGT, VT)                                                                  \
  store_grad_tile<CAP, FILTER, TGT, VT>(acc, nlse, cf, off, c1, filter_eps, vl0, vlen, half, wj, \
                                        lane, gt)
  if (wave_has_tgt) {
    if (vtail) CCE_STORE(true, true); else CCE_STORE(true, false);
  } else {
    if (vtail) CCE_STORE(false, true); else CCE_STORE(false, false);
  }
#undef CCE_STORE
}

// The tall form of the recompute (384 vocab rows x 256 tokens per tile, the
// forward's tall GEMM; fewer operand bytes per FLOP), used when the operands
// allow it and no tile is skipped (block_eps = 0, so the dh / dW contractions
// read no tile flags).  Wave wi holds vocab blocks 6 wi .. 6 wi + 5 of the
// tile: 4 in acc.a, 2 in acc.v.  Blocks at or past nkb (the blocks the dh
// contraction reads: the chunk rounded up to 256) are not stored; entries past
// vlen within the stored blocks are 0.
struct RecArgs {
  const u16* H;
  const u16* Wc;  // the chunk's head rows
  const int* y;
  const float* lse;
  const float* coef;
  int M, D, v0, vlen, nMt, nvt;  // nvt: tall tiles of the chunk
  float softcap, filter_eps;
  u16* G;    // the chunk's gradient buffer (blocked)
  int nkbV;  // 32-wide vocab blocks per token tile of G
  int nkb;   // blocks the dh contraction reads
  int nl;    // workgroups of the recompute (a multiple of 8)
  // block skip (the SKIP forms): per (token tile, 256-entry vocab block) flags
  // of this chunk, the chunk's part of the forward's saved block maximum (or
  // null: the skip is decided from the recomputed entries), and the bound
  int* flags;
  const float* bm;
  float block_eps;
  int* qzero;  // null, or a set of task-queue counters that workgroup 0 clears
};

// Task queues of the pipelined launches' recompute tiles: per launch one set
// of 8 counters (one per XCD, 64 bytes apart); launch c takes set c % 2 and
// clears the other for launch c + 1 (the launch before it used that set and
// has finished; the first launch's set is cleared by the recompute launch
// before it).
constexpr int kQueueStride = 16;
constexpr int kQueueSet = 8 * kQueueStride;
static_assert(2 * kQueueSet == kQueueInts, "two queue sets fill the counters");

__device__ __forceinline__ void clear_queue_set(int* set) {
  if (set && blockIdx.x == 0 && threadIdx.x < kQueueSet) set[threadIdx.x] = 0;
}

__device__ __forceinline__ int queue_len(int n, int x) { return (n - x + 7) >> 3; }

// A ticket from another XCD's queue once the own one is exhausted (-1: none
// left anywhere).
__device__ __forceinline__ int steal_task(int* queue, int home, int n) {
  for (int d = 1; d < 8; ++d) {
    const int x = (home + d) & 7;
    int* const c = queue + x * kQueueStride;
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= queue_len(n, x))
      continue;
    const int k = atomicAdd(c, 1);
    if (k < queue_len(n, x)) return x + 8 * k;
  }
  return -1;
}

// Whether v holds for any thread of the workgroup, through 16 bytes of LDS at
// `scratch` (the operand ring, which must not be in use: the tall tile's 160
// KB leave no room for the reduction __syncthreads_or would add).
__device__ __forceinline__ bool block_any(bool v, unsigned char* scratch) {
  const unsigned long long m = __ballot(v);
  volatile int* const s = reinterpret_cast<volatile int*>(scratch);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = m != 0ull ? 1 : 0;
  __syncthreads();
  const bool r = (s[0] | s[1] | s[2] | s[3]) != 0;
  __syncthreads();
  return r;
}

// The skip flag of 256-entry vocab block bb of token tile mt, as tall tile vt
// (of nvt3) sees it.  A block that lies inside the tile is written whole; one
// shared with a neighbouring tile is written by halves: 16 bits each, the
// lower by the tile below, the upper by the tile above, so that each half has
// one writer and the 32-bit flag the contractions read is nonzero when either
// part of the block is live.  Every flag of the chunk is written on every
// pass, so none is left from an earlier chunk.
__device__ __forceinline__ void put_block_flag(int* flags, int fstride, int mt, int bb, int vt,
                                               int nvt3, bool live) {
  int* const f = flags + (size_t)mt * fstride + bb;
  const int lo = bb * TILE, t0 = vt * TALL;
  if (lo < t0)
    reinterpret_cast<unsigned short*>(f)[1] = live ? 1 : 0;
  else if (lo + TILE > t0 + TALL && vt + 1 < nvt3)
    reinterpret_cast<unsigned short*>(f)[0] = live ? 1 : 0;
  else
    *f = live ? 1 : 0;
}

// Recompute task b (of r.nl) of a chunk: one tall tile.  SKIP: the block skip
// of (token tile, 256-entry vocab block) pairs.  A tall tile overlaps two such
// blocks (the first whole and half of the next, or half of one and the next
// whole).  With the saved block maximum the test comes first: each block's
// liveness is decided from it (exp(bm - lse) >= block_eps for some token, or a
// token's target in the block), and a tile whose blocks are both dead is not
// recomputed at all.  Without it the tile is recomputed, the store pass notes
// per block part whether some softmax entry reaches block_eps, and the parts'
// votes combine in the block's flag (put_block_flag); the tile's gradient
// entries are stored either way, and the contractions leave out the dead
// blocks.
template <bool FILTER, bool CAP, bool SKIP = false>
__device__ __forceinline__ void recompute_tall_tile(const RecArgs& r, int b, SmemTall& sm) {
  const u16* __restrict__ H = r.H;
  const u16* __restrict__ Wc = r.Wc;
  const int* __restrict__ y = r.y;
  const float* __restrict__ lse = r.lse;
  const float* __restrict__ coef = r.coef;
  const int M = r.M, D = r.D, v0 = r.v0, vlen = r.vlen, nkbV = r.nkbV, nkb = r.nkb;
  const float softcap = r.softcap, filter_eps = r.filter_eps;
  u16* __restrict__ G = r.G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;
  int mt, vt;
  if (!map_tile(b, r.nl, r.nMt, r.nvt, 8, mt, vt)) return;
  const int nblk = nkb / 8, fstride = nkbV / 8;
  const int b_lo = vt * TALL / TILE;
  const bool two = b_lo + 1 < nblk && vt * TALL + TALL > (b_lo + 1) * TILE;
  if (SKIP && r.bm) {
    // one token per thread
    const int j = mt * TILE + tid;
    bool any = false;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q == 1 && !two) break;
      const int bb = b_lo + q;
      int keep = 0;
      if (j < M) {
        const float pm = fast_exp2((r.bm[(size_t)bb * M + j] - lse[j]) * LOG2E);
        const int o = y[j] - (v0 + bb * TILE);
        keep = (pm >= r.block_eps || (unsigned)o < (unsigned)TILE) ? 1 : 0;
      }
      const bool live = block_any(keep != 0, sm.raw);
      if (tid == 0) put_block_flag(r.flags, fstride, mt, bb, vt, r.nvt, live);
      any |= live;
    }
    if (!any) return;
  }

  AccTall acc;
  gemm_tile_tall<false>(OpRef{Wc + (size_t)vt * TALL * D, D, min(TALL, vlen - vt * TALL), D},
                 OpRef{H + (size_t)mt * TILE * D, D, min(TILE, M - mt * TILE), D}, D, sm, acc);

  const int vl0 = vt * TALL + wi * 192;  // chunk-local vocab row of this wave's first A row
  float nlse[4], cf[4];
  int off[4], off2[4];
  bool any_tgt_lane = false;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = mt * TILE + wj * 128 + jj * 32 + (lane & 31);
    const bool ok = j < M;
    nlse[jj] = ok ? -lse[j] * LOG2E : NEG_INF;  // padding rows: no softmax entries
    cf[jj] = ok ? coef[j] : 0.f;
    const int yy = ok ? y[j] : -1;
    off[jj] = (yy >= 0) ? yy - (v0 + vl0) - 4 * half : -1000000;
    off2[jj] = off[jj] - 128;
    const int o = (yy >= 0) ? yy - (v0 + vl0) : -1;
    any_tgt_lane |= (unsigned)o < 192u;
  }
  const float c1 = CAP ? softcap * LOG2E : LOG2E;  // log2 of the softmax numerator per unit
  const float k2 = CAP ? 2.f * LOG2E / softcap : 0.f;  // the cap's tanh is taken at the store
  const bool vtail = vt * TALL + TALL > vlen;
  // SKIP without the saved maximum: the store pass notes, per block part,
  // whether some softmax entry is >= block_eps (tile rows below `split` are in
  // block b_lo, the rest in b_lo + 1; split is 256 or 128, a multiple of the
  // 32-row MFMA tiles); the parts' votes and the targets then set the flags.
  constexpr bool LIVE = SKIP;
  const int split = (b_lo + 1) * TILE - vt * TALL;
  PartLive la{r.block_eps, split - wi * 192, false, false};
  PartLive lv{r.block_eps, split - wi * 192 - 128, false, false};
  const bool wave_has_tgt = __ballot(any_tgt_lane) != 0ull;
  const int b0 = vt * 12 + wi * 6;  // this wave's first vocab block of the chunk
  const int nb = min(max(nkb - b0, 0), 6);
  u16* gt = G + ((size_t)mt * nkbV + b0) * 8192;
#define CCE_STORE(TGT, VT)                                                                     \
  do {                                                                                         \
    store_grad_tile<CAP, FILTER, TGT, VT, 4, true, LIVE>(acc.a, nlse, cf, off, c1, filter_eps, \
                                                         vl0, vlen, half, wj, lane, gt,        \
                                                         min(nb, 4), k2, &la);                 \
    store_grad_tile<CAP, FILTER, TGT, VT, 2, true, LIVE>(acc.v, nlse, cf, off2, c1,            \
                                                         filter_eps, vl0 + 128, vlen, half,    \
                                                         wj, lane, gt + 4 * 8192, nb - 4, k2,  \
                                                         &lv);                                 \
  } while (0)
  if (wave_has_tgt) {
    if (vtail) CCE_STORE(true, true); else CCE_STORE(true, false);
  } else {
    if (vtail) CCE_STORE(false, true); else CCE_STORE(false, false);
  }
#undef CCE_STORE
  if (SKIP && !r.bm) {
    bool tg[2] = {false, false};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = mt * TILE + wj * 128 + jj * 32 + (lane & 31);
      const int yy = j < M ? y[j] : -1;
      const int o = yy >= 0 ? yy - (v0 + b_lo * TILE) : -1;
      tg[0] |= (unsigned)o < (unsigned)TILE;
      tg[1] |= (unsigned)(o - TILE) < (unsigned)TILE;
    }
    const bool live0 = block_any(la.l0 || lv.l0 || tg[0], sm.raw);
    const bool live1 = block_any(la.l1 || lv.l1 || tg[1], sm.raw);
    if (tid == 0) {
      put_block_flag(r.flags, fstride, mt, b_lo, vt, r.nvt, live0);
      if (two) put_block_flag(r.flags, fstride, mt, b_lo + 1, vt, r.nvt, live1);
    }
  }
}

template <bool FILTER, bool CAP, bool SKIP>
__global__ __launch_bounds__(NT, 1) void k_recompute_tall(RecArgs r) {
  __shared__ SmemTall sm;
  clear_queue_set(r.qzero);
  recompute_tall_tile<FILTER, CAP, SKIP>(r, blockIdx.x, sm);
}

// One fp32-output contraction C[ta*256 + i][tb*256 + j] (+)= sum_k A[i][k] B[j][k]
// over an nA x nB tile grid launched as nl workgroups.  a / b describe tile 0;
// tile ta of A starts a_tile elements after a.p, tile tb of B b_tile elements
// after b.p (with b.cols reduced by tb*256).
//
// Split K (first problem only, the dh form: A blocked, B read transposed): the
// tiles of raster index >= n_full are each ks tasks, part q taking K blocks
// [q*nb/ks, (q+1)*nb/ks) of the nb = K/256 (tiles below n_full are one task
// over all of K).  Part 0 writes C as above; part q > 0 of split tile u writes
// (no accumulation) the 256 x 256 partial tile P + ((q-1)*nsplit + u)*65536
// (tile-local, leading dimension 256), and k_split_reduce adds the partials to
// C in the order q = 1, 2, ...  Tasks run full tiles first, then the parts.
struct GemmProb {
  OpRef a, b;
  size_t a_tile, b_tile;
  int K;
  float* C;
  int ldc, c_rows, c_cols;
  int nA, nB, nl;
  const int* kflags;  // per 256-wide K block of A tile ta: kflags[ta*fa + kb*fk]
  int fa, fk;
  int accum;   // 1: C += result, 0: C = result
  int ks;      // K parts of a split tile (1: no split)
  int n_full;  // tiles (raster order) that are not split
  float* P;
  int tall;    // the dW form in 384-row tiles (A = G^T over 12 vocab blocks; a.cols =
               // the blocks' columns per token tile, a_tile = 12 blocks)
};

// Workgroup b of a problem -> (tile, K part, split-tile index u or -1); false
// for the padding workgroups.  Unsplit: the XCD-contiguous grouped raster of
// map_tile.  Split (n_full a multiple of 8): each XCD (b % 8) takes its eighth
// of the full tiles first and then its eighth of the parts, so the long tasks
// are spread over all XCDs.
__device__ __forceinline__ bool split_task(const GemmProb& p, int b, int& ta, int& tb, int& part,
                                           int& u) {
  const int nT = p.nA * p.nB;
  int L;
  part = 0;
  u = -1;
  if (p.ks == 1) {
    L = xcd_task(b, p.nl);
    if (L >= nT) return false;
  } else {
    const int x = b & 7, i = b >> 3;
    const int nf8 = p.n_full / 8;
    if (i < nf8) {
      L = x * nf8 + i;
    } else {
      const int np = (nT - p.n_full) * p.ks, np8 = (np + 7) / 8;
      const int r = x * np8 + (i - nf8);
      if (i - nf8 >= np8 || r >= np) return false;
      u = r / p.ks;
      part = r - u * p.ks;
      L = p.n_full + u;
    }
  }
  raster_tile(L, p.nA, p.nB, 8, ta, tb);
  return true;
}

// 4x4 transpose inside each quad of lanes (lanes 4k .. 4k+3): lane x holds
// column x of a 4x4 block (v[0..3] = rows 0..3); afterwards it holds row x
// (v[0..3] = columns 0..3).  Two DPP stages: lanes x and x^2 trade a pair of
// values, then lanes x and x^1 trade one value of each pair.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(float (&v)[4], int lane) {
  const int x = lane & 3;
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = quad_perm<0x4E>(v[i]);  // lane x reads lane x^2
  const bool lo = x < 2;
  v[0] = lo ? v[0] : t[2];
  v[1] = lo ? v[1] : t[3];
  v[2] = lo ? t[0] : v[2];
  v[3] = lo ? t[1] : v[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = quad_perm<0xB1>(v[i]);  // lane x reads lane x^1
  const bool even = (x & 1) == 0;
  v[0] = even ? v[0] : t[1];
  v[1] = even ? t[0] : v[1];
  v[2] = even ? v[2] : t[3];
  v[3] = even ? t[2] : v[3];
}

// Output tiles leave the accumulators through LDS, one 32-row band of a
// wave's 128 columns at a time, so that each global load or store instruction
// covers two runs of 512 contiguous bytes (lane l: row 2k + l / 32, columns
// 4 (l % 32) ..): the per-CU store path moves about 3x more bytes per second
// that way than with the quad-transposed layout's 8 rows x 128 bytes per
// instruction.  Each wave owns kBandBytes of LDS at w * kBandBytes (the
// operand ring is free once the K loop has returned); the row pitch 576 bytes
// puts rows r and r + 1 16 banks apart, so neither the 16-byte writes of the
// quad-transposed fragments nor the row reads conflict within 16 lanes.  LDS
// accesses of one wave complete in order, so a band's reads see its writes
// and the next band's writes wait for them.
constexpr int kBandPitch = 576;
constexpr int kBandBytes = 32 * kBandPitch;

// Band rows 0..31 x columns 0..127 from t[jj] (32 x 32 accumulator tiles).
__device__ __forceinline__ void band_put(unsigned char* band, const floatx16 (&t)[4], int lane) {
  const int half = lane >> 5;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float v[4] = {t[jj][4 * r4], t[jj][4 * r4 + 1], t[jj][4 * r4 + 2], t[jj][4 * r4 + 3]};
      quad_transpose(v, lane);
      const int row = 8 * r4 + 4 * half + (lane & 3);
      const int col = jj * 32 + (lane & 28);
      *reinterpret_cast<float4*>(band + row * kBandPitch + col * 4) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Rows 2k and 2k + 1 of a band: lane l gets columns 4 (l % 32) .. + 3 of row
// 2k + l / 32.
__device__ __forceinline__ float4 band_get(const unsigned char* band, int k, int lane) {
  return *reinterpret_cast<const float4*>(band + (2 * k + (lane >> 5)) * kBandPitch +
                                          (lane & 31) * 16);
}

// The dh and dW contractions of one vocab chunk in a single launch: workgroups
// [0, p0.nl) take p0 (dh, the longer K), the rest take p1 (dW).  Dispatching
// the long tiles first lets the short ones fill the tail, so the two problems
// together keep every CU busy (dh alone has too few output tiles).
//   dh: A = G (blocked), B = W[chunk] read transposed (K = vocab)
//   dW: A = G read transposed (K = tokens), B = h read transposed
// dW of one tall tile (384 vocab rows x 256 columns of D): C rows ta*384 + ..,
// written (dW is never accumulated).  The output leaves the accumulators
// through the quad transpose, as 16-byte stores of 4 consecutive columns; the
// VGPR part first, so its registers are free before the AGPR part is read.
__device__ __forceinline__ void dw_tall_task(const GemmProb& p, int ta, int tb, const OpRef& bo,
                                             SmemTall& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;
  const OpRef at{p.a.p + ta * p.a_tile, p.a.ld, 0, p.a.cols - ta * TALL};
  AccTall acc;
  gemm_tile_tall<true>(at, bo, p.K, sm, acc);
  const bool vec4 = (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15u) == 0;
  if (vec4 && (ta + 1) * TALL <= p.c_rows && (tb + 1) * TILE <= p.c_cols) {
    // the whole tile inside C: row-contiguous stores through this wave's band
    unsigned char* const band = sm.raw + w * kBandBytes;
    float* const c0 = p.C + (size_t)(ta * TALL + wi * 192) * p.ldc + tb * TILE + wj * 128 +
                      (lane & 31) * 4;
    auto flush = [&](const floatx16 (&t)[4], int ii) {
      band_put(band, t, lane);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        *reinterpret_cast<float4*>(c0 + (size_t)(ii * 32 + 2 * k + half) * p.ldc) =
            band_get(band, k, lane);
    };
    // the VGPR part first, so its registers are free before the AGPRs are read
    flush(acc.v[0], 4);
    flush(acc.v[1], 5);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) flush(acc.a[ii], ii);
    return;
  }
  auto put = [&](const floatx16& t, int ii, int jj) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float v[4] = {t[4 * r4], t[4 * r4 + 1], t[4 * r4 + 2], t[4 * r4 + 3]};
      quad_transpose(v, lane);
      const int row = ta * TALL + wi * 192 + ii * 32 + 8 * r4 + 4 * half + (lane & 3);
      const int col0 = tb * TILE + wj * 128 + jj * 32 + (lane & 28);
      if (row >= p.c_rows) continue;
      float* const c = p.C + (size_t)row * p.ldc + col0;
      if (vec4 && col0 + 4 <= p.c_cols) {
        *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col0 + e < p.c_cols) c[e] = v[e];
      }
    }
  };
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) put(acc.v[ii][jj], 4 + ii, jj);
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) put(acc.a[ii][jj], ii, jj);
}

template <bool SKIP, bool VEC>
__device__ __forceinline__ void grads_task(const GemmProb& p0, const GemmProb& p1, int b,
                                           SmemTall& smt) {
  Smem& sm = *reinterpret_cast<Smem*>(&smt);
  const bool second = b >= p0.nl;
  const GemmProb p = second ? p1 : p0;
  if (second) b -= p0.nl;
  int ta, tb, part, u;
  if (!split_task(p, b, ta, tb, part, u)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;
  const int nb = p.K / TILE;
  const int parts = u < 0 ? 1 : p.ks;
  const int kb0 = part * nb / parts, kb1 = (part + 1) * nb / parts;
  // part offsets (the split problem is of the dh form: A blocked, 8 blocks of
  // 8192 elements per 256 K; B [k][i] with pitch ld)
  const OpRef a{p.a.p + ta * p.a_tile + (size_t)kb0 * 8 * 8192, p.a.ld, p.a.rows, p.a.cols};
  const OpRef bo{p.b.p + tb * p.b_tile + (size_t)kb0 * TILE * p.b.ld, p.b.ld,
                 p.b.rows - kb0 * TILE, p.b.cols - tb * TILE};
  if (VEC && !SKIP && second && p.tall) {
    dw_tall_task(p, ta, tb, bo, smt);
    return;
  }
  const int* kf = SKIP ? p.kflags + (size_t)ta * p.fa + (size_t)kb0 * p.fk : nullptr;
  floatx16 acc[4][4];
  if (!second)
    gemm_tile<VEC, SKIP, false, OP_BLK, OP_KROW>(a, bo, (kb1 - kb0) * TILE, kf, p.fk, sm, acc);
  else
    gemm_tile<VEC, SKIP, false, OP_KBLK, OP_KROW>(a, bo, p.K, kf, p.fk, sm, acc);
  const bool accum = p.accum != 0 && part == 0;
  if (part > 0) {
    // a partial tile, tile-local (rows and columns past C's are never read)
    const int nsplit = p.nA * p.nB - p.n_full;
    float* const Pt = p.P + ((size_t)(part - 1) * nsplit + u) * (TILE * TILE);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float v[4] = {acc[ii][jj][4 * r4], acc[ii][jj][4 * r4 + 1], acc[ii][jj][4 * r4 + 2],
                        acc[ii][jj][4 * r4 + 3]};
          quad_transpose(v, lane);
          const int row = wi * 128 + ii * 32 + 8 * r4 + 4 * half + (lane & 3);
          const int col0 = wj * 128 + jj * 32 + (lane & 28);
          *reinterpret_cast<float4*>(Pt + (size_t)row * TILE + col0) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
    return;
  }
  // Each lane holds 4 consecutive rows of one column per (ii, r4, jj); a quad
  // transpose gives it 4 consecutive columns of one row, stored (and for dh
  // accumulated) as 16 bytes when C's rows are 16-byte aligned.
  float* const Cb = p.C;
  const bool vec4 = (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15u) == 0;
  if (!SKIP && vec4 && (ta + 1) * TILE <= p.c_rows && (tb + 1) * TILE <= p.c_cols) {
    // The whole tile inside C: row-contiguous loads and stores through this
    // wave's band.  The accumulation reads two bands of C (2 x 16 x 16 bytes a
    // lane) before it adds and stores them: a store may alias a later read, so
    // reading each piece just before its store would cost one memory round
    // trip per piece.
    unsigned char* const band = sm.raw + w * kBandBytes;
    float* const c0 = Cb + (size_t)(ta * TILE + wi * 128) * p.ldc + tb * TILE + wj * 128 +
                      (lane & 31) * 4;
#pragma unroll
    for (int i2 = 0; i2 < 4; i2 += 2) {
      float4 q[2][16];
      if (accum) {
#pragma unroll
        for (int di = 0; di < 2; ++di)
#pragma unroll
          for (int k = 0; k < 16; ++k)
            q[di][k] = *reinterpret_cast<const float4*>(
                c0 + (size_t)((i2 + di) * 32 + 2 * k + half) * p.ldc);
      }
#pragma unroll
      for (int di = 0; di < 2; ++di) {
        band_put(band, acc[i2 + di], lane);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          float4 o = band_get(band, k, lane);
          if (accum) {
            o.x += q[di][k].x;
            o.y += q[di][k].y;
            o.z += q[di][k].z;
            o.w += q[di][k].w;
          }
          *reinterpret_cast<float4*>(c0 + (size_t)((i2 + di) * 32 + 2 * k + half) * p.ldc) = o;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v[4] = {acc[ii][jj][4 * r4], acc[ii][jj][4 * r4 + 1], acc[ii][jj][4 * r4 + 2],
                      acc[ii][jj][4 * r4 + 3]};
        quad_transpose(v, lane);
        const int row = ta * TILE + wi * 128 + ii * 32 + 8 * r4 + 4 * half + (lane & 3);
        const int col0 = tb * TILE + wj * 128 + jj * 32 + (lane & 28);
        if (row >= p.c_rows) continue;
        float* const c = Cb + (size_t)row * p.ldc + col0;
        if (vec4 && col0 + 4 <= p.c_cols) {
          float4 o = make_float4(v[0], v[1], v[2], v[3]);
          if (accum) {
            const float4 q = *reinterpret_cast<const float4*>(c);
            o.x += q.x;
            o.y += q.y;
            o.z += q.z;
            o.w += q.w;
          }
          *reinterpret_cast<float4*>(c) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col0 + e < p.c_cols) c[e] = accum ? c[e] + v[e] : v[e];
        }
      }
}

template <bool SKIP, bool VEC>
__global__ __launch_bounds__(NT, 1) void k_grads(GemmProb p0, GemmProb p1) {
  __shared__ SmemTall sm;  // the 256-row tasks use its first 128 KB
  grads_task<SKIP, VEC>(p0, p1, blockIdx.x, sm);
}

// One launch of the pipelined backward: the dh / dW tasks of vocab chunk c
// (workgroups [0, p0.nl + p1.nl), reading chunk c's gradient buffer) and the
// recompute tiles of chunk c + 1 (the rest, writing the other buffer).  The
// long dh tasks go first, then dW, then the recompute tiles; the two kinds
// fill each other's partial rounds, and the recompute's gradient stores
// overlap other workgroups' contractions.
// SKIP: the block skip (256-row dW tiles and the compacted K loops of the
// contractions read the flags the previous launch's recompute tiles wrote).
//
// The recompute tiles are taken by at most one workgroup per CU, each looping
// over tiles until none is left: tile t belongs to queue t % 8 (the XCD a
// one-tile-per-workgroup launch gives it, keeping the grouped raster's operand
// sharing inside one L2), and a queue hands its tiles out in order.  A worker
// takes from its own XCD's queue (workgroup g runs on XCD g % 8), then from
// the others: the XCDs that finish their share of the launch early take over
// the rest instead of idling through its tail.  Tiles are independent, every
// ticket is taken once by an atomic increment of a counter that only grows,
// and a worker leaves when all 8 queues are exhausted.
template <bool FILTER, bool CAP, bool SKIP>
__global__ __launch_bounds__(NT, 1) void k_bwd_fused(GemmProb p0, GemmProb p1, RecArgs r,
                                                     int* queue) {
  __shared__ SmemTall sm;
  clear_queue_set(r.qzero);
  const int b = blockIdx.x, ng = p0.nl + p1.nl;
  if (b < ng) {
    grads_task<SKIP, true>(p0, p1, b, sm);
    return;
  }
  const int home = b & 7;
  int* const own = queue + home * kQueueStride;
  volatile int* const slot = reinterpret_cast<volatile int*>(sm.raw);
  for (;;) {
    // the ring is free here (a tile ends with its loads drained and a
    // barrier; the loop's last barrier follows it)
    if (threadIdx.x == 0) {
      const int k = atomicAdd(own, 1);
      *slot = k < queue_len(r.nl, home) ? home + 8 * k : steal_task(queue, home, r.nl);
    }
    __syncthreads();
    const int t = *slot;
    __syncthreads();
    if (t < 0) break;
    recompute_tall_tile<FILTER, CAP, SKIP>(r, t, sm);
    __syncthreads();
  }
}

static inline int pad8(int n) { return (n + 7) / 8 * 8; }

// For each split tile u of p, C[tile] += P[0][u] + P[1][u] + ... + P[ks-2][u],
// the partials added in that order.  Workgroup (u, y) takes tile rows
// 16y .. 16y+15, one column per thread (each row a coalesced 1 KB).
__global__ __launch_bounds__(256) void k_split_reduce(GemmProb p) {
  const int nsplit = p.nA * p.nB - p.n_full;
  const int u = blockIdx.x;
  if (u >= nsplit) return;
  int ta, tb;
  raster_tile(p.n_full + u, p.nA, p.nB, 8, ta, tb);
  const int col = tb * TILE + (int)threadIdx.x;
  if (col >= p.c_cols) return;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = (int)blockIdx.y * 16 + k;
    const int row = ta * TILE + r;
    if (row < p.c_rows) {
      float c = p.C[(size_t)row * p.ldc + col];
      for (int q = 0; q < p.ks - 1; ++q)
        c += p.P[((size_t)q * nsplit + u) * (TILE * TILE) + (size_t)r * TILE + threadIdx.x];
      p.C[(size_t)row * p.ldc + col] = c;
    }
  }
}

// Split of the dh contraction over K for one vocab chunk of nvt tiles: either
// every tile in ks parts (n_full = 0), or only the tiles past the last full
// round of kCUs (a quarter-full second round of long tasks otherwise idles most
// of the chip).  Chosen by simulating the hardware's in-order dispatch of the
// launch (full tiles, then the parts, then the dW tasks, each to the earliest
// free CU) with a cost of one unit per 32-wide K slice plus a fixed per-task
// overhead, and adding the reduction's memory time; the partial tiles must fit
// max_tiles.  The model is optimistic (a quarter-full round also runs at a
// higher clock), so a split is taken only for a predicted gain of 20 % or more.
static DhSplit dh_split_sim(int nMt, int nDt, int nvt, bool with_dw, int Mpad, long long max_tiles) {
  const long long nT = (long long)nMt * nDt;
  const double over = 8.0, unit_us = 0.9, reduce_bpu = 4.0e6 * unit_us;  // bytes per unit
  const double tile_bytes = (double)kTile * kTile * 4;
  auto span_of = [&](long long n_full, int ks) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> q(
        std::greater<double>(), std::vector<double>(kCUs, 0.0));
    auto run = [&](double cost) {
      const double t = q.top();
      q.pop();
      q.push(t + cost);
    };
    for (long long t = 0; t < n_full; ++t) run(nvt * (kTile / 32) + over);
    for (long long t = n_full; t < nT; ++t)
      for (int part = 0; part < ks; ++part)
        run(((part + 1) * nvt / ks - part * nvt / ks) * (kTile / 32) + over);
    if (with_dw)
      for (long long t = 0; t < (long long)nvt * nDt; ++t) run(Mpad / 32 + over);
    double span = 0.0;
    while (!q.empty()) {
      span = q.top();
      q.pop();
    }
    if (n_full < nT) span += (double)(nT - n_full) * tile_bytes * (ks + 1) / reduce_bpu;
    return span;
  };
  DhSplit best{1, (int)nT};
  const double none = span_of(nT, 1);
  double best_span = none;
  const long long tails[2] = {0, nT > kCUs ? nT - nT % kCUs : nT};
  for (long long n_full : tails) {
    if (n_full >= nT) continue;
    for (int ks = 2; ks <= 8 && ks <= nvt; ++ks) {
      if ((long long)(ks - 1) * (nT - n_full) > max_tiles) break;
      const double sp = span_of(n_full, ks);
      if (sp < 0.8 * none && sp < best_span) {
        best_span = sp;
        best = DhSplit{ks, (int)n_full};
      }
    }
  }
  return best;
}

DhSplit dh_split(int nMt, int nDt, int nvt, bool with_dw, int Mpad, long long max_tiles) {
  const long long nT = (long long)nMt * nDt;
  if (max_tiles <= 0 || nT >= 4LL * kCUs || nvt < 2) return DhSplit{1, (int)nT};
  // the simulation takes up to milliseconds: one run per distinct shape
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, bool, int, long long>, DhSplit> memo;
  const auto key = std::make_tuple(nMt, nDt, nvt, with_dw, Mpad, max_tiles);
  {
    std::lock_guard<std::mutex> g(mu);
    const auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  const DhSplit r = dh_split_sim(nMt, nDt, nvt, with_dw, Mpad, max_tiles);
  std::lock_guard<std::mutex> g(mu);
  memo.emplace(key, r);
  return r;
}

// Vocabulary entries per backward step when the recompute runs tall tiles:
// the chunk (Vc, the workspace width) is narrowed to a multiple of 768 (two
// tall tiles, three 256-blocks) whose nMt x (width / 384) recompute tiles fill
// whole rounds of kCUs workgroups, if one within 1/8 of Vc exists (e.g. 15360
// at 32 or 64 token tiles: exactly 5 or 10 rounds, against 5.4 or 10.75 at
// 16384); otherwise Vc.
static int tall_chunk(int Vc, int nMt) {
  for (int w = Vc / 768 * 768; w >= Vc - Vc / 8 && w >= 768; w -= 768)
    if ((long long)nMt * (w / TALL) % kCUs == 0) return w;
  return Vc;
}

// The dh / dW problems of one vocab chunk [v0, v0 + vlen) over the gradient
// buffer G (see the kernels above for the operand forms).
static void grads_probs(const BwdArgs& a, int v0, int vlen, const u16* Wc, u16* G, GemmProb& dh,
                        GemmProb& dw, DhSplit& sp, bool tall_dw = false, bool no_split = false) {
  const int nDt = a.Dpad / kTile;
  const int nkbV = a.Vc / 32;
  const int nvt = (vlen + kTile - 1) / kTile;
  const int fstride = a.Vc / kTile;
  const bool with_dw = a.q.Wq == nullptr;
  const int nT = a.nMt * nDt;
  sp = no_split ? DhSplit{1, nT} : dh_split(a.nMt, nDt, nvt, with_dw, a.Mpad, a.P_tiles);
  const int dh_nl =
      sp.ks == 1 ? pad8(nT) : 8 * (sp.n_full / 8 + ((nT - sp.n_full) * sp.ks + 7) / 8);
  // dh accumulates into what launch_target_dh wrote (the onehot part)
  dh = GemmProb{OpRef{G, 0, 0, 0}, OpRef{Wc, a.D, vlen, a.D}, (size_t)nkbV * 8192,
                (size_t)kTile, nvt * kTile, a.dh, a.D, a.M, a.D, a.nMt, nDt, dh_nl, a.flags,
                fstride, 1, 1, sp.ks, sp.n_full, a.P, 0};
  dw = GemmProb{OpRef{G, nkbV, 0, 0}, OpRef{a.H, a.D, a.M, a.D}, (size_t)8 * 8192,
                (size_t)kTile, a.Mpad, a.dW ? a.dW + (size_t)v0 * a.D : nullptr, a.D, vlen,
                a.D, nvt, nDt, pad8(nvt * nDt), a.flags, 1, fstride, 0, 1, nvt * nDt, nullptr, 0};
  if (tall_dw) {  // 384-row vocab tiles: 12 blocks of G each
    const int nvt3 = (vlen + TALL - 1) / TALL;
    dw.a.cols = nkbV * 32;
    dw.a_tile = (size_t)12 * 8192;
    dw.nA = nvt3;
    dw.nl = pad8(nvt3 * nDt);
    dw.n_full = nvt3 * nDt;
    dw.tall = 1;
  }
}

static RecArgs rec_args(const BwdArgs& a, int v0, int vlen, const u16* Wc, u16* G) {
  const int nvt3 = (vlen + TALL - 1) / TALL;
  return RecArgs{a.H,     Wc,           a.y, a.lse, a.coef, a.M, a.D,        v0,
                 vlen,    a.nMt,        nvt3, a.softcap, a.filter_eps, G, a.Vc / 32,
                 (vlen + kTile - 1) / kTile * 8, pad8(a.nMt * nvt3), nullptr, nullptr, 0.f,
                 nullptr};
}

static hipError_t split_reduce(const GemmProb& dh, const DhSplit& sp, hipStream_t st) {
  const int nT = dh.nA * dh.nB;
  if (sp.n_full < nT)
    CCE_TIMED(KN_SPLIT_REDUCE, 0.0, st,
              hipLaunchKernelGGL(k_split_reduce, dim3(nT - sp.n_full, TILE / 16), dim3(256), 0, st,
                                 dh));
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t st) {
  hipError_t e;
  const int nkbV = a.Vc / 32;
  const bool filt = a.filter_eps > 0.f;
  const bool cap = a.softcap > 0.f;
  // tall recompute tiles (and the pipelined backward) need aligned row-major
  // operands with D % 32 == 0; with a tile skip only the pipelined bf16 form
  // takes them (its recompute keeps the flags per 256-entry block)
  const bool skip = a.block_eps > 0.f;
  const bool tall_ok = a.vec && a.D % BK == 0;
  const bool pipe = tall_ok && a.q.Wq == nullptr && a.G2 != nullptr && a.flags2 != nullptr;
  const bool tall = tall_ok && (pipe || !skip);
  const int vstep = tall ? tall_chunk(a.Vc, a.nMt) : a.Vc;
  // the vocabulary chunks; the last one takes whatever is left when it fits
  // the workspace width (no short remainder chunk that runs the chip a
  // fraction full)
  std::vector<std::pair<int, int>> chunks;
  for (int v0 = 0, vlen = 0; v0 < a.V; v0 += vlen) {
    vlen = a.V - v0 <= a.Vc ? a.V - v0 : vstep;
    chunks.emplace_back(v0, vlen);
  }
  const int nch = (int)chunks.size();
  if ((e = launch_target_dh(a, st)) != hipSuccess) return e;
  const bool with_dw_all = a.q.Wq == nullptr;

  // Pipelined form (bf16 head, tall recompute, a second gradient buffer):
  // recompute chunk 0, then one launch per chunk c running c's dh / dW tasks
  // and c + 1's recompute tiles into the other buffer.  Stream order keeps
  // every dependence: chunk c's buffer is complete before the launch that
  // reads it, and is rewritten (by chunk c + 2's recompute) only in the launch
  // after the one that read it; dh accumulates chunk by chunk as before.
  //
  // With the block skip, each recompute also writes its chunk's flags (one
  // array per gradient buffer), and the contractions take 256-row dW tiles and
  // the compacted K loops that leave the dead blocks out.
  if (pipe) {
    u16* const Gb[2] = {a.G, a.G2};
    int* const Fl[2] = {a.flags, a.flags2};
    auto with_skip = [&](RecArgs r, int v, int par) {
      if (skip) {
        r.flags = Fl[par];
        r.bm = a.bm ? a.bm + (size_t)(v / kTile) * a.M : nullptr;
        r.block_eps = a.block_eps;
      }
      return r;
    };
    {
      RecArgs r = with_skip(rec_args(a, 0, chunks[0].second, a.W, Gb[0]), 0, 0);
      r.qzero = a.queue;  // the first fused launch's queue set
#define CCE_REC(FILT, CAP, SK)                                                                \
  CCE_TIMED(KN_RECOMPUTE_TALL, 2.0 * a.M * a.D * r.vlen, st,                                  \
            hipLaunchKernelGGL((k_recompute_tall<FILT, CAP, SK>), dim3(r.nl), dim3(NT), 0, st, r))
#define CCE_REC_S(FILT, CAP) \
  do { if (skip) CCE_REC(FILT, CAP, true); else CCE_REC(FILT, CAP, false); } while (0)
      if (cap) { if (filt) CCE_REC_S(true, true); else CCE_REC_S(false, true); }
      else { if (filt) CCE_REC_S(true, false); else CCE_REC_S(false, false); }
#undef CCE_REC_S
#undef CCE_REC
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    for (int c = 0; c < nch; ++c) {
      const int v0 = chunks[c].first, vlen = chunks[c].second;
      GemmProb dh, dw;
      DhSplit sp;
      // 384-row dW tiles inside the pipelined launches; the last chunk's
      // contractions run alone, where 256-row dW tiles pack into whole rounds
      // (at 16384 wide: 320 dh tasks of two units and 640 dW tasks of one)
      grads_probs(a, v0, vlen, a.W + (size_t)v0 * a.D, Gb[c & 1], dh, dw, sp,
                  c + 1 < nch && !skip);
      dh.kflags = dw.kflags = Fl[c & 1];
      if (c + 1 < nch) {
        const int v1 = chunks[c + 1].first;
        RecArgs r = with_skip(
            rec_args(a, v1, chunks[c + 1].second, a.W + (size_t)v1 * a.D, Gb[(c + 1) & 1]), v1,
            (c + 1) & 1);
        int* const qset = a.queue + (c & 1) * kQueueSet;
        r.qzero = a.queue + ((c + 1) & 1) * kQueueSet;
        const dim3 grid(dh.nl + dw.nl + (r.nl < kCUs ? r.nl : kCUs));
#define CCE_FUSED(FILT, CAP, SK)                                                              \
  CCE_TIMED(KN_BWD_FUSED, 2.0 * a.M * a.D * (2.0 * vlen + r.vlen), st,                        \
            hipLaunchKernelGGL((k_bwd_fused<FILT, CAP, SK>), grid, dim3(NT), 0, st, dh, dw, r, \
                               qset))
#define CCE_FUSED_S(FILT, CAP) \
  do { if (skip) CCE_FUSED(FILT, CAP, true); else CCE_FUSED(FILT, CAP, false); } while (0)
        if (cap) { if (filt) CCE_FUSED_S(true, true); else CCE_FUSED_S(false, true); }
        else { if (filt) CCE_FUSED_S(true, false); else CCE_FUSED_S(false, false); }
#undef CCE_FUSED_S
#undef CCE_FUSED
      } else {
        const dim3 grid(dh.nl + dw.nl);
        if (skip)
          CCE_TIMED(KN_GRADS, 4.0 * a.M * a.D * vlen, st,
                    hipLaunchKernelGGL((k_grads<true, true>), grid, dim3(NT), 0, st, dh, dw));
        else
          CCE_TIMED(KN_GRADS, 4.0 * a.M * a.D * vlen, st,
                    hipLaunchKernelGGL((k_grads<false, true>), grid, dim3(NT), 0, st, dh, dw));
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = split_reduce(dh, sp, st)) != hipSuccess) return e;
    }
    return launch_target_dw(a, st);
  }

  // Pipelined quantised form (tall recompute, second gradient and chunk
  // buffers): chunk c + 1 is dequantised into the other chunk buffer before
  // launch c, which runs chunk c's dh tasks (no dW: the quantised head is
  // frozen) and chunk c + 1's recompute tiles.  The chunk buffer it overwrites
  // was last read by the dh tasks of launch c - 1, which has finished; the
  // gradient buffers alternate as above.  The dh tiles are not split over K
  // here: the recompute tiles fill the launch's rounds.
  if (tall && a.q.Wq != nullptr && a.G2 != nullptr && a.Wbuf2 != nullptr) {
    u16* const Gb[2] = {a.G, a.G2};
    u16* const Wb[2] = {a.Wbuf, a.Wbuf2};
    if ((e = launch_dequant(a.q, 0, chunks[0].second, a.D, Wb[0], st)) != hipSuccess) return e;
    {
      RecArgs r = rec_args(a, 0, chunks[0].second, Wb[0], Gb[0]);
      r.qzero = a.queue;
#define CCE_REC(FILT, CAP)                                                                    \
  CCE_TIMED(KN_RECOMPUTE_TALL, 2.0 * a.M * a.D * r.vlen, st,                                  \
            hipLaunchKernelGGL((k_recompute_tall<FILT, CAP, false>), dim3(r.nl), dim3(NT), 0, st, r))
      if (cap) { if (filt) CCE_REC(true, true); else CCE_REC(false, true); }
      else { if (filt) CCE_REC(true, false); else CCE_REC(false, false); }
#undef CCE_REC
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    for (int c = 0; c < nch; ++c) {
      const int v0 = chunks[c].first, vlen = chunks[c].second;
      const bool last = c + 1 == nch;
      GemmProb dh, dw;
      DhSplit sp;
      grads_probs(a, v0, vlen, Wb[c & 1], Gb[c & 1], dh, dw, sp, false, !last);
      if (!last) {
        const int v1 = chunks[c + 1].first, vlen1 = chunks[c + 1].second;
        if ((e = launch_dequant(a.q, v1, vlen1, a.D, Wb[(c + 1) & 1], st)) != hipSuccess) return e;
        RecArgs r = rec_args(a, v1, vlen1, Wb[(c + 1) & 1], Gb[(c + 1) & 1]);
        int* const qset = a.queue + (c & 1) * kQueueSet;
        r.qzero = a.queue + ((c + 1) & 1) * kQueueSet;
        dw.nl = 0;  // dh tasks only
        const dim3 grid(dh.nl + (r.nl < kCUs ? r.nl : kCUs));
#define CCE_FUSED(FILT, CAP)                                                                  \
  CCE_TIMED(KN_BWD_FUSED, 2.0 * a.M * a.D * ((double)vlen + r.vlen), st,                      \
            hipLaunchKernelGGL((k_bwd_fused<FILT, CAP, false>), grid, dim3(NT), 0, st, dh, dw, r, \
                               qset))
        if (cap) { if (filt) CCE_FUSED(true, true); else CCE_FUSED(false, true); }
        else { if (filt) CCE_FUSED(true, false); else CCE_FUSED(false, false); }
#undef CCE_FUSED
      } else {
        CCE_TIMED(KN_GRADS, 2.0 * a.M * a.D * vlen, st,
                  hipLaunchKernelGGL((k_grads<false, true>), dim3(dh.nl), dim3(NT), 0, st, dh,
                                     dw));
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = split_reduce(dh, sp, st)) != hipSuccess) return e;
    }
    return hipSuccess;
  }

  for (int c = 0; c < nch; ++c) {
    const int v0 = chunks[c].first, vlen = chunks[c].second;
    const int nvt = (vlen + kTile - 1) / kTile;
    const float* bmc = (a.bm && a.block_eps > 0.f) ? a.bm + (size_t)(v0 / kTile) * a.M : nullptr;
    const u16* Wc = a.q.Wq ? nullptr : a.W + (size_t)v0 * a.D;
    if (a.q.Wq) {  // quantised head: this chunk, dequantised into the chunk buffer
      if ((e = launch_dequant(a.q, v0, vlen, a.D, a.Wbuf, st)) != hipSuccess) return e;
      Wc = a.Wbuf;
    }
    // 1. recompute + gradient tile
    if (tall) {
      const RecArgs r = rec_args(a, v0, vlen, Wc, a.G);
#define CCE_REC(FILT, CAP)                                                                    \
  CCE_TIMED(KN_RECOMPUTE_TALL, 2.0 * a.M * a.D * r.vlen, st,                                  \
            hipLaunchKernelGGL((k_recompute_tall<FILT, CAP, false>), dim3(r.nl), dim3(NT), 0, st, r))
      if (cap) { if (filt) CCE_REC(true, true); else CCE_REC(false, true); }
      else { if (filt) CCE_REC(true, false); else CCE_REC(false, false); }
#undef CCE_REC
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      const int n = pad8(a.nMt * nvt);
#define CCE_RECOMPUTE(VEC, FILT, KT, CAP)                                                          \
  CCE_TIMED(KN_RECOMPUTE, 2.0 * a.M * a.D * vlen, st,                                              \
            hipLaunchKernelGGL((k_recompute<VEC, FILT, KT, CAP>), dim3(n), dim3(NT), 0, st, a.H,   \
                               Wc, a.y, a.lse, a.coef, a.M, a.D, v0, vlen, a.nMt, nvt, a.softcap,  \
                               a.filter_eps, a.block_eps, a.G, a.flags, nkbV, bmc))
#define CCE_RECOMPUTE_F(VEC, KT, CAP)                                                              \
  do {                                                                                             \
    if (filt) CCE_RECOMPUTE(VEC, true, KT, CAP); else CCE_RECOMPUTE(VEC, false, KT, CAP);          \
  } while (0)
      const bool kt = a.D % BK != 0;
      if (!a.vec) {
        if (cap) CCE_RECOMPUTE_F(false, false, true); else CCE_RECOMPUTE_F(false, false, false);
      } else if (kt) {
        if (cap) CCE_RECOMPUTE_F(true, true, true); else CCE_RECOMPUTE_F(true, true, false);
      } else {
        if (cap) CCE_RECOMPUTE_F(true, false, true); else CCE_RECOMPUTE_F(true, false, false);
      }
#undef CCE_RECOMPUTE_F
#undef CCE_RECOMPUTE
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 2. dh (+)= G W[chunk] and dW[chunk] = G^T h in one launch
    //   dh: A = G (row tiles = token tiles, K = nvt*256), B = W[chunk]^T (row tiles = D tiles)
    //   dW: A = G^T (row tiles = chunk vocab tiles, K = Mpad), B = h^T, both read in place
    {
      const bool skip = a.block_eps > 0.f;
      const bool with_dw = a.q.Wq == nullptr;
      GemmProb dh, dw;
      DhSplit sp;
      grads_probs(a, v0, vlen, Wc, a.G, dh, dw, sp);
      // the quantised head is frozen: dh only
      const dim3 grid(with_dw ? dh.nl + dw.nl : dh.nl);
#define CCE_GRADS(SKIP, VEC)                                                                  \
  CCE_TIMED(KN_GRADS, (with_dw ? 4.0 : 2.0) * a.M * a.D * vlen, st,                            \
            hipLaunchKernelGGL((k_grads<SKIP, VEC>), grid, dim3(NT), 0, st, dh, dw))
      if (a.vec) {
        if (skip) CCE_GRADS(true, true); else CCE_GRADS(false, true);
      } else {
        if (skip) CCE_GRADS(true, false); else CCE_GRADS(false, false);
      }
#undef CCE_GRADS
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = split_reduce(dh, sp, st)) != hipSuccess) return e;
    }
  }
  return with_dw_all ? launch_target_dw(a, st) : hipSuccess;
}

}  // namespace cce
