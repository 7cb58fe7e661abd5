// Forward of the flash-CCE head: per-row log-sum-exp over the vocabulary and
// the target logit, without storing the [M, V] logits.
//
// "Training — design (ORPO, flash-CCE head, …)" §5.1 and "ORPO training —
// design", lever 1 "Implementation spec": for each vocab tile take the running
// max m and sum s of exp(z - m), rescaling s when m grows; the target logit
// h_i . W_{y_i}; lse = m + log s, logp = tgt - lse.  With the final-logit
// softcap (same passages; the e4b head) every logit, the target's included,
// is cap * tanh(z / cap) before any of this.
//
// Work split: workgroup (mt, split) owns 256 token rows and a contiguous run of
// T vocab tiles (384 rows each in the tall kernel, 256 in k_fwd).  Each lane
// keeps (m, s) for the 4 tokens it owns across all of its tiles; at the end the
// two lanes and two waves that share a token merge, and the split writes one
// (m, s) pair per token into partials[split][Mpad].  The tall kernel masks the
// rows past V in its last tile (outside the K loop); k_fwd runs full tiles only
// and takes a ragged last tile (V % 256 != 0) in a second launch of the same
// kernel that masks the rows past V and writes one more partial slot.  The
// target logit is one dot product per row, computed by its own small kernel.
// The merge kernel combines the partials of a row in a fixed order: results
// are deterministic and nothing depends on atomics.
//
// Saved block maximum ([P1] §5.1, the blockMax the backward's block skip
// reads): optionally every tile also writes, per token, the largest (capped)
// logit over its 256 vocab rows, bm[tile][token]; the two waves that share a
// token combine through a small double-buffered LDS array, one barrier per
// tile.
#include "cce_device.hpp"
#include "cce_launch.hpp"

namespace cce {

// Online-softmax update of one vocab tile for the 4 tokens this lane owns;
// tmx gets the lane's largest entry per token.  TAIL: the tile runs past V;
// entries with v >= V take no part.
template <bool TAIL>
__device__ __forceinline__ void fwd_tile_update(const floatx16 (&acc)[4][4], int vw, int V, int half,
                                                float (&m_run)[4], float (&s_run)[4],
                                                float (&tmx)[4]) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float mx = NEG_INF;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V);
        if (ok) mx = fmaxf(mx, acc[ii][jj][r]);
      }
    tmx[jj] = mx;
    const float mn = fmaxf(m_run[jj], mx);
    if (TAIL && mn == NEG_INF) continue;  // no valid entry yet for this lane
    const float nb = -mn * LOG2E;
    float sum = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(acc[ii][jj][r], LOG2E, nb));
        if (!TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V)) sum += e;
      }
    s_run[jj] = s_run[jj] * fast_exp2((m_run[jj] - mn) * LOG2E) + sum;
    m_run[jj] = mn;
  }
}

// Workgroup (mt, split) runs vocab tiles [t0 + split*T, min(t0 + (split+1)*T, t1))
// and writes partial slot slot0 + split.  CAP: every logit is replaced by
// softcap * tanh(z / softcap) before the online update.  BM: tile t's per-token
// maximum goes to bm[t * M + token].
template <bool VEC, bool KTAIL, bool TAIL, bool CAP, bool BM>
__global__ __launch_bounds__(NT, 1) void k_fwd(const u16* __restrict__ H, const u16* __restrict__ W,
                                               int M, int V, int D, int nMt, int S, int T, int t0,
                                               int t1, int slot0, int nlaunch, float softcap,
                                               float* __restrict__ part_m,
                                               float* __restrict__ part_s, int Mpad,
                                               float* __restrict__ bm) {
  __shared__ Smem sm;
  __shared__ float bmx[2][TILE];
  int mt, split;
  if (!map_tile(blockIdx.x, nlaunch, nMt, S, 8, mt, split)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;

  float m_run[4], s_run[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    m_run[jj] = NEG_INF;
    s_run[jj] = 0.f;
  }
  const int t_end = min(t0 + (split + 1) * T, t1);
  // 64-wide K-slices: each tile's first loads are issued before the previous
  // tile's epilogue, so they land while it runs
  const bool k64 = VEC && !KTAIL && (D % 64) == 0;
  if (k64 && t0 + split * T < t_end) {
    const int v0 = (t0 + split * T) * TILE;
    gemm_tile64_first(OpRef{W + (size_t)v0 * D, D, min(TILE, V - v0), D},
                      OpRef{H + (size_t)mt * TILE * D, D, min(TILE, M - mt * TILE), D}, sm.raw);
  }

  for (int t = t0 + split * T; t < t_end; ++t) {
    // per-tile operand descriptors are rebuilt from scalars every tile (the
    // empty asm keeps them from being hoisted out of the loop and spilled:
    // a scratch reload in the prologue would wait for every load in flight)
    int mt_ = mt, D_ = D;
    asm volatile("" : "+s"(mt_), "+s"(D_));
    const u16* Hb = H + (size_t)mt_ * TILE * D_;
    const int hrows = min(TILE, M - mt_ * TILE);
    const int v0 = t * TILE;
    floatx16 acc[4][4];
    if (k64) {  // 64-wide K-slices: 128 bytes a row per load
      gemm_tile64<false>(OpRef{W + (size_t)v0 * D_, D_, min(TILE, V - v0), D_},
                         OpRef{Hb, D_, hrows, D_}, D_, sm.raw, acc);
      if (t + 1 < t_end) {
        const int v1 = v0 + TILE;
        gemm_tile64_first(OpRef{W + (size_t)v1 * D_, D_, min(TILE, V - v1), D_},
                          OpRef{Hb, D_, hrows, D_}, sm.raw);
      }
    } else
      gemm_tile<VEC, false, KTAIL>(OpRef{W + (size_t)v0 * D_, D_, min(TILE, V - v0), D_},
                                   OpRef{Hb, D_, hrows, D_}, D_, nullptr, 0, sm, acc);
    if (CAP) {
      const float k2 = 2.f * LOG2E / softcap;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[ii][jj][r] = softcap * tanh_scaled(acc[ii][jj][r], k2);
    }
    float tmx[4];
    fwd_tile_update<TAIL>(acc, v0 + wi * 128, V, half, m_run, s_run, tmx);
    if (BM) {
      // lanes l and l^32 hold the same token, waves wi = 0 and 1 too
      float* xb = bmx[t & 1];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) tmx[jj] = fmaxf(tmx[jj], __shfl_xor(tmx[jj], 32));
      if (wi == 1 && half == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xb[wj * 128 + jj * 32 + lane] = tmx[jj];
      }
      __syncthreads();
      if (wi == 0 && half == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = mt * TILE + wj * 128 + jj * 32 + lane;
          if (j < M) bm[(size_t)t * M + j] = fmaxf(tmx[jj], xb[wj * 128 + jj * 32 + lane]);
        }
      }
    }
  }

  // lanes l and l^32 hold the same token: merge them
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float mo = __shfl_xor(m_run[jj], 32);
    const float so = __shfl_xor(s_run[jj], 32);
    lse_merge(m_run[jj], s_run[jj], mo, so);
  }
  // waves wi = 0 and wi = 1 hold the same tokens (different vocab rows)
  float* xm = reinterpret_cast<float*>(&sm);
  float* xs = xm + 256;
  __syncthreads();
  if (wi == 1 && half == 0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      xm[wj * 128 + jj * 32 + lane] = m_run[jj];
      xs[wj * 128 + jj * 32 + lane] = s_run[jj];
    }
  }
  __syncthreads();
  if (wi == 0 && half == 0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float m = m_run[jj], s = s_run[jj];
      lse_merge(m, s, xm[wj * 128 + jj * 32 + lane], xs[wj * 128 + jj * 32 + lane]);
      const int j = mt * TILE + wj * 128 + jj * 32 + lane;
      part_m[(size_t)(slot0 + split) * Mpad + j] = m;
      part_s[(size_t)(slot0 + split) * Mpad + j] = s;
    }
  }
}

// The tall form of the forward (384 vocab rows x 256 tokens per tile; fewer
// operand bytes per FLOP, otherwise the same algorithm as k_fwd): used when
// the operands allow it (16-byte aligned, D % 32 == 0) and no block maximum is
// saved (that is kept per 256-entry block).  The last tile may run past V: its
// entries with v >= V take no part, so no second launch is needed.
// Online update of the running (m, s) of the 4 tokens of this lane with the
// NI x 16 entries per token of acc (vocab rows vw + ii*32 + ...); TAIL: rows
// >= V take no part.
// CAP: acc holds raw logits and the entries are cap * tanh(z / cap) (k2 =
// 2 log2(e) / cap); the cap is monotonic, so the largest entry is the cap of
// the largest raw logit.
template <int NI, bool TAIL, bool CAP>
__device__ __forceinline__ void fwd_rows_update(const floatx16 (&acc)[NI][4], int vw, int V,
                                                int half, float cap, float k2, float (&m_run)[4],
                                                float (&s_run)[4]) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float mx = NEG_INF;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V);
        if (ok) mx = fmaxf(mx, acc[ii][jj][r]);
      }
    if (CAP && mx != NEG_INF) mx = cap * tanh_scaled(mx, k2);
    const float mn = fmaxf(m_run[jj], mx);
    if (TAIL && mn == NEG_INF) continue;  // no valid entry yet for this lane
    const float nb = -mn * LOG2E;
    float sum = 0.f;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float z = CAP ? cap * tanh_scaled(acc[ii][jj][r], k2) : acc[ii][jj][r];
        const float e = fast_exp2(fmaf(z, LOG2E, nb));
        if (!TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V)) sum += e;
      }
    s_run[jj] = s_run[jj] * fast_exp2((m_run[jj] - mn) * LOG2E) + sum;
    m_run[jj] = mn;
    // one token at a time: the scheduler may not interleave the tokens' exps
    // (that raises the register demand past what the accumulators leave)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Online update with the VGPR part of a tall tile (vocab rows vw .. vw + 63 of
// the wave), read back from LDS where fwd_tall_stash left it: per token, its
// 32 entries, then the same max / sum-exp fold as fwd_rows_update.
template <bool TAIL, bool CAP>
__device__ __forceinline__ void fwd_stash_update(const unsigned char* st, int lane, int vw, int V,
                                                 int half, float cap, float k2, float (&m_run)[4],
                                                 float (&s_run)[4]) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float x[2][16];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 q = *reinterpret_cast<const float4*>(st + (((ii * 4 + jj) * 4 + r4) * 64 + lane) * 16);
        x[ii][4 * r4] = q.x;
        x[ii][4 * r4 + 1] = q.y;
        x[ii][4 * r4 + 2] = q.z;
        x[ii][4 * r4 + 3] = q.w;
      }
    float mx = NEG_INF;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V);
        if (ok) mx = fmaxf(mx, x[ii][r]);
      }
    if (CAP && mx != NEG_INF) mx = cap * tanh_scaled(mx, k2);
    const float mn = fmaxf(m_run[jj], mx);
    if (TAIL && mn == NEG_INF) continue;
    const float nb = -mn * LOG2E;
    float sum = 0.f;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float z = CAP ? cap * tanh_scaled(x[ii][r], k2) : x[ii][r];
        const float e = fast_exp2(fmaf(z, LOG2E, nb));
        if (!TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V)) sum += e;
      }
    s_run[jj] = s_run[jj] * fast_exp2((m_run[jj] - mn) * LOG2E) + sum;
    m_run[jj] = mn;
  }
}

// The VGPR part of a tall tile (8 MFMA tiles, 128 values a lane) into this
// wave's 32 KB of the drained operand ring, as float4 pieces ordered
// [tile][r/4][lane] (consecutive lanes, consecutive 16 bytes): the registers
// are then free before the epilogue reads the AGPR part.
__device__ __forceinline__ void fwd_tall_stash(const AccTall& acc, unsigned char* st, int lane) {
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(st + (((ii * 4 + jj) * 4 + r4) * 64 + lane) * 16) =
            make_float4(acc.v[ii][jj][4 * r4], acc.v[ii][jj][4 * r4 + 1], acc.v[ii][jj][4 * r4 + 2],
                        acc.v[ii][jj][4 * r4 + 3]);
}

// Workgroup (mt, split) runs tall vocab tiles [split*T, min((split+1)*T, nVt))
// and writes partial slot `split`.
template <bool CAP>
__global__ __launch_bounds__(NT, 1) void k_fwd_tall(const u16* __restrict__ H,
                                                    const u16* __restrict__ W, int M, int V, int D,
                                                    int nMt, int S, int T, int nVt, int nlaunch,
                                                    float softcap, float* __restrict__ part_m,
                                                    float* __restrict__ part_s, int Mpad) {
  __shared__ SmemTall sm;
  int mt, split;
  if (!map_tile(blockIdx.x, nlaunch, nMt, S, 8, mt, split)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;

  float m_run[4], s_run[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    m_run[jj] = NEG_INF;
    s_run[jj] = 0.f;
  }
  const int t_end = min((split + 1) * T, nVt);
  for (int t = split * T; t < t_end; ++t) {
    // per-tile descriptors from scalars every tile (not hoisted and spilled)
    int mt_ = mt, D_ = D;
    asm volatile("" : "+s"(mt_), "+s"(D_));
    const u16* Hb = H + (size_t)mt_ * TILE * D_;
    const int hrows = min(TILE, M - mt_ * TILE);
    const int v0 = t * TALL;
    AccTall acc;
    gemm_tile_tall<false>(OpRef{W + (size_t)v0 * D_, D_, min(TALL, V - v0), D_},
                   OpRef{Hb, D_, hrows, D_}, D_, sm, acc);
    const float k2 = CAP ? 2.f * LOG2E / softcap : 0.f;  // the cap is taken in the update
    // the ring is drained (gemm_tile_tall ended with a barrier); each wave
    // parks its VGPR part in its own 32 KB and reads it back itself
    unsigned char* st = sm.raw + w * 32768;
    fwd_tall_stash(acc, st, lane);
    const int vw = v0 + wi * 192;
    if (v0 + TALL > V) {
      fwd_rows_update<4, true, CAP>(acc.a, vw, V, half, softcap, k2, m_run, s_run);
      fwd_stash_update<true, CAP>(st, lane, vw + 128, V, half, softcap, k2, m_run, s_run);
    } else {
      fwd_rows_update<4, false, CAP>(acc.a, vw, V, half, softcap, k2, m_run, s_run);
      fwd_stash_update<false, CAP>(st, lane, vw + 128, V, half, softcap, k2, m_run, s_run);
    }
    __syncthreads();  // every wave's stash read before the next tile's loads fill the ring
  }

  // lanes l and l^32 hold the same token; so do waves wi = 0 and wi = 1
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float mo = __shfl_xor(m_run[jj], 32);
    const float so = __shfl_xor(s_run[jj], 32);
    lse_merge(m_run[jj], s_run[jj], mo, so);
  }
  float* xm = reinterpret_cast<float*>(&sm);
  float* xs = xm + 256;
  __syncthreads();
  if (wi == 1 && half == 0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      xm[wj * 128 + jj * 32 + lane] = m_run[jj];
      xs[wj * 128 + jj * 32 + lane] = s_run[jj];
    }
  }
  __syncthreads();
  if (wi == 0 && half == 0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float m = m_run[jj], s = s_run[jj];
      lse_merge(m, s, xm[wj * 128 + jj * 32 + lane], xs[wj * 128 + jj * 32 + lane]);
      const int j = mt * TILE + wj * 128 + jj * 32 + lane;
      part_m[(size_t)split * Mpad + j] = m;
      part_s[(size_t)split * Mpad + j] = s;
    }
  }
}

// tgt[i] = h_i . W_{y_i} (fp32 sum of exact bf16 products), one wave per row,
// then capped like every other logit when softcap > 0.  Rows whose target is
// outside [0, V) are skipped (the merge reports them).
__global__ __launch_bounds__(256) void k_target_logit(const u16* __restrict__ H,
                                                      const u16* __restrict__ W,
                                                      const int* __restrict__ y, int M, int V,
                                                      int D, float softcap,
                                                      float* __restrict__ tgt) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int yy = y[row];
  if (yy < 0 || yy >= V) return;
  const u16* hr = H + (size_t)row * D;
  const u16* wr = W + (size_t)yy * D;
  float s = 0.f;
  for (int k = lane; k < D; k += 64) {
    const float a = __builtin_bit_cast(float, (unsigned)hr[k] << 16);
    const float b = __builtin_bit_cast(float, (unsigned)wr[k] << 16);
    s = fmaf(a, b, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (softcap > 0.f) s = softcap * tanh_scaled(s, 2.f * LOG2E / softcap);
  if (lane == 0) tgt[row] = s;
}

__global__ __launch_bounds__(256) void k_fwd_merge(const float* __restrict__ part_m,
                                                   const float* __restrict__ part_s,
                                                   const float* __restrict__ tgt,
                                                   const int* __restrict__ y, int M, int V, int S,
                                                   int Mpad, float* __restrict__ logp,
                                                   float* __restrict__ lse, unsigned* status) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= M) return;
  float m = NEG_INF;
  for (int s = 0; s < S; ++s) m = fmaxf(m, part_m[(size_t)s * Mpad + j]);
  float sum = 0.f;
  for (int s = 0; s < S; ++s)
    sum += part_s[(size_t)s * Mpad + j] * exp2f((part_m[(size_t)s * Mpad + j] - m) * LOG2E);
  const float L = m + logf(sum);
  lse[j] = L;
  const int yy = y[j];
  unsigned err = 0u;
  if (yy >= 0 && yy < V) {
    logp[j] = fminf(tgt[j] - L, 0.f);  // log of a probability; rounding can only push it above 0
  } else {
    logp[j] = 0.f;
    if (yy != -1) err |= 1u;  // CCE_DERR_TARGET
  }
  if (!isfinite(L)) err |= 8u;  // CCE_DERR_NONFINITE
  if (err) atomicOr(status, err);
}

template <bool TAIL>
static void launch_fwd_tiles(const FwdArgs& a, int S, int T, int t0, int t1, int slot0,
                             hipStream_t st) {
  const int n = a.nMt * S;
  const double flops = 2.0 * a.M * a.D * (double)(min(a.V, t1 * TILE) - t0 * TILE);
  const int nl = (n + 7) / 8 * 8;
#define CCE_FWD2(VEC, KT, CAP, BM)                                                              \
  CCE_TIMED(KN_FWD, flops, st,                                                                  \
            hipLaunchKernelGGL((k_fwd<VEC, KT, TAIL, CAP, BM>), dim3(nl), dim3(NT), 0, st, a.H,  \
                               a.W, a.M, a.V, a.D, a.nMt, S, T, t0, t1, slot0, nl, a.softcap,    \
                               a.part_m, a.part_s, a.Mpad, a.bm))
#define CCE_FWD(VEC, KT, CAP)                                                                   \
  do {                                                                                          \
    if (a.bm) CCE_FWD2(VEC, KT, CAP, true); else CCE_FWD2(VEC, KT, CAP, false);                \
  } while (0)
  const bool cap = a.softcap > 0.f;
  if (!a.vec) {
    if (cap) CCE_FWD(false, false, true); else CCE_FWD(false, false, false);
  } else if (a.D % BK != 0) {
    if (cap) CCE_FWD(true, true, true); else CCE_FWD(true, true, false);
  } else {
    if (cap) CCE_FWD(true, false, true); else CCE_FWD(true, false, false);
  }
#undef CCE_FWD
#undef CCE_FWD2
}

void fwd_split_tiles(int nMt, int nVt, int& S, int& T) {
  // as many splits per token tile as one round of kCUs workgroups holds (a
  // second, nearly empty round would double the time), then the fewest splits
  // for that many tiles per workgroup
  int smax = kCUs / nMt;
  if (smax < 1) smax = 1;
  if (smax > nVt) smax = nVt;
  T = (nVt + smax - 1) / smax;
  S = (nVt + T - 1) / T;
}

// The 256 x 256 tiles with 64-wide K-slices (k_fwd, D % 64 == 0) stream their
// operands faster than the tall tiles with 32-wide slices, but pay a longer
// prologue per tile: they are taken when each workgroup runs at least 32 vocab
// tiles (the Gemma-4B head: 128), the tall tiles otherwise.
bool fwd_use_tall(const FwdArgs& a) {
  if (!(a.vec && a.D % BK == 0 && a.bm == nullptr)) return false;
  if (a.D % 64 == 0 && a.T >= 32) return false;
  return true;
}

hipError_t launch_forward_tiles(const FwdArgs& a, int& slots, hipStream_t st) {
  if (fwd_use_tall(a)) {
    const int nVt = (a.V + TALL - 1) / TALL;
    int S, T;
    fwd_split_tiles(a.nMt, nVt, S, T);
    const int nl = (a.nMt * S + 7) / 8 * 8;
    if (a.softcap > 0.f)
      CCE_TIMED(KN_FWD_TALL, 2.0 * a.M * a.V * a.D, st,
                hipLaunchKernelGGL(k_fwd_tall<true>, dim3(nl), dim3(NT), 0, st, a.H, a.W, a.M, a.V,
                                   a.D, a.nMt, S, T, nVt, nl, a.softcap, a.part_m, a.part_s, a.Mpad));
    else
      CCE_TIMED(KN_FWD_TALL, 2.0 * a.M * a.V * a.D, st,
                hipLaunchKernelGGL(k_fwd_tall<false>, dim3(nl), dim3(NT), 0, st, a.H, a.W, a.M, a.V,
                                   a.D, a.nMt, S, T, nVt, nl, a.softcap, a.part_m, a.part_s, a.Mpad));
    slots = S;
    return hipGetLastError();
  }
  const int full = a.V / TILE;  // full vocab tiles
  slots = 0;
  if (full > 0) {
    launch_fwd_tiles<false>(a, a.S, a.T, 0, full, 0, st);
    slots = a.S;
  }
  if (a.V % TILE != 0) {
    launch_fwd_tiles<true>(a, 1, 1, full, full + 1, slots, st);
    slots += 1;
  }
  return hipGetLastError();
}

hipError_t launch_forward_merge(const FwdArgs& a, const float* pm, const float* ps, int slots,
                                hipStream_t st) {
  CCE_TIMED(KN_FWD_MERGE, 0.0, st,
            hipLaunchKernelGGL(k_fwd_merge, dim3((a.M + 255) / 256), dim3(256), 0, st, pm, ps,
                               a.tgt, a.y, a.M, a.V, slots, a.Mpad, a.logp, a.lse, a.status));
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, hipStream_t st) {
  int slots = 0;
  hipError_t e = launch_forward_tiles(a, slots, st);
  if (e != hipSuccess) return e;
  CCE_TIMED(KN_TARGET_LOGIT, 2.0 * a.M * a.D, st,
            hipLaunchKernelGGL(k_target_logit, dim3((a.M + 3) / 4), dim3(256), 0, st, a.H, a.W,
                               a.y, a.M, a.V, a.D, a.softcap, a.tgt));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_forward_merge(a, a.part_m, a.part_s, slots, st);
}

}  // namespace cce
