// Forward of the flash-CCE head: per-row log-sum-exp over the vocabulary and
// the target logit, without storing the [M, V] logits.
//
// "Training — design (ORPO, flash-CCE head, …)" §5.1 and "ORPO training —
// design", lever 1 "Implementation spec": for each vocab tile take the running
// max m and sum s of exp(z - m), rescaling s when m grows; capture the target
// logit where the target falls in the tile; lse = m + log s, logp = tgt - lse.
//
// Work split: workgroup (mt, split) owns 256 token rows and a contiguous run of
// T vocab tiles of 256.  Each lane keeps (m, s) for the 4 tokens it owns across
// all of its tiles; at the end the two lanes and two waves that share a token
// merge, and the split writes one (m, s) pair per token into partials[S][Mpad].
// A second kernel merges the S partials of a row in a fixed order, so results
// are deterministic and nothing depends on atomics.
#include "cce_device.hpp"
#include "cce_launch.hpp"

namespace cce {

// Online-softmax update of one vocab tile for the 4 tokens this lane owns.
// TAIL: the tile runs past V; entries with v >= V take no part.
template <bool TAIL>
__device__ __forceinline__ void fwd_tile_update(const floatx16 (&acc)[4][4], int vw, int V, int half,
                                                const int (&yj)[4], float (&m_run)[4],
                                                float (&s_run)[4], float* __restrict__ tgt_row0,
                                                int lane) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    // target capture: the lane holding (token, y) stores the logit; rare, so
    // the per-element compare runs only when some lane of the wave has a hit
    const int off = yj[jj] - vw;
    const bool hit = (unsigned)off < 128u && ((off >> 2) & 1) == half;
    if (__ballot(hit) != 0ull) {
      const int offh = off - 4 * half;
      float tv = 0.f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (offh == ii * 32 + 8 * (r >> 2) + (r & 3)) tv = acc[ii][jj][r];
      if (hit) tgt_row0[jj * 32 + (lane & 31)] = tv;
    }
    float mx = NEG_INF;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V);
        if (ok) mx = fmaxf(mx, acc[ii][jj][r]);
      }
    const float mn = fmaxf(m_run[jj], mx);
    if (mn == NEG_INF) continue;
    const float nb = -mn * LOG2E;
    float sum = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !TAIL || (vw + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) < V);
        const float e = fast_exp2(fmaf(acc[ii][jj][r], LOG2E, nb));
        if (ok) sum += e;
      }
    s_run[jj] = s_run[jj] * fast_exp2((m_run[jj] - mn) * LOG2E) + sum;
    m_run[jj] = mn;
  }
}

template <bool VEC, bool KTAIL>
__global__ __launch_bounds__(NT, 1) void k_fwd(const u16* __restrict__ H, const u16* __restrict__ W,
                                               const int* __restrict__ y, int M, int V, int D,
                                               int nMt, int nVt, int S, int T, int nlaunch,
                                               float* __restrict__ part_m, float* __restrict__ part_s,
                                               float* __restrict__ tgt, int Mpad) {
  __shared__ Smem sm;
  int mt, split;
  if (!map_tile(blockIdx.x, nlaunch, nMt, S, 8, mt, split)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;

  int yj[4];
  float m_run[4], s_run[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = mt * TILE + wj * 128 + jj * 32 + (lane & 31);
    yj[jj] = (j < M) ? y[j] : -1;
    m_run[jj] = NEG_INF;
    s_run[jj] = 0.f;
  }
  const u16* Hb = H + (size_t)mt * TILE * D;
  const int hrows = min(TILE, M - mt * TILE);
  const int t_end = min((split + 1) * T, nVt);
  float* tgt_row0 = tgt + mt * TILE + wj * 128;

  for (int t = split * T; t < t_end; ++t) {
    const int v0 = t * TILE;
    floatx16 acc[4][4];
    gemm_tile<VEC, false, KTAIL>(W + (size_t)v0 * D, D, min(TILE, V - v0), Hb, D, hrows, D, nullptr, 0, sm,
                          acc);
    const int vw = v0 + wi * 128;  // first vocab row of this wave's half of the tile
    if (v0 + TILE > V)
      fwd_tile_update<true>(acc, vw, V, half, yj, m_run, s_run, tgt_row0, lane);
    else
      fwd_tile_update<false>(acc, vw, V, half, yj, m_run, s_run, tgt_row0, lane);
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
      part_m[(size_t)split * Mpad + j] = m;
      part_s[(size_t)split * Mpad + j] = s;
    }
  }
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
    logp[j] = tgt[j] - L;
  } else {
    logp[j] = 0.f;
    if (yy != -1) err |= 1u;  // CCE_DERR_TARGET
  }
  if (!isfinite(L)) err |= 8u;  // CCE_DERR_NONFINITE
  if (err) atomicOr(status, err);
}

hipError_t launch_forward(const FwdArgs& a, hipStream_t st) {
  const int n = a.nMt * a.S;
  const int nlaunch = (n + 7) / 8 * 8;
#define CCE_FWD(VEC, KT)                                                                          \
  hipLaunchKernelGGL((k_fwd<VEC, KT>), dim3(nlaunch), dim3(NT), 0, st, a.H, a.W, a.y, a.M, a.V,     \
                     a.D, a.nMt, a.nVt, a.S, a.T, nlaunch, a.part_m, a.part_s, a.tgt, a.Mpad)
  if (!a.vec) CCE_FWD(false, false);
  else if (a.D % BK != 0) CCE_FWD(true, true);
  else CCE_FWD(true, false);
#undef CCE_FWD
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fwd_merge, dim3((a.M + 255) / 256), dim3(256), 0, st, a.part_m, a.part_s,
                     a.tgt, a.y, a.M, a.V, a.S, a.Mpad, a.logp, a.lse, a.status);
  return hipGetLastError();
}

}  // namespace cce
