// ORPO epilogue on the per-row log-probs.
//
// "Training — design (ORPO, flash-CCE head, …)" §1 "The objective" and
// "ORPO training — design", "The objective" / "File-by-file changes":
//   L = NLL + lambda * OR,  OR = -log sigmoid(log_odds),
//   log_odds = (lw - lr) - (log1mexp(lw) - log1mexp(lr)),
//   lw, lr = length-normalised (mean) response log-probs of chosen / rejected,
//   NLL = -lw (response scope) or -((P-1) pm + Mw lw) / ((P-1) + Mw) (full).
// The per-row coefficient coef_i = -dL/dlogp_i feeds the head backward; the
// 1/(1 - e^l) factor of the OR gradient ("ORPO training — design",
// "Recommended defaults") enters through d log_odds / d l.
//
// The same kernels serve the preference-objective family ("Training — design
// …" §8.3 "Objective variants and data"; "ORPO from-base on UltraFeedback —
// results + research directions" §6.1-6.3): per pair a separation
//   s = log_odds (ORPO)  or  s = beta (lw - lr) - gamma (the others),
// a preference term P(s) = softplus(-s) (ORPO, sigmoid / SimPO), s^2 (IPO) or
// max(0, -s) (hinge, derivative 0 at the kink), and
//   L = mean_b (nll_weight NLL_b + lambda P_b).
//
// Each row is read once: a row pass records per-run partial sums (fp64, fixed
// order) for blocks of rows, a pair pass combines each pair's records in block
// order and forms its terms, then the batch means (one workgroup) and the
// per-row coefficients.  Every sum has a fixed order, so results are
// deterministic; the cost is linear in the rows plus the pairs (for pairs
// whose rows are contiguous, the usual layout).
#include <math.h>

#include "cce_launch.hpp"

namespace cce {

enum { P_LW = 0, P_LR, P_PM, P_LO, P_OR, P_NLL, P_CC, P_CR, P_CP, P_ACC, P_NC, P_NR, P_NP, P_BAD };

// log(1 - e^x): two-branch evaluation, clamped below at log(1e-7).
__device__ double log1mexp_d(double x) {
  if (x > -0.6931471805599453) return log(fmax(-expm1(x), 1e-7));
  return log1p(-exp(x));
}
// Its derivative -e^x / (1 - e^x); zero where the clamp binds.
__device__ double dlog1mexp_d(double x) {
  const double om = -expm1(x);
  if (om < 1e-7) return 0.0;
  return -exp(x) / om;
}
__device__ double softplus_d(double x) { return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x)); }
__device__ double sigmoid_d(double x) {
  if (x >= 0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

// Row pass: block k holds rows [kR, kR + R) (R = kEpiRows).  A run is a
// maximal range of consecutive rows of the block with the same pair index; each
// run gets one record (pair, per-kind fp64 sums and counts), written at
// rec[kR + j] for the block's j-th run, with nruns[k] = the block's run count.
// One wave reduces one run at a time (lane l takes rows s + l, s + l + 64, ...
// in order, then a fixed shuffle tree), so every sum has a fixed order.  Rows
// with an invalid pair index take part in no run's sums (status bit).  Each
// pair's first and last block are kept with integer atomic min / max
// (order-independent values).
struct EpiRec {
  int pair, nc, nr, np;
  double sc, sr, sp, pad;
};

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void k_epi_init(int B, int* __restrict__ first,
                                                  int* __restrict__ last) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < B) {
    first[b] = 0x7fffffff;
    last[b] = -1;
  }
}

__global__ __launch_bounds__(256) void k_epi_blocks(const float* __restrict__ logp,
                                                    const int* __restrict__ y,
                                                    const int* __restrict__ seg, int M, int B,
                                                    EpiRec* __restrict__ rec,
                                                    int* __restrict__ nruns,
                                                    int* __restrict__ first,
                                                    int* __restrict__ last, unsigned* status) {
  __shared__ int start[kEpiRows + 1];  // row offsets of the block's run starts (+ end)
  __shared__ int wcnt[4], wbase[4];
  const int k = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r0 = k * kEpiRows, nrow = min(kEpiRows, M - r0);
  constexpr int PER = kEpiRows / 256;  // consecutive rows per thread
  // 1. status checks and run starts; thread t owns rows PER t .. PER t + PER - 1
  int pr[PER + 1];
  unsigned err = 0u;
  pr[0] = -2;
  const int t0 = PER * tid;
  if (t0 > 0 && t0 - 1 < nrow) {
    const int p = seg[r0 + t0 - 1] >> 2;
    pr[0] = (p >= 0 && p < B) ? p : -1;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int r = t0 + u;
    pr[u + 1] = -3;
    if (r < nrow) {
      const int sg = seg[r0 + r];
      const int kind = sg & 3, p = sg >> 2;
      const bool ok = p >= 0 && p < B;
      if (!ok) err |= 2u;                            // CCE_DERR_PAIR
      if (kind != 0 && y[r0 + r] < 0) err |= 1u;     // CCE_DERR_TARGET
      pr[u + 1] = ok ? p : -1;
    }
  }
  if (err) atomicOr(status, err);
  int mystarts = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (t0 + u < nrow && (t0 + u == 0 || pr[u + 1] != pr[u])) ++mystarts;
  // 2. exclusive prefix of the start counts in thread order (wave scan, then waves)
  int incl = mystarts;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wcnt[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int q = 0; q < 4; ++q) {
      wbase[q] = acc;
      acc += wcnt[q];
    }
    start[kEpiRows] = acc;  // the block's run count, parked here for a moment
  }
  __syncthreads();
  int at = wbase[w] + incl - mystarts;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (t0 + u < nrow && (t0 + u == 0 || pr[u + 1] != pr[u])) start[at++] = t0 + u;
  __syncthreads();
  const int nr = start[kEpiRows];
  __syncthreads();
  if (tid == 0) {
    start[nr] = nrow;
    nruns[k] = nr;
  }
  __syncthreads();
  // 3. one wave per run, runs w, w + 4, ...
  for (int j = w; j < nr; j += 4) {
    const int s = start[j], e = start[j + 1];
    const int p0 = seg[r0 + s] >> 2;
    const int p = (p0 >= 0 && p0 < B) ? p0 : -1;
    double sc = 0, sr = 0, sp = 0;
    int nc = 0, nrr = 0, np = 0;
    if (p >= 0) {
      for (int r = s + lane; r < e; r += 64) {
        const int kind = seg[r0 + r] & 3;
        const double lp = (double)logp[r0 + r];
        if (kind == 2) { sc += lp; ++nc; }
        else if (kind == 3) { sr += lp; ++nrr; }
        else if (kind == 1) { sp += lp; ++np; }
      }
    }
    sc = wave_sum_d(sc);
    sr = wave_sum_d(sr);
    sp = wave_sum_d(sp);
    nc = wave_sum_i(nc);
    nrr = wave_sum_i(nrr);
    np = wave_sum_i(np);
    if (lane == 0) {
      EpiRec& R = rec[(size_t)r0 + j];
      R.pair = p;
      R.nc = nc;
      R.nr = nrr;
      R.np = np;
      R.sc = sc;
      R.sr = sr;
      R.sp = sp;
      R.pad = 0.0;
      if (p >= 0) {
        atomicMin(first + p, k);
        atomicMax(last + p, k);
      }
    }
  }
}

// Pair pass: one wave per pair b gathers the records of b from its first to
// its last block, in (block, run) order, then forms the pair's objective and
// coefficients.
__global__ __launch_bounds__(256) void k_epi_pairs(const EpiRec* __restrict__ rec,
                                                   const int* __restrict__ nruns,
                                                   const int* __restrict__ first,
                                                   const int* __restrict__ last, int B,
                                                   int objective, double nll_weight,
                                                   double lambda, double beta, double gamma,
                                                   int scope, double* __restrict__ pairs,
                                                   unsigned* status) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  double sc = 0, sr = 0, sp = 0;
  int nc = 0, nr = 0, np = 0;
  const int k1 = last[b];
  for (int k = first[b]; k <= k1; ++k) {
    const int n = nruns[k];
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const bool hit = j < n && rec[(size_t)k * kEpiRows + j].pair == b;
      unsigned long long m = __ballot(hit);
      while (m) {  // the matching records in order (uniform across the wave)
        const int jj = j0 + __builtin_ctzll(m);
        m &= m - 1ull;
        const EpiRec& R = rec[(size_t)k * kEpiRows + jj];
        sc += R.sc; sr += R.sr; sp += R.sp;
        nc += R.nc; nr += R.nr; np += R.np;
      }
    }
  }
  if (lane != 0) return;
  double* P = pairs + (size_t)b * kPairStride;
  if (nc == 0 || nr == 0) {
    atomicOr(status, 4u);  // CCE_DERR_EMPTY_SPAN
    const double nan = __builtin_nan("");
    for (int q = 0; q < kPairStride; ++q) P[q] = nan;
    P[P_CC] = P[P_CR] = P[P_CP] = 0.0;
    P[P_NC] = nc; P[P_NR] = nr; P[P_NP] = np;
    P[P_BAD] = 1.0;
    return;
  }
  const double lw = sc / nc, lr = sr / nr, pm = np > 0 ? sp / np : 0.0;
  double sep, ds_w, ds_r;  // separation and its derivatives by lw, lr
  if (objective == 0) {
    sep = (lw - lr) - (log1mexp_d(lw) - log1mexp_d(lr));
    ds_w = 1.0 - dlog1mexp_d(lw);
    ds_r = -1.0 + dlog1mexp_d(lr);
  } else {
    sep = beta * (lw - lr) - gamma;
    ds_w = beta;
    ds_r = -beta;
  }
  double pref, dpref;  // preference term and dP/ds
  if (objective == 2) {
    pref = sep * sep;
    dpref = 2.0 * sep;
  } else if (objective == 3) {
    pref = fmax(0.0, -sep);
    dpref = sep < 0.0 ? -1.0 : 0.0;
  } else {
    pref = softplus_d(-sep);
    dpref = -(1.0 - sigmoid_d(sep));
  }
  const double nll = scope == 0 ? -((np > 0 ? np * pm : 0.0) + nc * lw) / (double)(np + nc) : -lw;
  const double w_nll = nll_weight * (scope == 0 ? 1.0 / (double)(np + nc) : 1.0 / (double)nc);
  const double w_pref = -lambda * dpref;  // -dL_b/ds (before 1/B)
  P[P_LW] = lw; P[P_LR] = lr; P[P_PM] = pm; P[P_LO] = sep;
  P[P_OR] = pref;
  P[P_NLL] = nll;
  P[P_CC] = (w_nll + w_pref * ds_w / nc) / B;
  P[P_CR] = (w_pref * ds_r / nr) / B;
  P[P_CP] = scope == 0 ? w_nll / B : 0.0;
  P[P_ACC] = lw > lr ? 1.0 : 0.0;
  P[P_NC] = nc; P[P_NR] = nr; P[P_NP] = np;
  P[P_BAD] = 0.0;
}

__global__ __launch_bounds__(256) void k_epi_final(const double* __restrict__ pairs, int B,
                                                   double nll_weight, double lambda,
                                                   float* __restrict__ out5,
                                                   float* __restrict__ pair_stats,
                                                   unsigned* status) {
  __shared__ double sh[4][256];
  const int tid = threadIdx.x;
  double a[4] = {0, 0, 0, 0};
  for (int b = tid; b < B; b += 256) {
    const double* P = pairs + (size_t)b * kPairStride;
    a[0] += P[P_NLL]; a[1] += P[P_OR]; a[2] += P[P_LO]; a[3] += P[P_ACC];
    if (pair_stats) {
      float* o = pair_stats + 8 * (size_t)b;
      o[0] = (float)P[P_LW];
      o[1] = (float)P[P_LR];
      o[2] = (float)P[P_LO];
      o[3] = (float)P[P_NLL];
      o[4] = (float)P[P_OR];
      o[5] = (float)P[P_NC];
      o[6] = (float)P[P_NR];
      o[7] = (float)P[P_NP];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) sh[q][tid] = a[q];
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off)
#pragma unroll
      for (int q = 0; q < 4; ++q) sh[q][tid] += sh[q][tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    const double nll = sh[0][0] / B, orv = sh[1][0] / B;
    const double loss = nll_weight * nll + lambda * orv;
    out5[0] = (float)loss;
    out5[1] = (float)nll;
    out5[2] = (float)orv;
    out5[3] = (float)(sh[2][0] / B);
    out5[4] = (float)(sh[3][0] / B);
    if (!isfinite(loss)) atomicOr(status, 8u);  // CCE_DERR_NONFINITE
  }
}

__global__ __launch_bounds__(256) void k_epi_coef(const int* __restrict__ seg,
                                                  const double* __restrict__ pairs, int M, int B,
                                                  float* __restrict__ coef) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M) return;
  const int s = seg[i];
  const int kind = s & 3, pr = s >> 2;
  float c = 0.f;
  if (pr >= 0 && pr < B && kind != 0) {
    const double* P = pairs + (size_t)pr * kPairStride;
    c = (float)(kind == 2 ? P[P_CC] : kind == 3 ? P[P_CR] : P[P_CP]);
  }
  coef[i] = c;
}

hipError_t launch_epilogue(const EpiArgs& a, hipStream_t st) {
  const int nblk = (a.M + kEpiRows - 1) / kEpiRows;
  CCE_TIMED(KN_EPI_INIT, 0.0, st,
            hipLaunchKernelGGL(k_epi_init, dim3((a.n_pairs + 255) / 256), dim3(256), 0, st,
                               a.n_pairs, a.first, a.last));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CCE_TIMED(KN_EPI_BLOCKS, 0.0, st,
            hipLaunchKernelGGL(k_epi_blocks, dim3(nblk), dim3(256), 0, st, a.logp, a.y, a.seg,
                               a.M, a.n_pairs, reinterpret_cast<EpiRec*>(a.rec), a.nruns, a.first,
                               a.last, a.status));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CCE_TIMED(KN_EPI_PAIRS, 0.0, st,
            hipLaunchKernelGGL(k_epi_pairs, dim3((a.n_pairs + 3) / 4), dim3(256), 0, st,
                               reinterpret_cast<const EpiRec*>(a.rec), a.nruns, a.first, a.last,
                               a.n_pairs, a.objective, a.nll_weight, a.lambda, a.beta, a.gamma,
                               a.scope, a.pairs, a.status));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CCE_TIMED(KN_EPI_FINAL, 0.0, st,
            hipLaunchKernelGGL(k_epi_final, dim3(1), dim3(256), 0, st, a.pairs, a.n_pairs,
                               a.nll_weight, a.lambda, a.out5, a.pair_stats, a.status));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CCE_TIMED(KN_EPI_COEF, 0.0, st,
            hipLaunchKernelGGL(k_epi_coef, dim3((a.M + 255) / 256), dim3(256), 0, st, a.seg,
                               a.pairs, a.M, a.n_pairs, a.coef));
  return hipGetLastError();
}

}  // namespace cce
