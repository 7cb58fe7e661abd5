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
// Three small kernels: per-pair sums (one workgroup per pair, fixed-order fp64
// tree reduction), batch means (one workgroup), per-row coefficients.
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

__global__ __launch_bounds__(256) void k_epi_pairs(const float* __restrict__ logp,
                                                   const int* __restrict__ y,
                                                   const int* __restrict__ seg, int M, int B,
                                                   int objective, double nll_weight,
                                                   double lambda, double beta, double gamma,
                                                   int scope, double* __restrict__ pairs,
                                                   unsigned* status) {
  __shared__ double sh[3][256];
  __shared__ int shn[3][256];
  const int b = blockIdx.x, tid = threadIdx.x;
  double sc = 0, sr = 0, sp = 0;
  int nc = 0, nr = 0, np = 0;
  unsigned err = 0u;
  // Thread tid visits rows tid, tid + 256, tid + 512, ... in that order; the
  // loads of 8 of them are issued together so the scan is not one memory
  // latency per row.
  constexpr int U = 8;
  for (int base = 0; base < M; base += 256 * U) {
    int sv[U], yv[U];
    float lv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * 256 + tid;
      const bool in = i < M;
      sv[u] = in ? seg[i] : -4;  // pair -1: matches no pair, checked by nobody
      lv[u] = in ? logp[i] : 0.f;
      yv[u] = (in && b == 0) ? y[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * 256 + tid >= M) continue;
      const int s = sv[u];
      const int kind = s & 3, pr = s >> 2;
      if (b == 0) {
        if (pr < 0 || pr >= B) err |= 2u;                       // CCE_DERR_PAIR
        if (kind != 0 && yv[u] < 0) err |= 1u;                  // CCE_DERR_TARGET
      }
      if (pr != b) continue;
      const double lp = (double)lv[u];
      if (kind == 2) { sc += lp; ++nc; }
      else if (kind == 3) { sr += lp; ++nr; }
      else if (kind == 1) { sp += lp; ++np; }
    }
  }
  if (err) atomicOr(status, err);
  sh[0][tid] = sc; sh[1][tid] = sr; sh[2][tid] = sp;
  shn[0][tid] = nc; shn[1][tid] = nr; shn[2][tid] = np;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        sh[q][tid] += sh[q][tid + off];
        shn[q][tid] += shn[q][tid + off];
      }
    }
    __syncthreads();
  }
  if (tid != 0) return;
  sc = sh[0][0]; sr = sh[1][0]; sp = sh[2][0];
  nc = shn[0][0]; nr = shn[1][0]; np = shn[2][0];
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
  hipLaunchKernelGGL(k_epi_pairs, dim3(a.n_pairs), dim3(256), 0, st, a.logp, a.y, a.seg, a.M,
                     a.n_pairs, a.objective, a.nll_weight, a.lambda, a.beta, a.gamma, a.scope,
                     a.pairs, a.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_epi_final, dim3(1), dim3(256), 0, st, a.pairs, a.n_pairs, a.nll_weight,
                     a.lambda, a.out5, a.pair_stats, a.status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_epi_coef, dim3((a.M + 255) / 256), dim3(256), 0, st, a.seg, a.pairs, a.M,
                     a.n_pairs, a.coef);
  return hipGetLastError();
}

}  // namespace cce
