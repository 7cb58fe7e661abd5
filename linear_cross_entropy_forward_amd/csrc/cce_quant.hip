// Affine-quantised head: dequantisation, the target logit, and the chunked
// forward.
//
// "Training — design (ORPO, flash-CCE head, …)" §5.1 (the flash-CCE kernel's
// classifier is the quantised head, 4/8-bit affine, dequantised in-kernel;
// only dh flows back, the head is frozen) and §5.6 "Quantized base" (a vocab
// chunk is a row slice of the quantised weights, scales and biases).  A value
// is s * q + b per group of `group` columns.  Here each vocab chunk is
// dequantised into a bf16 chunk buffer (fp32 s * q + b, rounded to bf16) and
// the bf16 MFMA kernels run on it, so the quantised path shares every
// contraction, softmax and gradient step with the bf16 path; the workspace
// grows by one chunk buffer and stays independent of V.
#include "cce_device.hpp"
#include "cce_launch.hpp"

namespace cce {

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}

// code j of a packed word: bits bits*j .. bits*j + bits - 1
__device__ __forceinline__ float dq_value(unsigned word, int j, int bits, float s, float b) {
  const unsigned q = (word >> (bits * j)) & ((1u << bits) - 1u);
  return fmaf(s, (float)q, b);
}

// One thread per packed word: 8 (4-bit) or 4 (8-bit) consecutive columns.
__global__ __launch_bounds__(256) void k_dequant(const unsigned* __restrict__ Wq,
                                                 const u16* __restrict__ scale,
                                                 const u16* __restrict__ bias, int bits,
                                                 int group, int v0, int vlen, int D,
                                                 u16* __restrict__ dst) {
  const int per = 32 / bits;
  const int words = D / per;  // per row
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)vlen * words) return;
  const int r = (int)(idx / words), wcol = (int)(idx - (long long)r * words);
  const size_t v = (size_t)v0 + r;
  const unsigned word = Wq[v * words + wcol];
  const int d0 = wcol * per;
  const int G = D / group;
  const int g = d0 / group;  // a word never straddles a group (group % per == 0)
  const float s = bf16_to_f32(scale[v * G + g]);
  const float b = bf16_to_f32(bias[v * G + g]);
  u16* out = dst + (size_t)r * D + d0;
  if (bits == 4) {
    unsigned p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      p[k] = pack_bf16x2(dq_value(word, 2 * k, 4, s, b), dq_value(word, 2 * k + 1, 4, s, b));
    *reinterpret_cast<u32x4*>(out) = u32x4{p[0], p[1], p[2], p[3]};
  } else {
    unsigned p[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
      p[k] = pack_bf16x2(dq_value(word, 2 * k, 8, s, b), dq_value(word, 2 * k + 1, 8, s, b));
    *reinterpret_cast<u32x2*>(out) = u32x2{p[0], p[1]};
  }
}

hipError_t launch_dequant(const QuantW& q, int v0, int vlen, int D, u16* dst, hipStream_t st) {
  const long long n = (long long)vlen * (D * q.bits / 32);
  CCE_TIMED(KN_DEQUANT, 0.0, st,
            hipLaunchKernelGGL(k_dequant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, q.Wq,
                               q.scale, q.bias, q.bits, q.group, v0, vlen, D, dst));
  return hipGetLastError();
}

// tgt[i] = h_i . W_{y_i} with W_{y_i} dequantised exactly as in k_dequant
// (bf16-rounded values), then capped when softcap > 0.  One wave per row.
__global__ __launch_bounds__(256) void k_target_logit_q(const u16* __restrict__ H,
                                                        const unsigned* __restrict__ Wq,
                                                        const u16* __restrict__ scale,
                                                        const u16* __restrict__ bias, int bits,
                                                        int group, const int* __restrict__ y,
                                                        int M, int V, int D, float softcap,
                                                        float* __restrict__ tgt) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int yy = y[row];
  if (yy < 0 || yy >= V) return;
  const int per = 32 / bits, words = D / per, G = D / group;
  const u16* hr = H + (size_t)row * D;
  const unsigned* wr = Wq + (size_t)yy * words;
  float acc = 0.f;
  for (int wcol = lane; wcol < words; wcol += 64) {
    const unsigned word = wr[wcol];
    const int d0 = wcol * per;
    const float s = bf16_to_f32(scale[(size_t)yy * G + d0 / group]);
    const float b = bf16_to_f32(bias[(size_t)yy * G + d0 / group]);
    for (int j = 0; j < per; ++j) {
      const float w = bf16_to_f32(to_bf16(dq_value(word, j, bits, s, b)));
      acc = fmaf(bf16_to_f32(hr[d0 + j]), w, acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (softcap > 0.f) acc = softcap * tanh_scaled(acc, 2.f * LOG2E / softcap);
  if (lane == 0) tgt[row] = acc;
}

// Fold S partial (max, sum-exp) slots of this chunk into the running pair of
// each row, slots in order (deterministic).  first: the running pair starts
// empty.
__global__ __launch_bounds__(256) void k_fwd_fold(const float* __restrict__ part_m,
                                                  const float* __restrict__ part_s, int S, int M,
                                                  int Mpad, int first, float* __restrict__ run_m,
                                                  float* __restrict__ run_s) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= M) return;
  float m = first ? NEG_INF : run_m[j];
  float s = first ? 0.f : run_s[j];
  for (int k = 0; k < S; ++k) lse_merge(m, s, part_m[(size_t)k * Mpad + j], part_s[(size_t)k * Mpad + j]);
  run_m[j] = m;
  run_s[j] = s;
}

hipError_t launch_forward_quant(const FwdQArgs& a, hipStream_t st) {
  hipError_t e;
  const FwdArgs& f = a.f;
  for (int v0 = 0; v0 < f.V; v0 += a.Vc) {
    const int vlen = f.V - v0 < a.Vc ? f.V - v0 : a.Vc;
    if ((e = launch_dequant(a.q, v0, vlen, f.D, a.Wbuf, st)) != hipSuccess) return e;
    FwdArgs c = f;
    c.W = a.Wbuf;
    c.V = vlen;
    c.bm = f.bm ? f.bm + (size_t)(v0 / kTile) * f.M : nullptr;
    c.nVt = (vlen + kTile - 1) / kTile;
    c.S = c.T = 0;
    if (vlen / kTile > 0) fwd_split_tiles(c.nMt, vlen / kTile, c.S, c.T);
    int slots = 0;
    if ((e = launch_forward_tiles(c, slots, st)) != hipSuccess) return e;
    CCE_TIMED(KN_FWD_FOLD, 0.0, st,
              hipLaunchKernelGGL(k_fwd_fold, dim3((f.M + 255) / 256), dim3(256), 0, st, f.part_m,
                                 f.part_s, slots, f.M, f.Mpad, v0 == 0 ? 1 : 0, a.run_m, a.run_s));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  CCE_TIMED(KN_TARGET_LOGIT_Q, 2.0 * f.M * f.D, st,
            hipLaunchKernelGGL(k_target_logit_q, dim3((f.M + 3) / 4), dim3(256), 0, st, f.H,
                               a.q.Wq, a.q.scale, a.q.bias, a.q.bits, a.q.group, f.y, f.M, f.V,
                               f.D, f.softcap, f.tgt));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_forward_merge(f, a.run_m, a.run_s, 1, st);
}

}  // namespace cce
