// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef unsigned short u16;

// Tile size shared by every kernel (rows of each GEMM operand per workgroup).
constexpr int kTile = 256;
// Vocabulary entries per backward chunk: the chunk's bf16 gradient tile
// G[Mpad, kVocabChunk] is the V-independent workspace.
constexpr int kVocabChunk = 16384;
// Doubles per pair in the epilogue's pair table.
constexpr int kPairStride = 16;

struct FwdArgs {
  const u16* H;
  const u16* W;
  const int* y;
  int M, V, D;
  int nMt, nVt, S, T, Mpad;
  bool vec;
  float softcap;  // 0: off; else logits are softcap * tanh(z / softcap)
  float* part_m;
  float* part_s;
  float* tgt;
  float* logp;
  float* lse;
  unsigned* status;
};
hipError_t launch_forward(const FwdArgs& a, hipStream_t st);

struct EpiArgs {
  const float* logp;
  const int* y;
  const int* seg;
  int M, n_pairs;
  int objective;        // 0 ORPO, 1 sigmoid (SimPO), 2 IPO, 3 hinge
  double nll_weight;    // weight of the NLL term (1 for ORPO)
  double lambda;        // weight of the preference term
  double beta, gamma;   // s = beta (lw - lr) - gamma (objectives other than ORPO)
  int scope;
  double* pairs;  // [n_pairs, kPairStride]
  float* out5;
  float* pair_stats;  // may be null
  float* coef;
  unsigned* status;
};
hipError_t launch_epilogue(const EpiArgs& a, hipStream_t st);

struct BwdArgs {
  const u16* H;
  const u16* W;
  const int* y;
  const float* lse;
  const float* coef;
  int M, V, D;
  int nMt, Mpad, Dpad, Vc;
  bool vec;
  float softcap;  // as in FwdArgs
  float filter_eps, block_eps;
  float* dh;
  float* dW;
  u16* G;      // [Mpad, Vc] bf16, blocked (256 x 32 blocks)
  int* flags;  // [nMt, Vc / kTile]
  unsigned* status;
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t st);

}  // namespace cce
