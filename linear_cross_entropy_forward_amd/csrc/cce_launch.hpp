// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef unsigned short u16;

// Per-launch timing (the profiling hook cce_timing_begin / cce_timing_end of
// the C-ABI): every kernel launch is bracketed by timing_pre / timing_post on
// its stream, which record the caller's events when a timing window is open on
// the calling thread and do nothing otherwise.  Kinds name the kernels.
enum LaunchKind : int {
  KN_FWD = 1, KN_FWD_TALL, KN_TARGET_LOGIT, KN_FWD_MERGE,
  KN_EPI_BLOCKS, KN_EPI_PAIRS, KN_EPI_FINAL, KN_EPI_COEF, KN_EPI_INIT,
  KN_RECOMPUTE, KN_RECOMPUTE_TALL, KN_BWD_FUSED, KN_GRADS, KN_SPLIT_REDUCE,
  KN_DEQUANT, KN_TARGET_LOGIT_Q, KN_FWD_FOLD, KN_TARGET_DH, KN_SORT, KN_TARGET_DW,
  KN_COUNT
};
// FLOPS: the launch's algorithmic floating-point operations (2 per multiply-add
// of its contractions; 0 for kernels without one).
void timing_pre(hipStream_t st);
void timing_post(int kind, double flops, hipStream_t st);
#define CCE_TIMED(KIND, FLOPS, ST, ...)       \
  do {                                        \
    ::cce::timing_pre(ST);                    \
    __VA_ARGS__;                              \
    ::cce::timing_post(KIND, (FLOPS), ST);    \
  } while (0)

// Tile size shared by every kernel (rows of each GEMM operand per workgroup).
constexpr int kTile = 256;
// Vocabulary entries per backward chunk: the chunk's bf16 gradient tile
// G[Mpad, kVocabChunk] is the V-independent workspace.
constexpr int kVocabChunk = 16384;
// Doubles per pair in the epilogue's pair table.
constexpr int kPairStride = 16;
// Rows per block of the epilogue's row pass, and the bytes of one run record.
constexpr int kEpiRows = 2048;
constexpr int kEpiRecBytes = 48;
// Compute units of the target chip (MI355X): the workgroups one launch round holds.
constexpr int kCUs = 256;

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
  // null, or the saved block maximum of this launch's vocab range: vocab tile t
  // (relative to W) of token j at bm[t * M + j]
  float* bm;
};
hipError_t launch_forward(const FwdArgs& a, hipStream_t st);
// Forward split: S workgroups per token tile, T vocab tiles each, with
// nMt * S <= kCUs (one round, one workgroup per CU) when nMt <= kCUs.
void fwd_split_tiles(int nMt, int nVt, int& S, int& T);
// The forward's tile launches (full tiles, then a ragged last tile) writing
// `slots` partial (max, sum-exp) slots, and the final merge of `slots` slots.
hipError_t launch_forward_tiles(const FwdArgs& a, int& slots, hipStream_t st);
hipError_t launch_forward_merge(const FwdArgs& a, const float* pm, const float* ps, int slots,
                                hipStream_t st);

// An affine-quantised head: per row v and group g of `group` columns a scale
// and a bias (bf16), codes of `bits` bits packed little-endian in uint32 words
// along the row; value s * q + b.
struct QuantW {
  const unsigned* Wq;
  const u16* scale;
  const u16* bias;
  int bits, group;
};

// Forward over a quantised head: per vocab chunk of at most Vc rows, the chunk
// is dequantised into Wbuf (bf16, [vlen, D]) and run through the forward
// kernels; the chunk's partials fold into run_m / run_s ([Mpad] each).
struct FwdQArgs {
  FwdArgs f;  // f.W is unused; f.V is the whole vocabulary
  QuantW q;
  int Vc;
  u16* Wbuf;
  float* run_m;
  float* run_s;
};
hipError_t launch_forward_quant(const FwdQArgs& a, hipStream_t st);

// Dequantise rows v0 .. v0+vlen of a quantised head into dst ([vlen, D] bf16,
// row-major): fp32 s * q + b, rounded to bf16 (round-to-nearest-even).
hipError_t launch_dequant(const QuantW& q, int v0, int vlen, int D, u16* dst, hipStream_t st);

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
  void* rec;      // run records of the row pass: kEpiRows per block of rows
  int* nruns;     // [blocks]
  int* first;     // [n_pairs]: first and last block holding each pair
  int* last;
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
  u16* G2;     // null, or a second such buffer (the pipelined backward)
  int* flags;  // [nMt, Vc / kTile]
  int* flags2;  // null, or a second such array (the pipelined backward's other gradient buffer)
  unsigned* status;
  // quantised head (q.Wq != null): each chunk is dequantised into Wbuf first,
  // and dW is not formed (the quantised head is frozen; dW may be null)
  QuantW q;
  u16* Wbuf;
  u16* Wbuf2;  // null, or a second chunk buffer (the pipelined quantised backward)
  // null, or the forward's saved block maximum ([ceil(V / 256), M]): with
  // block_eps > 0 a tile's skip is decided from it before its recompute
  const float* bm;
  // split-K partials of the dh contraction: room for P_tiles fp32 256 x 256 tiles
  float* P;
  long long P_tiles;
  // the onehot part of the gradient (taken exactly, outside the bf16 tiles):
  // t_i per row, and the (target, row) sort's two buffer pairs and histogram
  float* tc;
  int* skey[2];
  int* sval[2];
  int* shist;
  float* tF;  // [ceil(M / 64), D]: per window of the sorted rows, a run's first / last piece
  float* tL;
  int* queue;  // kQueueInts: the recompute task queues of the pipelined launches
};
constexpr int kQueueInts = 256;  // two sets of 8 counters, 64 bytes apart
hipError_t launch_backward(const BwdArgs& a, hipStream_t st);
// dh = -t_i W_{y_i} for every row (before the chunks accumulate into it), and
// t / the sort input; then, after the chunks wrote dW, dW_v -= sum t_i h_i over
// each target's rows in row order (bf16 head only).
hipError_t launch_target_dh(const BwdArgs& a, hipStream_t st);
hipError_t launch_target_dw(const BwdArgs& a, hipStream_t st);
// Split of one chunk's dh contraction: the tiles from raster index n_full on are
// computed in ks K-parts (ks = 1: no split); (ks - 1) * (tiles - n_full) partial
// tiles, at most max_tiles.
struct DhSplit {
  int ks;
  int n_full;
};
DhSplit dh_split(int nMt, int nDt, int nvt, bool with_dw, int Mpad, long long max_tiles);

}  // namespace cce
