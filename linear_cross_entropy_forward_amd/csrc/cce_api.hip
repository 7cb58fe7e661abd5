// C-ABI entry points of the flash-CCE head (declared in include/flashcce.h).
//
// Each entry point validates its arguments on the host (before any HIP call,
// so argument errors can be checked without a GPU), checks that the current
// device is gfx950, carves the caller's workspace, and enqueues its kernels on
// the caller's stream.  Nothing is allocated here.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "flashcce.h"
#include "cce_launch.hpp"

namespace {

using cce::kTile;
using cce::kVocabChunk;

constexpr int64_t kMaxM = int64_t(1) << 21;  // keeps 256 * Mpad * 2 bytes < 2^31
constexpr int64_t kMaxV = int64_t(1) << 30;
constexpr int64_t kMaxD = 65536;
constexpr size_t kAlign = 256;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool sizes_ok(int64_t M, int64_t V, int64_t D) {
  return M >= 1 && V >= 1 && D >= 1 && M <= kMaxM && V <= kMaxV && D <= kMaxD;
}

// Upper bound of the partial slots over all V for this M (so the workspace does
// not grow with V): the splits over the full vocab tiles plus one slot for a
// ragged last tile.
int64_t fwd_split_cap(int64_t nMt) { return 256 / nMt + 2; }

struct Layout {
  int64_t Mpad, Dpad, Vc, nMt;
  size_t part_m, part_s, tgt, pairs, g, flags, flags2;
  size_t epi_rec, epi_nruns, epi_first, epi_last, epi_end;  // the epilogue's row-pass state
  size_t tc, skey[2], sval[2], shist, tF, tL;  // the backward's exact onehot part
  size_t queue;  // the pipelined backward's task-queue counters
  size_t g2;  // the second gradient buffer of the pipelined backward (0: none)
  size_t psplit;  // split-K partial tiles of dh (psplit_tiles of 256 x 256 fp32)
  long long psplit_tiles;
  size_t total;
  // quantised head only: running (max, sum-exp), the bf16 chunk buffer and its
  // own dh partials (no dW there, so dh splits further)
  size_t run_m, run_s, wbuf, psplit_q;
  size_t g2q, wbuf2;  // the pipelined quantised backward's second G and chunk buffers (0: none)
  long long psplit_tiles_q;
  size_t total_q;
  int64_t vcf;  // rows of the quantised forward's dequantised chunk
};

// dh split-K partial tiles reserved for a full vocab chunk: as many as its
// split schedule needs, within half the gradient chunk's bytes.
long long split_tiles(const Layout& L, bool with_dw) {
  const long long tile = (long long)kTile * kTile * 4;
  const long long cap = (long long)L.Mpad * L.Vc * 2 / 2 / tile;
  const int nMt = (int)L.nMt, nDt = (int)(L.Dpad / kTile);
  const cce::DhSplit sp =
      cce::dh_split(nMt, nDt, (int)(L.Vc / kTile), with_dw, (int)L.Mpad, cap);
  return (long long)(sp.ks - 1) * ((long long)nMt * nDt - sp.n_full);
}

Layout layout(int64_t M, int64_t V, int64_t D) {
  Layout L{};
  L.nMt = (M + kTile - 1) / kTile;
  L.Mpad = L.nMt * kTile;
  L.Dpad = round_up(D, kTile);
  L.Vc = round_up(V, kTile) < kVocabChunk ? round_up(V, kTile) : kVocabChunk;
  const int64_t Scap = fwd_split_cap(L.nMt);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.part_m = take((size_t)Scap * L.Mpad * sizeof(float));
  L.part_s = take((size_t)Scap * L.Mpad * sizeof(float));
  L.tgt = take((size_t)L.Mpad * sizeof(float));
  L.pairs = take((size_t)L.Mpad * cce::kPairStride * sizeof(double));
  {
    const int64_t nblk = (M + cce::kEpiRows - 1) / cce::kEpiRows;
    L.epi_rec = take((size_t)nblk * cce::kEpiRows * cce::kEpiRecBytes);
    L.epi_nruns = take((size_t)nblk * sizeof(int));
    L.epi_first = take((size_t)L.Mpad * sizeof(int));
    L.epi_last = take((size_t)L.Mpad * sizeof(int));
    L.epi_end = off;
  }
  L.tc = take((size_t)L.Mpad * sizeof(float));
  for (int q = 0; q < 2; ++q) {
    L.skey[q] = take((size_t)L.Mpad * sizeof(int));
    L.sval[q] = take((size_t)L.Mpad * sizeof(int));
  }
  L.shist = take((size_t)256 * ((M + 2047) / 2048) * sizeof(int));
  L.tF = take((size_t)((M + 63) / 64) * D * sizeof(float));
  L.tL = take((size_t)((M + 63) / 64) * D * sizeof(float));
  L.queue = take((size_t)cce::kQueueInts * sizeof(int));
  L.g = take((size_t)L.Mpad * L.Vc * 2);
  L.flags = take((size_t)L.nMt * (L.Vc / kTile) * sizeof(int));
  L.flags2 = take((size_t)L.nMt * (L.Vc / kTile) * sizeof(int));
  const size_t base = off;
  // the pipelined backward (tall recompute tiles, D % 32 == 0) alternates
  // between two gradient buffers
  L.g2 = D % 32 == 0 ? take((size_t)L.Mpad * L.Vc * 2) : 0;
  L.psplit_tiles = split_tiles(L, true);
  L.psplit = take((size_t)L.psplit_tiles * kTile * kTile * 4);
  L.total = off;
  off = base;  // the quantised layout does not use the bf16 head's partials
  L.run_m = take((size_t)L.Mpad * sizeof(float));
  L.run_s = take((size_t)L.Mpad * sizeof(float));
  L.wbuf = take((size_t)L.Vc * D * 2);
  // the pipelined quantised backward (tall tiles, D % 32 == 0) alternates
  // between two gradient buffers and two dequantised chunk buffers
  L.g2q = D % 32 == 0 ? take((size_t)L.Mpad * L.Vc * 2) : 0;
  L.wbuf2 = D % 32 == 0 ? take((size_t)L.Vc * D * 2) : 0;
  L.psplit_tiles_q = split_tiles(L, false);
  L.psplit_q = take((size_t)L.psplit_tiles_q * kTile * kTile * 4);
  L.total_q = off;
  // the quantised forward dequantises into the chunk and gradient buffers that
  // follow one another from wbuf (the backward's, free during the forward):
  // as few equal chunks of whole 256-row tiles as that region holds, so each
  // launch runs many vocab tiles per workgroup
  {
    const size_t row = (size_t)D * 2;
    const size_t region = (L.wbuf2 ? L.wbuf2 : L.wbuf) + (size_t)L.Vc * row - L.wbuf;
    const int64_t cap_rows = std::max<int64_t>(L.Vc, (int64_t)(region / row) / kTile * kTile);
    const int64_t Vpad = round_up(V, kTile);
    const int64_t nch = (Vpad + cap_rows - 1) / cap_rows;
    L.vcf = round_up((Vpad + nch - 1) / nch, kTile);
  }
  return L;
}

// gfx950 check of the current device, cached per device id.
cce_status device_ok() {
  static std::mutex mu;
  static int cache[64];  // 0 unknown, 1 ok, 2 not ok
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CCE_EDEVICE;
  if (dev < 64) {
    std::lock_guard<std::mutex> g(mu);
    if (cache[dev] != 0) return cache[dev] == 1 ? CCE_OK : CCE_EDEVICE;
  }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return CCE_EDEVICE;
  const bool ok = strncmp(p.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> g(mu);
    cache[dev] = ok ? 1 : 2;
  }
  return ok ? CCE_OK : CCE_EDEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void set_target_regions(cce::BwdArgs& a, const Layout& L, char* base) {
  a.tc = reinterpret_cast<float*>(base + L.tc);
  for (int q = 0; q < 2; ++q) {
    a.skey[q] = reinterpret_cast<int*>(base + L.skey[q]);
    a.sval[q] = reinterpret_cast<int*>(base + L.sval[q]);
  }
  a.shist = reinterpret_cast<int*>(base + L.shist);
  a.tF = reinterpret_cast<float*>(base + L.tF);
  a.tL = reinterpret_cast<float*>(base + L.tL);
  a.queue = reinterpret_cast<int*>(base + L.queue);
}

// Scratch of the no-allocation forward (cce_forward_noalloc): one array per
// device, held for the life of the process.  Host code never uses its name as
// an address: each device's copy is found with hipGetSymbolAddress (once per
// device, with that device current) and only that pointer is passed on.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int64_t kNoAllocMaxM = 786432;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Forward-only layout: partial (max, sum-exp) slots and the target logits.
struct FwdLayout {
  int64_t Mpad, nMt;
  size_t part_m, part_s, tgt, total;
};
FwdLayout fwd_layout(int64_t M) {
  FwdLayout L{};
  L.nMt = (M + kTile - 1) / kTile;
  L.Mpad = L.nMt * kTile;
  const int64_t Scap = fwd_split_cap(L.nMt);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.part_m = take((size_t)Scap * L.Mpad * sizeof(float));
  L.part_s = take((size_t)Scap * L.Mpad * sizeof(float));
  L.tgt = take((size_t)L.Mpad * sizeof(float));
  L.total = off;
  return L;
}
static_assert(kNoAllocMaxM <= kMaxM, "no-allocation row limit within the library's");

// This device's scratch address (cached per device id); null on failure.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// The calling thread's timing window (cce_timing_begin .. cce_timing_end).
struct TimingLog {
  void* const* ev;  // 2 * cap caller-owned events: before / after launch i
  int32_t* kinds;   // cap entries
  double* flops;    // cap entries, or null
  int32_t cap, n;
  bool on, failed;
};
thread_local TimingLog g_tlog{};

}  // namespace

namespace cce {
void timing_pre(hipStream_t st) {
  TimingLog& t = g_tlog;
  if (!t.on || t.n >= t.cap) return;
  if (hipEventRecord(static_cast<hipEvent_t>(t.ev[2 * t.n]), st) != hipSuccess) t.failed = true;
}
void timing_post(int kind, double flops, hipStream_t st) {
  TimingLog& t = g_tlog;
  if (!t.on || t.n >= t.cap) return;
  if (hipEventRecord(static_cast<hipEvent_t>(t.ev[2 * t.n + 1]), st) != hipSuccess) t.failed = true;
  if (t.flops) t.flops[t.n] = flops;
  t.kinds[t.n++] = kind;
}
}  // namespace cce

extern "C" {

int cce_abi_version(void) { return 6; }

cce_status cce_timing_begin(void* const* events, int32_t* kinds, double* flops,
                            int32_t capacity) {
  if (!events || !kinds || capacity < 1) return CCE_EINVAL;
  for (int32_t i = 0; i < 2 * capacity; ++i)
    if (!events[i]) return CCE_EINVAL;
  g_tlog = TimingLog{events, kinds, flops, capacity, 0, true, false};
  return CCE_OK;
}

int32_t cce_timing_end(void) {
  TimingLog& t = g_tlog;
  const int32_t n = t.on && !t.failed ? t.n : -1;
  t = TimingLog{};
  return n;
}

const char* cce_kernel_name(int32_t kind) {
  switch (kind) {
    case cce::KN_FWD: return "k_fwd";
    case cce::KN_FWD_TALL: return "k_fwd_tall";
    case cce::KN_TARGET_LOGIT: return "k_target_logit";
    case cce::KN_FWD_MERGE: return "k_fwd_merge";
    case cce::KN_EPI_BLOCKS: return "k_epi_blocks";
    case cce::KN_EPI_PAIRS: return "k_epi_pairs";
    case cce::KN_EPI_FINAL: return "k_epi_final";
    case cce::KN_EPI_COEF: return "k_epi_coef";
    case cce::KN_EPI_INIT: return "k_epi_init";
    case cce::KN_RECOMPUTE: return "k_recompute";
    case cce::KN_RECOMPUTE_TALL: return "k_recompute_tall";
    case cce::KN_BWD_FUSED: return "k_bwd_fused";
    case cce::KN_GRADS: return "k_grads";
    case cce::KN_SPLIT_REDUCE: return "k_split_reduce";
    case cce::KN_DEQUANT: return "k_dequant";
    case cce::KN_TARGET_LOGIT_Q: return "k_target_logit_q";
    case cce::KN_FWD_FOLD: return "k_fwd_fold";
    case cce::KN_TARGET_DH: return "k_target_dh";
    case cce::KN_SORT: return "k_sort";
    case cce::KN_TARGET_DW: return "k_target_dw";
    default: return "unknown";
  }
}

const char* cce_status_string(int status) {
  switch (status) {
    case CCE_OK: return "CCE_OK";
    case CCE_EINVAL: return "CCE_EINVAL: invalid argument (null pointer, bad enum or non-finite scalar)";
    case CCE_ESHAPE: return "CCE_ESHAPE: invalid sizes";
    case CCE_EWORKSPACE: return "CCE_EWORKSPACE: workspace too small or misaligned";
    case CCE_EDEVICE: return "CCE_EDEVICE: current device is not gfx950";
    case CCE_ELAUNCH: return "CCE_ELAUNCH: kernel launch failed";
    default: return "unknown cce_status";
  }
}

size_t cce_workspace_bytes(int64_t M, int64_t V, int64_t D) {
  if (!sizes_ok(M, V, D)) return 0;
  return layout(M, V, D).total;
}

size_t cce_workspace_bytes_q(int64_t M, int64_t V, int64_t D) {
  if (!sizes_ok(M, V, D)) return 0;
  return layout(M, V, D).total_q;
}

cce_status cce_forward(const void* h, const void* W, const int32_t* y, int64_t M, int64_t V,
                       int64_t D, float softcap, float* logp, float* lse, float* block_max,
                       uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  if (!h || !W || !y || !logp || !lse || !dev_status || !ws) return CCE_EINVAL;
  if (!(softcap >= 0.f) || !isfinite(softcap)) return CCE_EINVAL;
  if (!sizes_ok(M, V, D)) return CCE_ESHAPE;
  const Layout L = layout(M, V, D);
  if (ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return CCE_EWORKSPACE;
  const cce_status ds = device_ok();
  if (ds != CCE_OK) return ds;
  char* base = static_cast<char*>(ws);
  cce::FwdArgs a{};
  a.H = static_cast<const cce::u16*>(h);
  a.W = static_cast<const cce::u16*>(W);
  a.y = y;
  a.M = (int)M;
  a.V = (int)V;
  a.D = (int)D;
  a.nMt = (int)L.nMt;
  a.nVt = (int)((V + kTile - 1) / kTile);
  a.S = a.T = 0;
  if (V / kTile > 0) cce::fwd_split_tiles(a.nMt, (int)(V / kTile), a.S, a.T);  // full vocab tiles
  a.Mpad = (int)L.Mpad;
  a.vec = (D % 8 == 0) && aligned16(h) && aligned16(W);
  a.softcap = softcap;
  a.part_m = reinterpret_cast<float*>(base + L.part_m);
  a.part_s = reinterpret_cast<float*>(base + L.part_s);
  a.tgt = reinterpret_cast<float*>(base + L.tgt);
  a.logp = logp;
  a.lse = lse;
  a.status = dev_status;
  a.bm = block_max;
  return cce::launch_forward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? CCE_OK
                                                                               : CCE_ELAUNCH;
}

cce_status cce_forward_noalloc(const void* h, const void* W, const int32_t* y, int64_t M,
                               int64_t V, int64_t D, float softcap, float* logp, float* lse,
                               float* block_max, uint32_t* dev_status, void* stream) {
  if (!h || !W || !y || !logp || !lse || !dev_status) return CCE_EINVAL;
  if (!(softcap >= 0.f) || !isfinite(softcap)) return CCE_EINVAL;
  if (!sizes_ok(M, V, D) || M > kNoAllocMaxM) return CCE_ESHAPE;
  const FwdLayout L = fwd_layout(M);
  if (L.total > kScratchBytes) return CCE_ESHAPE;
  const cce_status ds = device_ok();
  if (ds != CCE_OK) return ds;
  char* base = static_cast<char*>(scratch_ptr());
  if (!base) return CCE_EDEVICE;
  cce::FwdArgs a{};
  a.H = static_cast<const cce::u16*>(h);
  a.W = static_cast<const cce::u16*>(W);
  a.y = y;
  a.M = (int)M;
  a.V = (int)V;
  a.D = (int)D;
  a.nMt = (int)L.nMt;
  a.nVt = (int)((V + kTile - 1) / kTile);
  a.S = a.T = 0;
  if (V / kTile > 0) cce::fwd_split_tiles(a.nMt, (int)(V / kTile), a.S, a.T);
  a.Mpad = (int)L.Mpad;
  a.vec = (D % 8 == 0) && aligned16(h) && aligned16(W);
  a.softcap = softcap;
  a.part_m = reinterpret_cast<float*>(base + L.part_m);
  a.part_s = reinterpret_cast<float*>(base + L.part_s);
  a.tgt = reinterpret_cast<float*>(base + L.tgt);
  a.logp = logp;
  a.lse = lse;
  a.status = dev_status;
  a.bm = block_max;
  return cce::launch_forward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? CCE_OK
                                                                               : CCE_ELAUNCH;
}

// Both epilogue entry points: argument checks, then the same kernels.
static cce_status epilogue_common(const float* logp, const int32_t* y, const int32_t* seg,
                                  int64_t M, int32_t n_pairs, int objective, float nll_weight,
                                  float lambda, float beta, float gamma, int scope, float* out5,
                                  float* pair_stats, float* coef, uint32_t* dev_status, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!logp || !y || !seg || !out5 || !coef || !dev_status || !ws) return CCE_EINVAL;
  if (scope != CCE_SCOPE_FULL && scope != CCE_SCOPE_RESPONSE) return CCE_EINVAL;
  if (objective < CCE_OBJ_ORPO || objective > CCE_OBJ_HINGE) return CCE_EINVAL;
  if (!isfinite(lambda) || !isfinite(nll_weight) || !isfinite(beta) || !isfinite(gamma))
    return CCE_EINVAL;
  if (M < 1 || M > kMaxM || n_pairs < 1 || (int64_t)n_pairs > M) return CCE_ESHAPE;
  // the epilogue's part of the workspace depends on M only; any V, D >= 1 give it
  const Layout L = layout(M, 1, 1);
  if (ws_bytes < L.epi_end || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return CCE_EWORKSPACE;
  const cce_status ds = device_ok();
  if (ds != CCE_OK) return ds;
  cce::EpiArgs a{};
  a.logp = logp;
  a.y = y;
  a.seg = seg;
  a.M = (int)M;
  a.n_pairs = n_pairs;
  a.objective = objective;
  a.nll_weight = (double)nll_weight;
  a.lambda = (double)lambda;
  a.beta = (double)beta;
  a.gamma = (double)gamma;
  a.scope = scope;
  char* base = static_cast<char*>(ws);
  a.pairs = reinterpret_cast<double*>(base + L.pairs);
  a.rec = base + L.epi_rec;
  a.nruns = reinterpret_cast<int*>(base + L.epi_nruns);
  a.first = reinterpret_cast<int*>(base + L.epi_first);
  a.last = reinterpret_cast<int*>(base + L.epi_last);
  a.out5 = out5;
  a.pair_stats = pair_stats;
  a.coef = coef;
  a.status = dev_status;
  return cce::launch_epilogue(a, static_cast<hipStream_t>(stream)) == hipSuccess ? CCE_OK
                                                                                : CCE_ELAUNCH;
}

cce_status orpo_epilogue(const float* logp, const int32_t* y, const int32_t* seg, int64_t M,
                         int32_t n_pairs, float lambda, int scope, float* out5, float* pair_stats,
                         float* coef, uint32_t* dev_status, void* ws, size_t ws_bytes,
                         void* stream) {
  return epilogue_common(logp, y, seg, M, n_pairs, CCE_OBJ_ORPO, 1.f, lambda, 0.f, 0.f, scope,
                         out5, pair_stats, coef, dev_status, ws, ws_bytes, stream);
}

cce_status pref_epilogue(const float* logp, const int32_t* y, const int32_t* seg, int64_t M,
                         int32_t n_pairs, int objective, float nll_weight, float lambda,
                         float beta, float gamma, int scope, float* out5, float* pair_stats,
                         float* coef, uint32_t* dev_status, void* ws, size_t ws_bytes,
                         void* stream) {
  return epilogue_common(logp, y, seg, M, n_pairs, objective, nll_weight, lambda, beta, gamma,
                         scope, out5, pair_stats, coef, dev_status, ws, ws_bytes, stream);
}

cce_status cce_backward(const void* h, const void* W, const int32_t* y, const float* lse,
                        const float* coef, const float* block_max, int64_t M, int64_t V,
                        int64_t D, float softcap,
                        float filter_eps, float block_eps, float* dh, float* dW,
                        uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  if (!h || !W || !y || !lse || !coef || !dh || !dW || !dev_status || !ws) return CCE_EINVAL;
  if (!(softcap >= 0.f) || !isfinite(softcap)) return CCE_EINVAL;
  if (!(filter_eps >= 0.f) || !(block_eps >= 0.f) || !isfinite(filter_eps) || !isfinite(block_eps))
    return CCE_EINVAL;
  if (!sizes_ok(M, V, D)) return CCE_ESHAPE;
  const Layout L = layout(M, V, D);
  if (ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return CCE_EWORKSPACE;
  const cce_status ds = device_ok();
  if (ds != CCE_OK) return ds;
  char* base = static_cast<char*>(ws);
  cce::BwdArgs a{};
  a.H = static_cast<const cce::u16*>(h);
  a.W = static_cast<const cce::u16*>(W);
  a.y = y;
  a.lse = lse;
  a.coef = coef;
  a.M = (int)M;
  a.V = (int)V;
  a.D = (int)D;
  a.nMt = (int)L.nMt;
  a.Mpad = (int)L.Mpad;
  a.Dpad = (int)L.Dpad;
  a.Vc = (int)L.Vc;
  a.vec = (D % 8 == 0) && aligned16(h) && aligned16(W);
  a.softcap = softcap;
  a.filter_eps = filter_eps;
  a.block_eps = block_eps;
  a.dh = dh;
  a.dW = dW;
  a.G = reinterpret_cast<cce::u16*>(base + L.g);
  a.G2 = L.g2 ? reinterpret_cast<cce::u16*>(base + L.g2) : nullptr;
  a.flags = reinterpret_cast<int*>(base + L.flags);
  a.flags2 = reinterpret_cast<int*>(base + L.flags2);
  a.status = dev_status;
  a.bm = block_max;
  a.P = reinterpret_cast<float*>(base + L.psplit);
  a.P_tiles = L.psplit_tiles;
  set_target_regions(a, L, base);
  return cce::launch_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? CCE_OK
                                                                                : CCE_ELAUNCH;
}

static bool quant_ok(const void* Wq, const void* scales, const void* biases, int bits,
                     int group_size, int64_t D) {
  if (!Wq || !scales || !biases) return false;
  if (bits != 4 && bits != 8) return false;
  if (group_size != 32 && group_size != 64 && group_size != 128) return false;
  return D % group_size == 0;
}

cce_status cce_forward_q(const void* h, const uint32_t* Wq, const void* scales, const void* biases,
                         int bits, int group_size, const int32_t* y, int64_t M, int64_t V,
                         int64_t D, float softcap, float* logp, float* lse, float* block_max,
                         uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  if (!h || !y || !logp || !lse || !dev_status || !ws) return CCE_EINVAL;
  if (!(softcap >= 0.f) || !isfinite(softcap)) return CCE_EINVAL;
  if (!sizes_ok(M, V, D)) return CCE_ESHAPE;
  if (!quant_ok(Wq, scales, biases, bits, group_size, D)) return CCE_EINVAL;
  const Layout L = layout(M, V, D);
  if (ws_bytes < L.total_q || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return CCE_EWORKSPACE;
  const cce_status ds = device_ok();
  if (ds != CCE_OK) return ds;
  char* base = static_cast<char*>(ws);
  cce::FwdQArgs a{};
  a.f.H = static_cast<const cce::u16*>(h);
  a.f.W = nullptr;
  a.f.y = y;
  a.f.M = (int)M;
  a.f.V = (int)V;
  a.f.D = (int)D;
  a.f.nMt = (int)L.nMt;
  a.f.Mpad = (int)L.Mpad;
  a.f.vec = (D % 8 == 0) && aligned16(h);  // the chunk buffer is aligned by construction
  a.f.softcap = softcap;
  a.f.part_m = reinterpret_cast<float*>(base + L.part_m);
  a.f.part_s = reinterpret_cast<float*>(base + L.part_s);
  a.f.tgt = reinterpret_cast<float*>(base + L.tgt);
  a.f.logp = logp;
  a.f.lse = lse;
  a.f.status = dev_status;
  a.f.bm = block_max;
  a.q = cce::QuantW{reinterpret_cast<const unsigned*>(Wq), static_cast<const cce::u16*>(scales),
                    static_cast<const cce::u16*>(biases), bits, group_size};
  a.Vc = (int)L.vcf;
  a.Wbuf = reinterpret_cast<cce::u16*>(base + L.wbuf);
  a.run_m = reinterpret_cast<float*>(base + L.run_m);
  a.run_s = reinterpret_cast<float*>(base + L.run_s);
  return cce::launch_forward_quant(a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? CCE_OK
             : CCE_ELAUNCH;
}

cce_status cce_backward_q(const void* h, const uint32_t* Wq, const void* scales,
                          const void* biases, int bits, int group_size, const int32_t* y,
                          const float* lse, const float* coef, const float* block_max, int64_t M,
                          int64_t V, int64_t D, float softcap, float filter_eps, float block_eps,
                          float* dh,
                          uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  if (!h || !y || !lse || !coef || !dh || !dev_status || !ws) return CCE_EINVAL;
  if (!(softcap >= 0.f) || !isfinite(softcap)) return CCE_EINVAL;
  if (!(filter_eps >= 0.f) || !(block_eps >= 0.f) || !isfinite(filter_eps) || !isfinite(block_eps))
    return CCE_EINVAL;
  if (!sizes_ok(M, V, D)) return CCE_ESHAPE;
  if (!quant_ok(Wq, scales, biases, bits, group_size, D)) return CCE_EINVAL;
  const Layout L = layout(M, V, D);
  if (ws_bytes < L.total_q || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return CCE_EWORKSPACE;
  const cce_status ds = device_ok();
  if (ds != CCE_OK) return ds;
  char* base = static_cast<char*>(ws);
  cce::BwdArgs a{};
  a.H = static_cast<const cce::u16*>(h);
  a.W = nullptr;
  a.y = y;
  a.lse = lse;
  a.coef = coef;
  a.M = (int)M;
  a.V = (int)V;
  a.D = (int)D;
  a.nMt = (int)L.nMt;
  a.Mpad = (int)L.Mpad;
  a.Dpad = (int)L.Dpad;
  a.Vc = (int)L.Vc;
  a.vec = (D % 8 == 0) && aligned16(h);
  a.softcap = softcap;
  a.filter_eps = filter_eps;
  a.block_eps = block_eps;
  a.dh = dh;
  a.dW = nullptr;
  a.G = reinterpret_cast<cce::u16*>(base + L.g);
  a.flags = reinterpret_cast<int*>(base + L.flags);
  a.flags2 = reinterpret_cast<int*>(base + L.flags2);
  a.status = dev_status;
  a.bm = block_max;
  a.P = reinterpret_cast<float*>(base + L.psplit_q);
  a.P_tiles = L.psplit_tiles_q;
  set_target_regions(a, L, base);
  a.q = cce::QuantW{reinterpret_cast<const unsigned*>(Wq), static_cast<const cce::u16*>(scales),
                    static_cast<const cce::u16*>(biases), bits, group_size};
  a.Wbuf = reinterpret_cast<cce::u16*>(base + L.wbuf);
  a.G2 = L.g2q ? reinterpret_cast<cce::u16*>(base + L.g2q) : nullptr;
  a.Wbuf2 = L.wbuf2 ? reinterpret_cast<cce::u16*>(base + L.wbuf2) : nullptr;
  return cce::launch_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? CCE_OK
                                                                                : CCE_ELAUNCH;
}

}  // extern "C"
