/*
 * flashcce.h — C-ABI of the flash-CCE ORPO head for MI355X (gfx950).
 *
 * The head computes, for hidden rows h[M,D] and a vocabulary head W[V,D]
 * (both bf16, row-major, D contiguous) and targets y[M]:
 *
 *   logp_i = h_i . W_{y_i} - logsumexp_v (h_i . W_v)
 *
 * without ever storing the [M,V] logits ("Training — design (ORPO, flash-CCE
 * head, prefix sharing, segmented backward)", §5.1 "The head"; "ORPO training
 * — design", "Ranked levers", lever 1 and its "Implementation spec — fused
 * linear-CE log-prob head": online max / sum-exp over vocab tiles, O(M) saved
 * state), the ORPO objective on those log-probs (same pages, "The objective")
 * and the head backward (dh, dW) from the saved per-row log-sum-exp.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Array arguments are DEVICE pointers unless stated otherwise; scalars are
 *    passed by value.  `stream` is a hipStream_t (NULL = the null stream).
 *  - Every call only validates its arguments on the host and enqueues kernels
 *    on `stream`; it returns before the GPU work completes.  Inputs must stay
 *    alive and unmodified until that work has completed.  Nothing is
 *    allocated: the caller owns every buffer, including the workspace.
 *  - Host-detectable errors (NULL pointer, non-positive size, workspace too
 *    small, bad enum, a current device that is not gfx950) return a status
 *    immediately and enqueue nothing.  No exception crosses the ABI.
 *  - Data errors found on the device are OR-ed into the caller's uint32
 *    `dev_status` word as CCE_DERR_* bits; the library never clears it (the
 *    caller zeroes it before the first call and reads it after a sync).
 *  - Any M, V, D >= 1 is accepted; ragged tiles are masked inside the kernels.
 *  - Results are deterministic: no floating-point atomics are used, so for
 *    fixed inputs, shapes and eps the output bytes are identical run to run.
 *  - Segment codes: seg_i = (pair << 2) | kind, kind one of CCE_KIND_*.
 *    A row with y_i = -1 is ignored (logp 0, coef 0); such a row must have
 *    kind CCE_KIND_IGNORE.
 */
#ifndef FLASHCCE_H
#define FLASHCCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cce_status {
  CCE_OK = 0,
  CCE_EINVAL = 1,      /* NULL pointer, bad enum or non-finite scalar */
  CCE_ESHAPE = 2,      /* M, V or D < 1, n_pairs < 1, or sizes too large */
  CCE_EWORKSPACE = 3,  /* ws_bytes < cce_workspace_bytes(M, V, D) or ws misaligned */
  CCE_EDEVICE = 4,     /* the current HIP device is not gfx950 */
  CCE_ELAUNCH = 5      /* a kernel launch failed */
} cce_status;

enum { CCE_KIND_IGNORE = 0, CCE_KIND_PROMPT = 1, CCE_KIND_CHOSEN = 2, CCE_KIND_REJECTED = 3 };
enum { CCE_SCOPE_FULL = 0, CCE_SCOPE_RESPONSE = 1 };

/* Bits of the device status word. */
enum {
  CCE_DERR_TARGET = 1u,     /* y_i outside [-1, V), or y_i = -1 on a row that is not IGNORE */
  CCE_DERR_PAIR = 2u,       /* a pair index >= n_pairs */
  CCE_DERR_EMPTY_SPAN = 4u, /* a pair with no CHOSEN or no REJECTED row */
  CCE_DERR_NONFINITE = 8u   /* a non-finite log-sum-exp or loss */
};

/* Version of this ABI (incremented on incompatible changes). */
int cce_abi_version(void);

/* Human-readable name of a status code (static string; never NULL). */
const char* cce_status_string(int status);

/*
 * Workspace bytes needed by cce_forward, orpo_epilogue and cce_backward for
 * these sizes (one workspace serves all three).  Host-only; no GPU call.
 * It depends on M and D and is independent of V once V exceeds one backward
 * vocab chunk (16384 entries): the backward walks the vocabulary in chunks of
 * at most that width, through a bf16 gradient buffer of Mpad x 16384 (two
 * when D % 32 == 0: the backward then pipelines one chunk's contractions with
 * the next chunk's recompute).  Returns 0 for invalid sizes.
 */
size_t cce_workspace_bytes(int64_t M, int64_t V, int64_t D);

/*
 * Forward: per-row target log-prob and log-sum-exp.
 *   "Training — design …" §5.1; "ORPO training — design", lever 1 spec.
 *   h        [M, D] bf16 row-major (16-byte aligned rows are the fast path)
 *   W        [V, D] bf16 row-major
 *   y        [M] int32 target ids in [0, V), or -1 for an ignored row
 *   softcap  0 (off) or the final-logit cap c > 0: every logit becomes
 *            z = c tanh(h_i . W_v / c) before the log-sum-exp and the target
 *            gather ("Training — design …" §5.1, the e4b head with c = 30;
 *            "ORPO training — design", lever 1 spec).  Finite and >= 0, else
 *            CCE_EINVAL.
 *   logp     [M] fp32 out: z_{i,y_i} - lse_i, and 0 for rows with y_i = -1
 *   lse      [M] fp32 out: logsumexp_v z_{i,v} (written for every row)
 *   block_max  NULL, or [ceil(V / 256), M] fp32 out: the largest (capped)
 *            logit of row i over vocab block b = [256 b, 256 b + 256), at
 *            block_max[b * M + i] ("Training — design …" §5.1: the blockMax
 *            the forward saves for the backward's block skip).  Costs one
 *            barrier per tile and 4 bytes per row per vocab block.
 *   dev_status  uint32 (device) OR-ed with CCE_DERR_TARGET / _NONFINITE
 *   ws, ws_bytes  device workspace of at least cce_workspace_bytes(M, V, D)
 *                 bytes, 256-byte aligned; contents on entry are ignored.
 */
cce_status cce_forward(const void* h, const void* W, const int32_t* y,
                       int64_t M, int64_t V, int64_t D, float softcap,
                       float* logp, float* lse, float* block_max, uint32_t* dev_status,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * ORPO epilogue on the per-row log-probs.
 *   "Training — design …" §1 "The objective"; "ORPO training — design",
 *   "The objective" and "File-by-file changes" (loss.ts):
 *     per pair b: lw = mean logp over CHOSEN rows, lr = mean over REJECTED,
 *                 pm = mean over PROMPT rows (the P-1 prompt next-token rows);
 *     log_odds_b = (lw - lr) - (log1mexp(lw) - log1mexp(lr)),
 *       log1mexp(x) = log(1 - e^x), two-branch, clamped below at log(1e-7);
 *     or_b  = softplus(-log_odds_b)  (= -log sigmoid(log_odds_b));
 *     nll_b = -lw (RESPONSE scope) or -((P-1) pm + Mw lw) / ((P-1) + Mw) (FULL);
 *     loss = mean_b nll_b + lambda * mean_b or_b.
 *   logp     [M] fp32 (from cce_forward);  y [M] int32 (checked only);
 *   seg      [M] int32 segment codes; n_pairs >= 1; scope CCE_SCOPE_*.
 *   out5     [5] fp32 out: loss, nll, or, margin (= mean log_odds), accuracy
 *            (= fraction of pairs with lw > lr).
 *   pair_stats [n_pairs, 8] fp32 out (may be NULL): lw, lr, log_odds, nll_b,
 *            or_b, and the span sizes Mw, Mr, P-1 (integers, exact in fp32).
 *   coef     [M] fp32 out: -dloss/dlogp_i (positive on CHOSEN rows, negative on
 *            REJECTED rows, 1/(B((P-1)+Mw)) on PROMPT rows in FULL scope, else 0).
 *   dev_status OR-ed with CCE_DERR_PAIR / _EMPTY_SPAN / _TARGET / _NONFINITE.
 *   Sums are accumulated in fp64 in a fixed order.
 */
cce_status orpo_epilogue(const float* logp, const int32_t* y, const int32_t* seg,
                         int64_t M, int32_t n_pairs, float lambda, int scope,
                         float* out5, float* pair_stats, float* coef,
                         uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/* Preference objectives of pref_epilogue. */
enum { CCE_OBJ_ORPO = 0, CCE_OBJ_SIGMOID = 1, CCE_OBJ_IPO = 2, CCE_OBJ_HINGE = 3 };

/*
 * Preference-objective epilogue: the ORPO epilogue's family on the same
 * per-pair means lw, lr, pm and NLL_b ("Training — design …" §8.3 "Objective
 * variants and data"; "ORPO from-base on UltraFeedback (mixed-5bpw) — results
 * + research directions" §6.1 SimPO, §6.2 the gamma-hybrid, §6.3):
 *   s_b = log_odds_b (CCE_OBJ_ORPO)  or  beta (lw - lr) - gamma (the others);
 *   P_b = softplus(-s_b) = -log sigmoid(s_b)   (CCE_OBJ_ORPO, CCE_OBJ_SIGMOID)
 *       = s_b^2                                (CCE_OBJ_IPO; beta = 1 and
 *                                               gamma = 1/(2 tau) give IPO)
 *       = max(0, -s_b)                         (CCE_OBJ_HINGE; derivative 0 at
 *                                               the kink);
 *   loss = mean_b (nll_weight NLL_b + lambda P_b).
 * SimPO is CCE_OBJ_SIGMOID with nll_weight 0 and lambda 1; the gamma-hybrid is
 * CCE_OBJ_SIGMOID with nll_weight 1; orpo_epilogue is CCE_OBJ_ORPO with
 * nll_weight 1 (beta, gamma unused).
 *   Arguments as for orpo_epilogue, plus objective (CCE_OBJ_*), nll_weight,
 *   beta, gamma (finite, else CCE_EINVAL).
 *   out5 [5]: loss, nll (mean NLL_b), pref (mean P_b), margin (mean s_b),
 *             accuracy (fraction of pairs with lw > lr).
 *   pair_stats [n_pairs, 8] (may be NULL): lw, lr, s_b, NLL_b, P_b, Mw, Mr, P-1.
 *   coef [M]: -dloss/dlogp_i, as for orpo_epilogue.
 */
cce_status pref_epilogue(const float* logp, const int32_t* y, const int32_t* seg,
                         int64_t M, int32_t n_pairs, int objective, float nll_weight,
                         float lambda, float beta, float gamma, int scope,
                         float* out5, float* pair_stats, float* coef,
                         uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the head given the per-row coefficient coef_i = -dL/dlogp_i:
 *   G_{i,v} = coef_i (softmax_{i,v} - [v = y_i]) s_{i,v},  dh = G W,  dW = G^T h,
 *   with s = 1 - tanh^2(h_i . W_v / c) under a softcap c, else 1.
 *   "Training — design …" §5.1 (analytic backward from the saved LSE;
 *   backward skips; the sech^2 factor of the capped head); "ORPO training —
 *   design", lever 1 spec (backward).
 *   h, W, y, softcap  as for cce_forward (the same softcap as the forward that
 *            produced lse);  lse [M], coef [M] fp32.
 *   filter_eps  >= 0; softmax entries below it are dropped (never the target's).
 *   block_eps   >= 0; a 256x256 (row, vocab) tile whose largest softmax entry
 *               is below it and that holds no row's target is skipped.
 *               0 and 0 give the exact gradient.
 *   block_max   NULL, or the forward's block_max (same h, W, softcap): with
 *               block_eps > 0 the skip test is taken from it before the tile's
 *               logits are recomputed, so a skipped tile costs no contraction
 *               at all (without it the test needs the recomputed tile; the
 *               decision is the same up to fp32 rounding).  Ignored when
 *               block_eps = 0.
 *   dh [M, D] fp32 out (overwritten); dW [V, D] fp32 out (overwritten).
 *   G is rounded to bf16 (round-to-nearest-even) before the two contractions;
 *   accumulation is fp32.
 */
cce_status cce_backward(const void* h, const void* W, const int32_t* y,
                        const float* lse, const float* coef, const float* block_max,
                        int64_t M, int64_t V, int64_t D, float softcap,
                        float filter_eps, float block_eps,
                        float* dh, float* dW, uint32_t* dev_status,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Affine-quantised head (frozen): the forward and dh of the head when W is held
 * as 4- or 8-bit codes with a bf16 scale and bias per row and group of
 * group_size columns ("Training — design …" §5.1, the classifier is the
 * quantised head, dequantised inside the kernel, frozen so only dh flows back;
 * §5.6 "Quantized base", a vocab chunk is a row slice of the codes, scales and
 * biases).  Element (v, d) of the head is
 *     W[v, d] = s[v, d / group_size] * q[v, d] + b[v, d / group_size],
 * q[v, d] the bits-bit code at bit offset bits * (d % (32 / bits)) of word
 * d / (32 / bits) of row v (little-endian packing in uint32).
 *   Wq      [V, D * bits / 32] uint32;  scales, biases [V, D / group_size] bf16.
 *   bits    4 or 8;  group_size 32, 64 or 128 dividing D; else CCE_EINVAL.
 * The library computes s * q + b in fp32 and rounds it to bf16 (nearest-even)
 * one vocab chunk (16384 rows) at a time into the workspace; the chunk then
 * takes the bf16 path of cce_forward / cce_backward, so every other argument,
 * output and error behaves as there.  The results are those of cce_forward /
 * cce_backward on the bf16-rounded dequantised head.
 */

/* Workspace bytes for cce_forward_q / cce_backward_q: the parts of
 * cce_workspace_bytes the two calls share (forward partials, epilogue state,
 * exact onehot buffers, the first gradient buffer and its flags), then two
 * [M] fp32 rows, two bf16 chunks of the dequantised head (16384 x D each) with
 * a second gradient buffer between them when D % 32 == 0 (the pipelined
 * backward alternates between the two of each), and the dh split partials;
 * independent of V above one chunk.  0 for invalid sizes.  Host-only. */
size_t cce_workspace_bytes_q(int64_t M, int64_t V, int64_t D);

/* Forward over the quantised head; outputs as for cce_forward.  The head is
 * dequantised chunk by chunk into the chunk and gradient buffers of the
 * workspace (the backward's, free during the forward): as few equal chunks of
 * whole 256-row tiles as that space holds.  The running (max, sum-exp) of each
 * row is folded chunk by chunk in a fixed order. */
cce_status cce_forward_q(const void* h, const uint32_t* Wq, const void* scales,
                         const void* biases, int bits, int group_size,
                         const int32_t* y, int64_t M, int64_t V, int64_t D, float softcap,
                         float* logp, float* lse, float* block_max, uint32_t* dev_status,
                         void* ws, size_t ws_bytes, void* stream);

/* Backward over the quantised head: dh [M, D] fp32 out (overwritten), as for
 * cce_backward; no dW (the head is frozen). */
cce_status cce_backward_q(const void* h, const uint32_t* Wq, const void* scales,
                          const void* biases, int bits, int group_size,
                          const int32_t* y, const float* lse, const float* coef,
                          const float* block_max, int64_t M, int64_t V, int64_t D, float softcap,
                          float filter_eps, float block_eps, float* dh,
                          uint32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/*
 * cce_forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that forbid
 * allocation).  The forward's scratch (the per-split partial max / sum-exp of
 * each row and the target logits) lives in a fixed 16 MiB array of the
 * library's own device memory, one per device the library runs on, held until
 * the process ends; nothing is allocated by the call.  Arguments, outputs and
 * results are those of cce_forward (the same kernels; bytes identical to it).
 *   M        at most 786432 rows, else CCE_ESHAPE (the scratch would not fit).
 * Every call on one device shares that device's array: calls that overlap on
 * one GPU (on different streams, or from several threads) race and must not
 * be issued; calls ordered on one stream are fine.  No scratch contents carry
 * from one call to the next (each call writes before it reads).
 */
cce_status cce_forward_noalloc(const void* h, const void* W, const int32_t* y,
                               int64_t M, int64_t V, int64_t D, float softcap,
                               float* logp, float* lse, float* block_max, uint32_t* dev_status,
                               void* stream);

/*
 * Per-launch timing (a profiling hook; no result depends on it).  Between
 * cce_timing_begin and cce_timing_end, every kernel that a call of this
 * library enqueues from the calling thread is bracketed by two of the caller's
 * events, recorded on that call's stream: events[2 i] before launch i and
 * events[2 i + 1] after it, with kinds[i] = the kernel (cce_kernel_name gives
 * its name) and flops[i] = the launch's algorithmic floating-point operations
 * (2 per multiply-add of the contractions it performs, counted at their
 * nominal sizes: M rows, the vocabulary entries the launch covers, D; 0 for a
 * kernel without a contraction), for the first `capacity` launches of the
 * window (later launches are not bracketed).  The time of launch i is the
 * elapsed time between its two events once the stream has completed them.
 *   events    2 * capacity hipEvent_t handles (host array of device events,
 *             created by the caller with timing enabled; none may be NULL)
 *   kinds     capacity int32 (host array)
 *   flops     capacity doubles (host array), or NULL
 *   capacity  >= 1, else CCE_EINVAL.  The window belongs to the calling
 *             thread; a new begin replaces an open window.
 * cce_timing_end closes the window and returns the number of launches
 * bracketed, or -1 if no window was open or an event could not be recorded.
 * Recording events between launches adds a few microseconds per launch.
 */
cce_status cce_timing_begin(void* const* events, int32_t* kinds, double* flops,
                            int32_t capacity);
int32_t cce_timing_end(void);

/* Name of a kernel kind reported by the timing hook (static string). */
const char* cce_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif

#endif /* FLASHCCE_H */
