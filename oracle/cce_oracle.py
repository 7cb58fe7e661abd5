"""fp64 CPU oracle for the flash-CCE ORPO head.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark do.  It shares no code with the HIP library (no kernels,
headers, helpers, constants or pre/post-processing); it receives plain arrays.

What it computes is the plain definition, with every logit materialised (in
row chunks of at most ~1 GB of fp64), so that a reader can check it against the
pages by eye.  Citations name the page and the section:

  [P1]  "Training — design (ORPO, flash-CCE head, prefix sharing, segmented
        backward)" (mlx-bun 1.0.0 docs, orpo-training.md)
  [P2]  "ORPO training — design" (mlx-bun 0.0.6 docs, orpo-training.md)
  [P3]  "flash-CCE host-buffer pin leak — post-mortem + L3 verification
        approach" (mlx-bun 0.0.6 investigations)

Readings taken where the pages leave a step open (each one is listed with its
reason in the design notes of the repository):
  * pm is the mean log-prob over the prompt's P-1 next-token rows;
  * log1mexp uses the two-branch form with a clamp at eps = 1e-7 (the pages
    say "clip ... small eps" and "clamp / two-branch" without a value);
  * coef = -dL/dlogp (so chosen rows are positive), and the per-logit
    gradient is coef * (softmax - onehot);
  * with several pairs the NLL and OR terms are formed per pair and then
    averaged over pairs; accuracy uses a strict lw > lr; margin is the mean
    log-odds;
  * the gradient filter compares the softmax value itself with eps and never
    drops the target entry;
  * a row with target -1 is ignored: its log-prob is 0 and its coefficient 0;
  * the final-logit softcap is cap * tanh(z / cap) evaluated exactly (the pages'
    head divides by a bf16-rounded cap inside its framework's op; here the cap
    is a plain float argument), applied before both the log-sum-exp and the
    target gather, with sech^2(z / cap) in the backward; cap = 0 means off;
  * the preference objectives other than ORPO use s = beta (lw - lr) - gamma
    (SimPO's margin gamma is not scaled by beta, as in the research-directions
    page; the design page's softplus(-beta((lw - lr) - gamma)) is the same
    family with gamma replaced by beta * gamma); IPO is the reference-free
    (s)^2 on the length-normalised means; the hinge's derivative at its kink is
    taken as 0; every member may add the NLL term with a weight (0 for pure
    SimPO, 1 for ORPO and the gamma-hybrid);
  * the quantised head's value is s * q + b exactly, and its contractions take
    that value rounded to bf16 (the pages dequantise into fp32 on their GPU;
    bf16 is the operand type of the matrix cores used here), so the quantised
    forward and backward are the bf16 head's on round_bf16(dequantize(...)).

Every function here has a pin in the test-suite (closed forms, library special
cases, finite differences, brute force, invariants); none is "parity unpinned".
The filtered-gradient mode is pinned by brute force on a tiny case (scalar
loops, an entry exactly at eps, a target far below it); how far it moves the
gradient from the exact one is reported, not gated.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

KIND_IGNORE, KIND_PROMPT, KIND_CHOSEN, KIND_REJECTED = 0, 1, 2, 3
SCOPE_FULL, SCOPE_RESPONSE = 0, 1
LOG1MEXP_EPS = 1e-7
_CHUNK_BYTES = 1 << 30


def _row_chunk(V: int) -> int:
    return max(1, _CHUNK_BYTES // (8 * max(1, V)))


# ----------------------------------------------------------------------------
# Forward: per-row target log-prob and log-sum-exp.
# [P1] §5.1 and [P2] "Ranked levers", lever 1: logp_t = h_t.W_{y_t} -
# logsumexp_v(h_t.W_v); the full logits are the plain definition.
# ----------------------------------------------------------------------------
def logits(H: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = H W^T in fp64 (all of it)."""
    return np.asarray(H, np.float64) @ np.asarray(W, np.float64).T


def capped(Z: np.ndarray, softcap: float) -> np.ndarray:
    """Final-logit softcap ([P1] §5.1, the e4b head with cap 30; [P2] lever 1
    "Implementation spec"): cap * tanh(z / cap); softcap = 0 leaves Z as is."""
    if softcap == 0.0:
        return Z
    return softcap * np.tanh(Z / softcap)


def dcapped(Z: np.ndarray, softcap: float) -> np.ndarray:
    """d capped / d z = sech^2(z / cap) = 1 - tanh^2(z / cap) (1 when off)."""
    if softcap == 0.0:
        return np.ones_like(Z)
    t = np.tanh(Z / softcap)
    return 1.0 - t * t


def dequantize(Wq: np.ndarray, scale: np.ndarray, bias: np.ndarray, bits: int,
               group_size: int) -> np.ndarray:
    """The affine-quantised head's values ([P1] §5.1 "in-Metal 4/8-bit affine
    dequant", §5.6 "Quantized base"): W[v, d] = s[v, g] * q[v, d] + b[v, g] with
    g = d // group_size, q the bits-wide code of column d, stored little-endian
    in uint32 words along the row (code j of a word in bits bits*j ..).
    scale and bias are the per-group values (any float dtype); fp64 result."""
    Wq = np.asarray(Wq, np.uint64)
    V = Wq.shape[0]
    per = 32 // bits
    D = Wq.shape[1] * per
    q = np.empty((V, D), np.float64)
    mask = np.uint64((1 << bits) - 1)
    for j in range(per):
        q[:, j::per] = ((Wq >> np.uint64(bits * j)) & mask).astype(np.float64)
    g = np.arange(D) // group_size
    return np.asarray(scale, np.float64)[:, g] * q + np.asarray(bias, np.float64)[:, g]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Each value rounded to the nearest bfloat16 number (8 significant bits,
    ties to the even significand), returned as fp64.  The operand precision of
    the quantised head's contractions: its dequantised values are taken in
    bf16, like the bf16 head's.  Normal range only (no subnormal or overflow
    handling: head values are far from both ends)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)               # x = m * 2^e with 0.5 <= |m| < 1 (m = 0 for x = 0)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # np.round: half to even


def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    """log sum_v exp(Z[i, v]) with the row max factored out."""
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def forward(H: np.ndarray, W: np.ndarray, y: np.ndarray, softcap: float = 0.0):
    """Returns (logp[M], lse[M]) in fp64.  Rows with y = -1 get logp = 0 (their
    lse is still computed).  With softcap > 0 every logit is capped first
    (both the log-sum-exp and the target logit see the capped value)."""
    H = np.asarray(H, np.float64)
    W = np.asarray(W, np.float64)
    y = np.asarray(y, np.int64)
    M, V = H.shape[0], W.shape[0]
    lse = np.empty(M)
    logp = np.zeros(M)
    step = _row_chunk(V)
    for i0 in range(0, M, step):
        i1 = min(M, i0 + step)
        Z = capped(logits(H[i0:i1], W), softcap)
        lse[i0:i1] = logsumexp_rows(Z)
        yy = y[i0:i1]
        ok = yy >= 0
        rows = np.nonzero(ok)[0]
        logp[i0 + rows] = Z[rows, yy[rows]] - lse[i0 + rows]
    return logp, lse


def forward_rows(H: np.ndarray, W: np.ndarray, y: np.ndarray, rows: np.ndarray,
                 softcap: float = 0.0):
    """The forward for a subset of rows only (used for sampled checks at large
    sizes)."""
    rows = np.asarray(rows, np.int64)
    lp, ls = forward(np.asarray(H)[rows], W, np.asarray(y)[rows], softcap)
    return lp, ls


# ----------------------------------------------------------------------------
# log1mexp.  [P1] §1 ("stable log(clip(1 - exp(x), eps, 1))") and [P2] "File-by-
# file changes" (no expm1/log1p there) and "Recommended defaults" ("clamp /
# two-branch").  We use both: the two-branch evaluation avoids the cancellation
# of 1 - exp(x) near 0, and the clamp at eps keeps it finite at x -> 0-.
# ----------------------------------------------------------------------------
def log1mexp(x: float, eps: float = LOG1MEXP_EPS) -> float:
    """log(1 - e^x) for x <= 0, clamped below at log(eps)."""
    x = float(x)
    if x > -math.log(2.0):
        return math.log(max(-math.expm1(x), eps))
    return math.log1p(-math.exp(x))


def dlog1mexp(x: float, eps: float = LOG1MEXP_EPS) -> float:
    """d/dx log1mexp(x): -e^x / (1 - e^x), and 0 where the clamp binds."""
    x = float(x)
    if -math.expm1(x) < eps:
        return 0.0
    return -math.exp(x) / (-math.expm1(x))


def softplus(x: float) -> float:
    """log(1 + e^x), evaluated without overflow."""
    x = float(x)
    if x > 0:
        return x + math.log1p(math.exp(-x))
    return math.log1p(math.exp(x))


def sigmoid(x: float) -> float:
    x = float(x)
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


# ----------------------------------------------------------------------------
# ORPO scalars for one pair.  [P1] §1 and [P2] "The objective":
#   L = L_NLL(y_w) + lambda * L_OR,  L_OR = -log sigma(log_odds),
#   log_odds = (lw - lr) - (log1mexp(lw) - log1mexp(lr)).
# ----------------------------------------------------------------------------
def log_odds(lw: float, lr: float) -> float:
    return (lw - lr) - (log1mexp(lw) - log1mexp(lr))


def or_term(lw: float, lr: float) -> float:
    """-log sigma(log_odds) = softplus(-log_odds)."""
    return softplus(-log_odds(lw, lr))


def full_nll(pm: float, Pm1: int, lw: float, Mw: int) -> float:
    """[P1] §1, scope `full`: -((P-1) pm + M lw) / ((P-1) + M); with P-1 = 0
    this is -lw."""
    return -((Pm1 * pm if Pm1 > 0 else 0.0) + Mw * lw) / (Pm1 + Mw)


def orpo_pair_loss(lw: float, lr: float, lam: float, nll: Optional[float] = None) -> float:
    """Loss of one pair from its length-normalised means; nll defaults to the
    response-scope -lw ([P2] "The objective")."""
    if nll is None:
        nll = -lw
    return nll + lam * or_term(lw, lr)


def orpo_pair_grad(lw: float, lr: float, lam: float):
    """(dL/dlw, dL/dlr) for response scope, by the chain rule through
    log_odds; d log_odds/d lw = 1 - dlog1mexp(lw) = 1/(1 - e^lw)."""
    lo = log_odds(lw, lr)
    s = sigmoid(lo)
    dlo_dlw = 1.0 - dlog1mexp(lw)
    dlo_dlr = -1.0 + dlog1mexp(lr)
    # d softplus(-lo)/d lo = -(1 - sigma(lo))
    return -1.0 - lam * (1.0 - s) * dlo_dlw, -lam * (1.0 - s) * dlo_dlr


# ----------------------------------------------------------------------------
# Epilogue over a batch of pairs.  [P1] §1 (mean, not sum; scope full vs
# response; the chosen forward does double duty; no rejected NLL) and [P2]
# "File-by-file changes" (nll = mean(-lw), or = mean(softplus(-logOdds)),
# loss = nll + lambda*or; metrics loss/nll/or/accuracy/margin).
# ----------------------------------------------------------------------------
def pair_row_sets(seg: np.ndarray, n_pairs: int):
    """For each pair b: the ascending row indices of its CHOSEN, REJECTED and
    PROMPT rows (the sets {i: pair_i = b, kind_i = K}).  Rows are grouped once
    with a stable sort, so each pair costs only its own rows."""
    seg = np.asarray(seg, np.int64)
    kind = seg & 3
    pair = seg >> 2
    order = np.argsort(pair, kind="stable")
    bounds = np.searchsorted(pair[order], np.arange(int(n_pairs) + 1))
    out = []
    for b in range(int(n_pairs)):
        idx = order[bounds[b]:bounds[b + 1]]
        out.append(tuple(idx[kind[idx] == k] for k in (KIND_CHOSEN, KIND_REJECTED, KIND_PROMPT)))
    return out


def epilogue(logp: np.ndarray, seg: np.ndarray, n_pairs: int, lam: float, scope: int) -> Dict:
    logp = np.asarray(logp, np.float64)
    seg = np.asarray(seg, np.int64)
    B = int(n_pairs)
    sets = pair_row_sets(seg, B)
    Mw = np.zeros(B, np.int64)
    Mr = np.zeros(B, np.int64)
    Pm1 = np.zeros(B, np.int64)
    lw = np.zeros(B)
    lr = np.zeros(B)
    pm = np.zeros(B)
    lo = np.zeros(B)
    orb = np.zeros(B)
    nllb = np.zeros(B)
    sig = np.zeros(B)
    dlo_w = np.zeros(B)
    dlo_r = np.zeros(B)
    for b in range(B):
        C, R, Q = sets[b]
        Mw[b], Mr[b], Pm1[b] = len(C), len(R), len(Q)
        if Mw[b] == 0 or Mr[b] == 0:
            raise ValueError(f"pair {b} has an empty response span")
        lw[b] = logp[C].sum() / Mw[b]
        lr[b] = logp[R].sum() / Mr[b]
        pm[b] = logp[Q].sum() / Pm1[b] if Pm1[b] > 0 else 0.0
        lo[b] = log_odds(lw[b], lr[b])
        orb[b] = softplus(-lo[b])
        sig[b] = sigmoid(lo[b])
        nllb[b] = full_nll(pm[b], int(Pm1[b]), lw[b], int(Mw[b])) if scope == SCOPE_FULL else -lw[b]
        dlo_w[b] = 1.0 - dlog1mexp(lw[b])
        dlo_r[b] = -1.0 + dlog1mexp(lr[b])
    nll = nllb.mean()
    orv = orb.mean()
    loss = nll + lam * orv
    margin = lo.mean()
    accuracy = float(np.mean(lw > lr))

    # coef_i = -dloss/dlogp_i
    coef = np.zeros(logp.shape[0])
    for b in range(B):
        C, R, Q = sets[b]
        w_or = lam * (1.0 - sig[b])          # = -dloss_b/dlo (before 1/B)
        if scope == SCOPE_FULL:
            w_nll = 1.0 / (Pm1[b] + Mw[b])
            coef[Q] = w_nll / B
        else:
            w_nll = 1.0 / Mw[b]
        coef[C] = (w_nll + w_or * dlo_w[b] / Mw[b]) / B
        coef[R] = (w_or * dlo_r[b] / Mr[b]) / B
    return dict(loss=loss, nll=nll, orv=orv, margin=margin, accuracy=accuracy,
                lw=lw, lr=lr, pm=pm, log_odds=lo, nll_b=nllb, or_b=orb,
                Mw=Mw, Mr=Mr, Pm1=Pm1, coef=coef)


def loss_from_logp(logp: np.ndarray, seg: np.ndarray, n_pairs: int, lam: float, scope: int) -> float:
    return epilogue(logp, seg, n_pairs, lam, scope)["loss"]


# ----------------------------------------------------------------------------
# Preference-objective family on the same per-pair means.  [P1] §8.3 "Objective
# variants and data" (SimPO softplus(-beta((lw - lr) - gamma)), IPO, hinge /
# SLiC margin) and "ORPO from-base on UltraFeedback (mixed-5bpw) — results +
# research directions" §6.1 (SimPO: -log sigma(beta (lw - ll) - gamma), no SFT
# term), §6.2 (the gamma-hybrid: NLL(chosen) + lambda [-log sigma(beta (lw -
# ll) - gamma)]), §6.3 (SFT + SimPO in one stage).  Per pair b:
#   s_b = log_odds_b                      (ORPO)
#       = beta (lw_b - lr_b) - gamma      (SIGMOID, IPO, HINGE)
#   P_b = softplus(-s_b)  (ORPO, SIGMOID)  = -log sigma(s_b)
#       = s_b^2           (IPO: reference-free, length-normalised; beta = 1 and
#                          gamma = 1/(2 tau) give IPO's (h - 1/(2 tau))^2)
#       = max(0, -s_b)    (HINGE: max(0, gamma - beta (lw - lr)); derivative 0
#                          at the kink)
#   L = mean_b (w_nll NLL_b + lambda P_b),  NLL_b as in the ORPO epilogue.
# ORPO with w_nll = 1 is exactly `epilogue` above.
# ----------------------------------------------------------------------------
OBJ_ORPO, OBJ_SIGMOID, OBJ_IPO, OBJ_HINGE = 0, 1, 2, 3


def pref_term(objective: int, s: float) -> float:
    if objective in (OBJ_ORPO, OBJ_SIGMOID):
        return softplus(-s)
    if objective == OBJ_IPO:
        return s * s
    if objective == OBJ_HINGE:
        return max(0.0, -s)
    raise ValueError(objective)


def dpref_term(objective: int, s: float) -> float:
    """dP/ds."""
    if objective in (OBJ_ORPO, OBJ_SIGMOID):
        return -(1.0 - sigmoid(s))
    if objective == OBJ_IPO:
        return 2.0 * s
    if objective == OBJ_HINGE:
        return -1.0 if s < 0.0 else 0.0
    raise ValueError(objective)


def pref_epilogue(logp: np.ndarray, seg: np.ndarray, n_pairs: int, objective: int,
                  nll_weight: float, lam: float, beta: float, gamma: float, scope: int) -> Dict:
    logp = np.asarray(logp, np.float64)
    seg = np.asarray(seg, np.int64)
    B = int(n_pairs)
    sets = pair_row_sets(seg, B)
    out = {k: np.zeros(B) for k in ("lw", "lr", "pm", "s", "pref_b", "nll_b")}
    Mw = np.zeros(B, np.int64)
    Mr = np.zeros(B, np.int64)
    Pm1 = np.zeros(B, np.int64)
    coef = np.zeros(logp.shape[0])
    for b in range(B):
        C, R, Q = sets[b]
        Mw[b], Mr[b], Pm1[b] = len(C), len(R), len(Q)
        if Mw[b] == 0 or Mr[b] == 0:
            raise ValueError(f"pair {b} has an empty response span")
        lw = logp[C].sum() / Mw[b]
        lr = logp[R].sum() / Mr[b]
        pm = logp[Q].sum() / Pm1[b] if Pm1[b] > 0 else 0.0
        if objective == OBJ_ORPO:
            s = log_odds(lw, lr)
            ds_w, ds_r = 1.0 - dlog1mexp(lw), -1.0 + dlog1mexp(lr)
        else:
            s = beta * (lw - lr) - gamma
            ds_w, ds_r = beta, -beta
        nll_b = full_nll(pm, int(Pm1[b]), lw, int(Mw[b])) if scope == SCOPE_FULL else -lw
        for k, v in (("lw", lw), ("lr", lr), ("pm", pm), ("s", s),
                     ("pref_b", pref_term(objective, s)), ("nll_b", nll_b)):
            out[k][b] = v
        # coef_i = -dL/dlogp_i
        dP = dpref_term(objective, s)
        if scope == SCOPE_FULL:
            w = nll_weight / (Pm1[b] + Mw[b])
            coef[Q] = w / B
        else:
            w = nll_weight / Mw[b]
        coef[C] = (w - lam * dP * ds_w / Mw[b]) / B
        coef[R] = (-lam * dP * ds_r / Mr[b]) / B
    nll = out["nll_b"].mean()
    pref = out["pref_b"].mean()
    return dict(loss=nll_weight * nll + lam * pref, nll=nll, pref=pref, margin=out["s"].mean(),
                accuracy=float(np.mean(out["lw"] > out["lr"])), Mw=Mw, Mr=Mr, Pm1=Pm1,
                coef=coef, **out)


# ----------------------------------------------------------------------------
# Backward.  [P1] §5.1 (analytic backward: g.(onehot - softmax), dh = grad.W)
# and [P2] "Implementation spec — fused linear-CE log-prob head" (softmax from
# the saved per-row LSE).  With coef = -g the per-logit gradient is
# G = coef (softmax - onehot); dh = G W and dW = G^T H.
# Filter mode ([P1] §5.1 skips; [P3] "The coeff filter"): softmax entries
# below eps are dropped, never the target's.
# Softcap ([P1] §5.1; [P2] lever 1 "Implementation spec"): the softmax is that
# of the capped logits, and the chain rule through the cap multiplies each
# entry by sech^2(z / cap).
# ----------------------------------------------------------------------------
def grad_logits(Z: np.ndarray, lse: np.ndarray, y: np.ndarray, coef: np.ndarray,
                filter_eps: float = 0.0, softcap: float = 0.0) -> np.ndarray:
    """G = coef * (softmax(capped Z) - onehot) * d capped / d z, from the raw
    logits Z."""
    P = np.exp(capped(Z, softcap) - lse[:, None])
    onehot = np.zeros_like(P)
    rows = np.nonzero(y >= 0)[0]
    onehot[rows, y[rows]] = 1.0
    if filter_eps > 0.0:
        P = np.where((P < filter_eps) & (onehot == 0.0), 0.0, P)
    return coef[:, None] * (P - onehot) * dcapped(Z, softcap)


# ----------------------------------------------------------------------------
# Block skip ([P1] §5.1 "Apple-CCE backward skips": the blockMax skip, whose
# per-(row, vocab block) maximum the forward saves next to the LSE).  The
# vocabulary and the rows are cut into blocks of `block` (256 here, from 0);
# block_max[b, i] is the largest (capped) logit of row i over vocab block b.
# A (row block, vocab block) pair is dead when every softmax entry in it,
# exp(block_max - lse) bounding them all, is below block_eps and none of its
# rows has its target in the vocab block; dead pairs contribute nothing.
# ----------------------------------------------------------------------------
def block_max(H: np.ndarray, W: np.ndarray, softcap: float = 0.0, block: int = 256) -> np.ndarray:
    """[ceil(V / block), M]: the largest capped logit of each row per vocab block."""
    H = np.asarray(H, np.float64)
    W = np.asarray(W, np.float64)
    M, V = H.shape[0], W.shape[0]
    nb = (V + block - 1) // block
    out = np.empty((nb, M), np.float64)
    step = _row_chunk(V)
    for i0 in range(0, M, step):
        i1 = min(M, i0 + step)
        Z = capped(logits(H[i0:i1], W), softcap)
        for b in range(nb):
            out[b, i0:i1] = Z[:, b * block:(b + 1) * block].max(axis=1)
    return out


def dead_blocks(bmax: np.ndarray, lse: np.ndarray, y: np.ndarray, block_eps: float,
                block: int = 256) -> np.ndarray:
    """[ceil(M / block), ceil(V / block)] bool: the pairs the block skip drops."""
    bmax = np.asarray(bmax, np.float64)
    lse = np.asarray(lse, np.float64)
    y = np.asarray(y, np.int64)
    nvb, M = bmax.shape
    nrb = (M + block - 1) // block
    dead = np.zeros((nrb, nvb), bool)
    if block_eps <= 0.0:
        return dead
    pmax = np.exp(bmax - lse[None, :])                    # [nvb, M]
    for a in range(nrb):
        rows = slice(a * block, min(M, (a + 1) * block))
        below = pmax[:, rows].max(axis=1) < block_eps
        has_tgt = np.zeros(nvb, bool)
        yt = y[rows]
        has_tgt[np.unique(yt[yt >= 0] // block)] = True
        dead[a] = below & ~has_tgt
    return dead


def backward(H: np.ndarray, W: np.ndarray, y: np.ndarray, lse: np.ndarray, coef: np.ndarray,
             filter_eps: float = 0.0, softcap: float = 0.0, block_eps: float = 0.0,
             block: int = 256):
    """Returns (dh[M,D], dW[V,D]) in fp64, given the forward's lse and the
    epilogue's coef; block_eps > 0 applies the block skip."""
    H = np.asarray(H, np.float64)
    W = np.asarray(W, np.float64)
    y = np.asarray(y, np.int64)
    lse = np.asarray(lse, np.float64)
    coef = np.asarray(coef, np.float64)
    M, V = H.shape[0], W.shape[0]
    dead = None
    if block_eps > 0.0:
        dead = dead_blocks(block_max(H, W, softcap, block), lse, y, block_eps, block)
    dh = np.zeros_like(H)
    dW = np.zeros_like(W)
    step = _row_chunk(V)
    for i0 in range(0, M, step):
        i1 = min(M, i0 + step)
        G = grad_logits(logits(H[i0:i1], W), lse[i0:i1], y[i0:i1], coef[i0:i1], filter_eps,
                        softcap)
        if dead is not None:
            G = np.where(dead[np.arange(i0, i1)[:, None] // block, np.arange(V)[None, :] // block],
                         0.0, G)
        dh[i0:i1] = G @ W
        dW += G.T @ H[i0:i1]
    return dh, dW


def backward_dh_rows(H, W, y, lse, coef, rows, filter_eps: float = 0.0, softcap: float = 0.0):
    """dh for a subset of rows (each row of dh depends only on its own row)."""
    rows = np.asarray(rows, np.int64)
    H = np.asarray(H, np.float64)
    W = np.asarray(W, np.float64)
    Z = logits(H[rows], W)
    G = grad_logits(Z, np.asarray(lse, np.float64)[rows], np.asarray(y, np.int64)[rows],
                    np.asarray(coef, np.float64)[rows], filter_eps, softcap)
    return G @ W


def backward_dW_rows(H, W, y, lse, coef, vrows, filter_eps: float = 0.0, softcap: float = 0.0):
    """dW for a subset of vocab rows: dW[v] = sum_i G[i, v] h_i, which needs the
    logits of every row against those vocab rows only (lse for all rows is
    an input)."""
    vrows = np.asarray(vrows, np.int64)
    H = np.asarray(H, np.float64)
    W = np.asarray(W, np.float64)
    y = np.asarray(y, np.int64)
    lse = np.asarray(lse, np.float64)
    coef = np.asarray(coef, np.float64)
    Z = H @ W[vrows].T                                   # [M, |vrows|]
    P = np.exp(capped(Z, softcap) - lse[:, None])
    onehot = (y[:, None] == vrows[None, :]).astype(np.float64)
    if filter_eps > 0.0:
        P = np.where((P < filter_eps) & (onehot == 0.0), 0.0, P)
    G = coef[:, None] * (P - onehot) * dcapped(Z, softcap)
    return G.T @ H


def step(H, W, y, seg, n_pairs, lam, scope, filter_eps: float = 0.0,
         softcap: float = 0.0) -> Dict:
    """One whole pass: forward, epilogue, backward."""
    logp, lse = forward(H, W, y, softcap)
    ep = epilogue(logp, seg, n_pairs, lam, scope)
    dh, dW = backward(H, W, y, lse, ep["coef"], filter_eps, softcap)
    ep.update(logp=logp, lse=lse, dh=dh, dW=dW)
    return ep
