"""Seeded synthetic inputs for the flash-CCE ORPO head.

This module only *draws* inputs; it holds none of the head's arithmetic (no
logits, no softmax, no loss).  Both the HIP path (through the binding) and the
fp64 CPU oracle read what it returns, so the two sides see the same bf16 bit
patterns.

Row layout.  Each row of ``h`` is one next-token position.  A row carries a
segment code ``seg = (pair << 2) | kind`` with kind one of IGNORE (0), PROMPT
(1), CHOSEN (2), REJECTED (3); IGNORE rows have target ``y = -1``.  Per pair the
rows are laid out as ``P-1`` prompt rows, then the chosen response rows, then
the rejected response rows (the row order does not change any result).

Value recipe (the pages measure on real model hiddens, which are not available
here; these draws stand in for them):
  * every tensor is drawn in fp32 from ``numpy.random.Generator(PCG64)`` seeded
    with ``SeedSequence(20261202 + k)`` and spawned per tensor;
  * hidden ~ N(0, 1) (times 4 for the long-context case, giving a peaked
    softmax), head weight ~ N(0, 0.02^2);
  * fp32 values are rounded to bf16 with round-to-nearest-even, once;
  * targets are Zipf(s=1.1) over the vocab, P(id=k) ~ (k+1)^-1.1 on [0, V),
    drawn by inverse CDF (rank = id), or uniform for the tiny case;
  * the "peaked" Gemma case adds a token-frequency prior to the logits, the
    way a trained head concentrates the softmax on frequent ids: hidden
    coordinate 0 is 1 on every row and head coordinate 0 of vocab row v is
    -1.1 * ln(1 + v) (the targets' own Zipf exponent), so a logit is the
    random part plus -1.1 ln(1 + v) and the rare-id vocab tiles carry almost
    no softmax mass (what the backward's block skip exploits on real data).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

KIND_IGNORE, KIND_PROMPT, KIND_CHOSEN, KIND_REJECTED = 0, 1, 2, 3
SCOPE_FULL, SCOPE_RESPONSE = 0, 1
BASE_SEED = 20261202


# ----------------------------------------------------------------------------
# bf16 bit patterns (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------
def zipf_ids(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """n ids in [0, V) with P(k) proportional to (k+1)^-s, by inverse CDF."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int32)


def uniform_ids(rng: np.random.Generator, n: int, V: int) -> np.ndarray:
    return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ----------------------------------------------------------------------------
# segment layouts
# ----------------------------------------------------------------------------
def layout_pairs(spans) -> np.ndarray:
    """spans: list of (n_prompt_rows, n_chosen, n_rejected[, n_ignore]) per pair.

    Returns seg[M] int32 with rows laid out pair by pair: prompt, chosen,
    rejected, then ignore (padding) rows.
    """
    out = []
    for b, sp in enumerate(spans):
        npm, nc, nr = sp[:3]
        ni = sp[3] if len(sp) > 3 else 0
        out += [(b << 2) | KIND_PROMPT] * npm
        out += [(b << 2) | KIND_CHOSEN] * nc
        out += [(b << 2) | KIND_REJECTED] * nr
        out += [(b << 2) | KIND_IGNORE] * ni
    return np.asarray(out, dtype=np.int32)


def _split_total(rng: np.random.Generator, total: int, parts: int, lo: int, hi: int) -> np.ndarray:
    """Integer lengths drawn U[lo, hi], rescaled to sum to `total`, clamped to [lo, hi]."""
    raw = rng.uniform(lo, hi, size=parts)
    x = np.clip(np.round(raw * total / raw.sum()), lo, hi).astype(np.int64)
    # fix the rounding/clamping residual one unit at a time, keeping [lo, hi]
    i = 0
    while x.sum() != total:
        j = i % parts
        if x.sum() < total and x[j] < hi:
            x[j] += 1
        elif x.sum() > total and x[j] > lo:
            x[j] -= 1
        i += 1
        if i > 100 * total:
            raise ValueError("cannot split total within bounds")
    return x


def _split_even(total: int, parts: int) -> np.ndarray:
    base = np.full(parts, total // parts, dtype=np.int64)
    base[: total - base.sum()] += 1
    return base


def stress_spans(rng: np.random.Generator, M: int = 16384, n_pairs: int = 8,
                 masked_frac: float = 0.30, lo: int = 64, hi: int = 4096):
    """Stress layout: ~30% masked rows (2/3 PROMPT, 1/3 IGNORE padding); the
    remaining response rows are split over 2*n_pairs responses with lengths
    drawn U[lo, hi], rescaled to the total and clamped."""
    n_masked = int(round(masked_frac * M))
    n_ign = n_masked // 3
    n_prompt = n_masked - n_ign
    n_resp = M - n_masked
    lens = _split_total(rng, n_resp, 2 * n_pairs, lo, hi)
    prm = _split_even(n_prompt, n_pairs)
    ign = _split_even(n_ign, n_pairs)
    return [(int(prm[b]), int(lens[2 * b]), int(lens[2 * b + 1]), int(ign[b])) for b in range(n_pairs)]


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    M: int
    D: int
    V: int
    h_bits: np.ndarray          # uint16 [M, D]  bf16 bit patterns
    W_bits: np.ndarray          # uint16 [V, D]
    y: np.ndarray               # int32 [M], -1 on IGNORE rows
    seg: np.ndarray             # int32 [M]
    n_pairs: int
    lam: float
    scope: int
    filter_eps: float = 0.0
    h_f32_raw: Optional[np.ndarray] = None   # the fp32 draws before rounding (tiny case)
    W_f32_raw: Optional[np.ndarray] = None

    def h64(self) -> np.ndarray:
        return bf16_bits_to_f32(self.h_bits).astype(np.float64)

    def W64(self) -> np.ndarray:
        return bf16_bits_to_f32(self.W_bits).astype(np.float64)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of one forward+backward step: 8*M*V*D."""
        return 8.0 * self.M * self.V * self.D


CONFIG_NAMES = ["tiny", "small_1b", "long_1b", "gemma4b_head", "stress", "gemma4b_peaked"]
PRIOR_EXPONENT = 1.1


def _draw(k: int, M: int, D: int, V: int, spans, hidden_scale: float, targets: str,
          keep_raw: bool, seed_k: Optional[int] = None, prior: bool = False):
    ss = np.random.SeedSequence(BASE_SEED + (k if seed_k is None else seed_k))
    s_h, s_w, s_y, _s_layout = ss.spawn(4)
    rh, rw, ry = (np.random.Generator(np.random.PCG64(s)) for s in (s_h, s_w, s_y))
    h = _normal_f32(rh, (M, D), 1.0)
    if hidden_scale != 1.0:
        h *= np.float32(hidden_scale)
    W = _normal_f32(rw, (V, D), 0.02)
    if prior:
        h[:, 0] = 1.0
        W[:, 0] = (-PRIOR_EXPONENT * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    seg = layout_pairs(spans)
    assert seg.shape[0] == M, (seg.shape, M)
    if targets == "zipf":
        y = zipf_ids(ry, M, V)
    else:
        y = uniform_ids(ry, M, V)
    y = np.where((seg & 3) == KIND_IGNORE, -1, y).astype(np.int32)
    hb, wb = f32_to_bf16_bits(h), f32_to_bf16_bits(W)
    return hb, wb, y, seg, (h if keep_raw else None), (W if keep_raw else None)


def make_workload(name: str, V: Optional[int] = None, M_scale: float = 1.0,
                  seed_k: Optional[int] = None) -> Workload:
    """Build one of the named workloads (the five configurations, and the
    Gemma-4B head with the token-frequency prior, "gemma4b_peaked").

    V overrides the vocab (used for the workspace-vs-V sweep and for reduced
    parity cases); M_scale shrinks every span (reduced parity cases).
    """
    k = CONFIG_NAMES.index(name)

    def sc(n, minimum=1):
        return max(minimum, int(round(n * M_scale)))

    if name == "tiny":
        spans = [(sc(31, 0), sc(128), sc(128))]
        D, VV, hs, tg, lam, scope, feps = 256, 4096, 1.0, "uniform", 0.1, SCOPE_FULL, 0.0
    elif name == "small_1b":
        spans = [(sc(255, 0), sc(512), sc(512))]
        D, VV, hs, tg, lam, scope, feps = 2048, 73448, 1.0, "zipf", 0.1, SCOPE_FULL, 0.0
    elif name == "long_1b":
        spans = [(sc(1023, 0), sc(2048), sc(2048))]
        D, VV, hs, tg, lam, scope, feps = 2048, 73448, 4.0, "zipf", 0.1, SCOPE_FULL, 1e-6
    elif name == "gemma4b_head":
        spans = [(sc(2048, 0), sc(3072), sc(3072))]
        D, VV, hs, tg, lam, scope, feps = 2560, 262144, 1.0, "zipf", 0.1, SCOPE_FULL, 0.0
    elif name == "gemma4b_peaked":
        # the Gemma-4B head's shape and layout; the pages' default skip eps 1e-5
        spans = [(sc(2048, 0), sc(3072), sc(3072))]
        D, VV, hs, tg, lam, scope, feps = 2560, 262144, 1.0, "zipf", 0.1, SCOPE_FULL, 1e-5
    elif name == "stress":
        ss = np.random.SeedSequence(BASE_SEED + (k if seed_k is None else seed_k))
        r_layout = np.random.Generator(np.random.PCG64(ss.spawn(4)[3]))
        Mtot = sc(16384, 64)
        spans = stress_spans(r_layout, M=Mtot, lo=min(64, max(1, Mtot // 256)),
                             hi=min(4096, max(2, Mtot // 4)))
        D, VV, hs, tg, lam, scope, feps = 4096, 262144, 1.0, "zipf", 0.5, SCOPE_RESPONSE, 1e-5
    else:
        raise KeyError(name)
    if V is not None:
        VV = int(V)
    M = int(sum(sum(sp) for sp in spans))
    hb, wb, y, seg, hr, wr = _draw(k, M, D, VV, spans, hs, tg, keep_raw=(name == "tiny"),
                                   seed_k=seed_k, prior=(name == "gemma4b_peaked"))
    return Workload(name=name, M=M, D=D, V=VV, h_bits=hb, W_bits=wb, y=y, seg=seg,
                    n_pairs=len(spans), lam=lam, scope=scope, filter_eps=feps,
                    h_f32_raw=hr, W_f32_raw=wr)


def make_custom(M_spans, D: int, V: int, seed: int, hidden_scale: float = 1.0,
                w_std: float = 0.02, targets: str = "uniform", lam: float = 0.1,
                scope: int = SCOPE_FULL) -> Workload:
    """Arbitrary shapes for edge-case tests (ragged M/V/D, many pairs, ...)."""
    ss = np.random.SeedSequence([BASE_SEED, seed])
    s_h, s_w, s_y = ss.spawn(3)
    rh, rw, ry = (np.random.Generator(np.random.PCG64(s)) for s in (s_h, s_w, s_y))
    seg = layout_pairs(M_spans)
    M = seg.shape[0]
    h = _normal_f32(rh, (M, D), 1.0) * np.float32(hidden_scale)
    W = _normal_f32(rw, (V, D), w_std)
    y = zipf_ids(ry, M, V) if targets == "zipf" else uniform_ids(ry, M, V)
    y = np.where((seg & 3) == KIND_IGNORE, -1, y).astype(np.int32)
    return Workload(name=f"custom_{seed}", M=M, D=D, V=V, h_bits=f32_to_bf16_bits(h),
                    W_bits=f32_to_bf16_bits(W), y=y, seg=seg, n_pairs=len(M_spans),
                    lam=lam, scope=scope)


# ----------------------------------------------------------------------------
# Quantised heads (input preparation): the affine group format of the pages'
# head ("Training — design …" §5.1 and §5.6: 4/8-bit affine with per-group
# scales and biases, one spec per head).  Per row v and group g of group_size
# consecutive columns: a scale s and a bias b (bf16 bit patterns), codes
# q in [0, 2^bits), packed little-endian into uint32 words along the row
# (code j of a word in bits [bits*j, bits*j + bits)).  The head value the
# codes stand for is s*q + b; computing it is the method's business, not this
# module's.  Codes are chosen by rounding against the stored (bf16) s and b.
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class QuantHead:
    bits: int
    group_size: int
    Wq: np.ndarray            # uint32 [V, D * bits / 32]
    scale_bits: np.ndarray    # uint16 [V, D / group_size]  bf16
    bias_bits: np.ndarray     # uint16 [V, D / group_size]  bf16


def quantize_affine(W: np.ndarray, bits: int, group_size: int) -> QuantHead:
    W = np.asarray(W, np.float64)
    V, D = W.shape
    assert bits in (4, 8) and D % group_size == 0 and (D * bits) % 32 == 0
    G = D // group_size
    Wg = W.reshape(V, G, group_size)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    levels = (1 << bits) - 1
    scale = np.where(hi > lo, (hi - lo) / levels, 1.0)
    s_bits = f32_to_bf16_bits(scale.astype(np.float32))
    b_bits = f32_to_bf16_bits(lo.astype(np.float32))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    b = bf16_bits_to_f32(b_bits).astype(np.float64)
    q = np.clip(np.rint((Wg - b[:, :, None]) / s[:, :, None]), 0, levels).astype(np.uint64)
    q = q.reshape(V, D)
    per = 32 // bits
    words = np.zeros((V, D // per), np.uint64)
    for j in range(per):
        words |= q[:, j::per] << np.uint64(bits * j)
    return QuantHead(bits=bits, group_size=group_size, Wq=words.astype(np.uint32),
                     scale_bits=s_bits, bias_bits=b_bits)
