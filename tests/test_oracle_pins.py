"""Pins of the fp64 oracle against things other than itself.

Each test fixes a part of the oracle by a closed form, a library routine, a
finite difference, brute force or an invariant, chosen so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand) fails at
least one of them.  Formulas cited are from:
  [P1] "Training — design (ORPO, flash-CCE head, prefix sharing, segmented
       backward)", §1 "The objective" and §5.1 "The head";
  [P2] "ORPO training — design", "The objective", "File-by-file changes",
       "Recommended defaults", "Parity".
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import cce_oracle as O
from linear_cross_entropy_forward_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers (test-side, independent evaluations)
# ----------------------------------------------------------------------------
def odds_ratio_log(lw, lr):
    """Textbook log odds ratio: odds(p) = p / (1 - p) with p = e^l."""
    pw, pr = math.exp(lw), math.exp(lr)
    return math.log(pw / (1 - pw)) - math.log(pr / (1 - pr))


def dec_log1mexp(x, digits=60):
    """log(1 - e^x) in high-precision decimal arithmetic."""
    getcontext().prec = digits
    d = Decimal(repr(x))
    return float((Decimal(1) - d.exp()).ln())


def pair_rows(spans):
    return WL.layout_pairs(spans)


# ----------------------------------------------------------------------------
# P1: closed-form ORPO scalars (hand-derived from [P1] §1 / [P2] "The objective")
# ----------------------------------------------------------------------------
E = math.e


@pytest.mark.parametrize("lw,lr,lam,lo,lor,L,dlw,dlr", [
    # (-1, -2): odds ratio = (e^2 - 1)/(e - 1) = e + 1, so log_odds = ln(1 + e);
    # sigma(log_odds) = (1+e)/(2+e); d log_odds/d lw = e/(e-1), d/d lr = -e^2/(e^2-1).
    (-1.0, -2.0, 0.1, math.log(1 + E), math.log((2 + E) / (1 + E)),
     1.0 + 0.1 * math.log((2 + E) / (1 + E)),
     -1.0 - 0.1 / (2 + E) * E / (E - 1), 0.1 / (2 + E) * E * E / (E * E - 1)),
    # (-0.5, -0.5): log_odds = 0, L_OR = ln 2, sigma = 1/2.
    (-0.5, -0.5, 0.1, 0.0, math.log(2.0), 0.5 + 0.1 * math.log(2.0),
     -1.0 - 0.05 / (1 - math.exp(-0.5)), 0.05 / (1 - math.exp(-0.5))),
    # (-1.5, -0.7), lambda 0.5: log_odds = -0.8 - ln((1 - e^-1.5) / (1 - e^-0.7)), worked by
    # hand to 12 digits (and checked against 50-digit decimal arithmetic below)
    (-1.5, -0.7, 0.5, -1.233858543883, 1.489404947951, 2.244702473976,
     -1.498470371973, 0.769239755935),
])
def test_p1_closed_form_scalars(lw, lr, lam, lo, lor, L, dlw, dlr):
    # the third point's values are printed to 12 digits: compare at that precision
    rel = 1e-11 if lw == -1.5 else 1e-12
    assert O.log_odds(lw, lr) == pytest.approx(lo, rel=max(rel, 1e-13), abs=1e-14)
    assert O.or_term(lw, lr) == pytest.approx(lor, rel=max(rel, 1e-13))
    assert O.orpo_pair_loss(lw, lr, lam) == pytest.approx(L, rel=max(rel, 1e-13))
    g = O.orpo_pair_grad(lw, lr, lam)
    assert g[0] == pytest.approx(dlw, rel=rel)
    assert g[1] == pytest.approx(dlr, rel=rel)


def test_p1_third_point_in_decimal_arithmetic():
    """(lw, lr) = (-1.5, -0.7), lambda 0.5, response scope, evaluated from the
    definitions in 50-digit decimal arithmetic (no oracle code): log_odds,
    L_OR = ln(1 + e^-log_odds), L = -lw + lambda L_OR, and the partials by the
    chain rule, d log_odds/d l = 1 / (1 - e^l)."""
    getcontext().prec = 50
    lw, lr, lam = Decimal("-1.5"), Decimal("-0.7"), Decimal("0.5")
    one = Decimal(1)
    lo = (lw - lr) - ((one - lw.exp()).ln() - (one - lr.exp()).ln())
    lor = (one + (-lo).exp()).ln()
    L = -lw + lam * lor
    sig = one / (one + (-lo).exp())
    dlw = -one - lam * (one - sig) / (one - lw.exp())
    dlr = lam * (one - sig) / (one - lr.exp())
    assert float(lo) == pytest.approx(-1.233858543883, abs=5e-13)
    assert float(lor) == pytest.approx(1.489404947951, abs=5e-13)
    assert float(L) == pytest.approx(2.244702473976, abs=5e-13)
    assert float(dlw) == pytest.approx(-1.498470371973, abs=5e-13)
    assert float(dlr) == pytest.approx(0.769239755935, abs=5e-13)
    g = O.orpo_pair_grad(-1.5, -0.7, 0.5)
    assert O.orpo_pair_loss(-1.5, -0.7, 0.5) == pytest.approx(float(L), rel=1e-14)
    assert g[0] == pytest.approx(float(dlw), rel=1e-13)
    assert g[1] == pytest.approx(float(dlr), rel=1e-13)


def test_oracle_regression_fixture():
    """The oracle's outputs on a tiny seeded case, written by
    tests/golden/make_oracle_fixture.py (which calls only the oracle).  A
    change here must come with the passage or reading that justifies it."""
    with open(os.path.join(GOLDEN, "oracle_tiny_fixture.json")) as f:
        fx = json.load(f)
    H = np.array(fx["H"]); W = np.array(fx["W"])
    y = np.array(fx["y"], np.int64); seg = np.array(fx["seg"], np.int64)
    for sc, key in ((O.SCOPE_FULL, "full"), (O.SCOPE_RESPONSE, "response")):
        out = O.step(H, W, y, seg, fx["n_pairs"], fx["lambda"], sc)
        ref = fx[key]
        for k in ("loss", "nll", "orv", "margin", "accuracy"):
            assert out[k] == pytest.approx(ref[k], rel=1e-12, abs=1e-15)
        for k in ("logp", "lse", "coef", "dh", "dW"):
            np.testing.assert_allclose(out[k], np.array(ref[k]), rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("lw,lr", [(-1.5, -0.7), (-11.2, -11.9), (-0.01, -3.0), (-25.0, -0.2)])
def test_p1_log_odds_is_the_odds_ratio(lw, lr):
    """log_odds equals the log of the ratio of odds p/(1-p) ([P1] §1)."""
    assert O.log_odds(lw, lr) == pytest.approx(odds_ratio_log(lw, lr), rel=1e-9, abs=1e-12)


def test_p1_mlx_lm_lora_variant_differs():
    """The log_sigmoid(chosen - rejected) variant without the NLL term ([P1] §2)
    is not our loss."""
    for lw, lr in [(-1.0, -2.0), (-11.0, -12.0), (-3.0, -1.0)]:
        ours = O.orpo_pair_loss(lw, lr, 0.1)
        theirs = -math.log(1 / (1 + math.exp(-(lw - lr))))
        assert abs(ours - theirs) > 1e-3


# ----------------------------------------------------------------------------
# P2: log1mexp stability ([P1] §1; [P2] "Recommended defaults": clamp / two-branch)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("x", [-math.log(2.0), -1.0, -20.0, -50.0, -1e-3, -0.3, -0.9, -700.0])
def test_p2_log1mexp_matches_high_precision(x):
    ref = dec_log1mexp(x)
    got = O.log1mexp(x)
    assert got == pytest.approx(ref, rel=1e-14, abs=1e-300)


def test_p2_log1mexp_tail_not_zero():
    # naive log(1 - exp(-50)) rounds to 0 in fp64; the two-branch form does not
    assert O.log1mexp(-50.0) == pytest.approx(-1.9287498479639178e-22, rel=1e-12)
    assert O.log1mexp(-800.0) == 0.0


def test_p2_log1mexp_clamp():
    clamp = math.log(1e-7)
    assert O.log1mexp(-1e-10) == pytest.approx(clamp, rel=1e-15)
    assert O.log1mexp(-1e-7) == pytest.approx(clamp, rel=1e-15)
    assert O.dlog1mexp(-1e-10) == 0.0
    # just outside the clamp the value is the exact one
    x = -2e-7
    assert O.log1mexp(x) == pytest.approx(dec_log1mexp(x), rel=1e-12)
    # derivative: -e^x / (1 - e^x), checked by a central difference
    for x in [-0.05, -1.0, -7.0]:
        h = 1e-6
        fd = (O.log1mexp(x + h) - O.log1mexp(x - h)) / (2 * h)
        assert O.dlog1mexp(x) == pytest.approx(fd, rel=1e-7)


# ----------------------------------------------------------------------------
# P3: full-scope NLL combine ([P1] §1)
# ----------------------------------------------------------------------------
def test_p3_full_nll_combine():
    assert O.full_nll(-2.0, 3, -1.0, 2) == pytest.approx(1.6, rel=1e-15)
    assert O.full_nll(-7.0, 0, -1.25, 9) == pytest.approx(1.25, rel=1e-15)
    # in the batch epilogue: one pair, 3 prompt rows with logp -2, 2 chosen with -1
    seg = pair_rows([(3, 2, 1)])
    logp = np.array([-2, -2, -2, -1, -1, -0.5], float)
    ep = O.epilogue(logp, seg, 1, 0.0, O.SCOPE_FULL)
    assert ep["nll"] == pytest.approx(1.6, rel=1e-15)
    assert ep["loss"] == pytest.approx(1.6, rel=1e-15)
    ep = O.epilogue(logp, seg, 1, 0.0, O.SCOPE_RESPONSE)
    assert ep["nll"] == pytest.approx(1.0, rel=1e-15)


# ----------------------------------------------------------------------------
# P4: library special case — lambda = 0, response scope: loss = mean CE over
# the chosen rows; check forward against torch.nn.functional.cross_entropy and
# the backward against torch.autograd (fp64, CPU).
# ----------------------------------------------------------------------------
def test_p4_torch_cross_entropy_and_autograd():
    torch = pytest.importorskip("torch")
    wl = WL.make_custom([(3, 9, 7, 2)], D=24, V=53, seed=11, hidden_scale=2.0, w_std=0.3)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    logp, lse = O.forward(H, W, y)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    Z = Ht @ Wt.T
    valid = torch.tensor(y >= 0)
    yt = torch.tensor(np.maximum(y, 0), dtype=torch.long)
    ce = torch.nn.functional.cross_entropy(Z, yt, reduction="none")
    np.testing.assert_allclose(logp[y >= 0], (-ce[valid]).detach().numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(Z, 1).detach().numpy(), rtol=1e-14)
    assert np.all(logp[y < 0] == 0.0)

    chosen = torch.tensor((seg & 3) == WL.KIND_CHOSEN)
    loss_t = torch.nn.functional.cross_entropy(Z[chosen], yt[chosen], reduction="mean")
    loss_t.backward()
    ep = O.epilogue(logp, seg, 1, 0.0, O.SCOPE_RESPONSE)
    assert ep["loss"] == pytest.approx(loss_t.item(), rel=1e-13)
    dh, dW = O.backward(H, W, y, lse, ep["coef"])
    np.testing.assert_allclose(dh, Ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_p4_autograd_full_orpo_chain():
    """The analytic backward (coef from the epilogue, then G W / G^T H) equals
    autograd through the plain composition logits -> log_softmax -> gather ->
    per-pair means -> ORPO loss (torch fp64)."""
    torch = pytest.importorskip("torch")
    spans = [(4, 6, 5, 1), (0, 3, 4), (2, 5, 5, 3)]
    wl = WL.make_custom(spans, D=16, V=29, seed=5, hidden_scale=1.5, w_std=0.4, lam=0.7)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    kind, pair = seg & 3, seg >> 2
    for scope in (O.SCOPE_FULL, O.SCOPE_RESPONSE):
        Ht = torch.tensor(H, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        lsm = torch.log_softmax(Ht @ Wt.T, dim=1)
        lp = lsm[torch.arange(len(y)), torch.tensor(np.maximum(y, 0))] * torch.tensor(y >= 0)
        losses = []
        for b in range(len(spans)):
            C = torch.tensor((pair == b) & (kind == WL.KIND_CHOSEN))
            R = torch.tensor((pair == b) & (kind == WL.KIND_REJECTED))
            Q = torch.tensor((pair == b) & (kind == WL.KIND_PROMPT))
            lw, lr = lp[C].mean(), lp[R].mean()
            lo = (lw - lr) - (torch.log(-torch.expm1(lw)) - torch.log(-torch.expm1(lr)))
            orb = -torch.nn.functional.logsigmoid(lo)
            if scope == O.SCOPE_FULL:
                nll = -(lp[Q].sum() + lp[C].sum()) / (int(Q.sum()) + int(C.sum()))
            else:
                nll = -lw
            losses.append((nll, orb))
        nll = torch.stack([a for a, _ in losses]).mean()
        orv = torch.stack([b for _, b in losses]).mean()
        loss = nll + wl.lam * orv
        loss.backward()
        logp, lse = O.forward(H, W, y)
        ep = O.epilogue(logp, seg, len(spans), wl.lam, scope)
        assert ep["loss"] == pytest.approx(loss.item(), rel=1e-12)
        assert ep["nll"] == pytest.approx(nll.item(), rel=1e-12)
        assert ep["orv"] == pytest.approx(orv.item(), rel=1e-12)
        dh, dW = O.backward(H, W, y, lse, ep["coef"])
        np.testing.assert_allclose(dh, Ht.grad.numpy(), rtol=1e-10, atol=1e-15)
        np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-15)


# ----------------------------------------------------------------------------
# P5: closed form at W = 0
# ----------------------------------------------------------------------------
def test_p5_zero_head():
    wl = WL.make_custom([(5, 7, 6, 2), (1, 4, 9)], D=12, V=37, seed=3)
    H, y, seg = wl.h64(), wl.y, wl.seg
    V = wl.V
    W = np.zeros((V, wl.D))
    logp, lse = O.forward(H, W, y)
    assert np.all(lse == pytest.approx(math.log(V), rel=1e-15))
    assert np.all(logp[y >= 0] == pytest.approx(-math.log(V), rel=1e-15))
    ep = O.epilogue(logp, seg, 2, 0.3, O.SCOPE_FULL)
    dh, dW = O.backward(H, W, y, lse, ep["coef"])
    assert np.all(dh == 0.0)
    coef = ep["coef"]
    ref = np.zeros((V, wl.D))
    for i in range(wl.M):
        for v in range(V):
            ref[v] += coef[i] * (1.0 / V - (1.0 if y[i] == v else 0.0)) * H[i]
    np.testing.assert_allclose(dW, ref, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------
# P6: invariants
# ----------------------------------------------------------------------------
def _case():
    spans = [(3, 8, 6, 2), (2, 5, 7)]
    return WL.make_custom(spans, D=10, V=31, seed=9, hidden_scale=2.0, w_std=0.5, lam=0.4)


def test_p6_invariants_forward():
    wl = _case()
    H, W, y = wl.h64(), wl.W64(), wl.y
    logp, lse = O.forward(H, W, y)
    Z = H @ W.T
    assert np.all(logp <= 0.0)
    assert np.all(lse >= Z.max(axis=1))
    # vocab permutation
    perm = np.random.default_rng(0).permutation(wl.V)
    inv = np.argsort(perm)
    y2 = np.where(y >= 0, inv[np.maximum(y, 0)], -1)
    lp2, ls2 = O.forward(H, W[perm], y2)
    np.testing.assert_allclose(lp2, logp, rtol=1e-13)
    np.testing.assert_allclose(ls2, lse, rtol=1e-13)


def test_p6_invariants_backward():
    wl = _case()
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    logp, lse = O.forward(H, W, y)
    ep = O.epilogue(logp, seg, wl.n_pairs, wl.lam, O.SCOPE_FULL)
    coef = ep["coef"]
    dh, dW = O.backward(H, W, y, lse, coef)
    # sum over the vocab of dW is zero: each row's softmax sums to 1 = its onehot
    np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-12)
    # per-row form of dh
    P = np.exp(H @ W.T - lse[:, None])
    for i in range(wl.M):
        ref = coef[i] * (P[i] @ W - (W[y[i]] if y[i] >= 0 else 0.0))
        np.testing.assert_allclose(dh[i], ref, rtol=1e-11, atol=1e-15)
    # ignore rows: coef and dh rows exactly 0
    ign = (seg & 3) == WL.KIND_IGNORE
    assert np.all(coef[ign] == 0.0)
    assert np.all(dh[ign] == 0.0)
    # vocab permutation permutes dW
    perm = np.random.default_rng(1).permutation(wl.V)
    inv = np.argsort(perm)
    y2 = np.where(y >= 0, inv[np.maximum(y, 0)], -1)
    lp2, ls2 = O.forward(H, W[perm], y2)
    ep2 = O.epilogue(lp2, seg, wl.n_pairs, wl.lam, O.SCOPE_FULL)
    dh2, dW2 = O.backward(H, W[perm], y2, ls2, ep2["coef"])
    np.testing.assert_allclose(dW2, dW[perm], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dh2, dh, rtol=1e-10, atol=1e-14)


def test_p6_invariants_epilogue():
    rng = np.random.default_rng(4)
    seg = WL.layout_pairs([(3, 5, 4, 1), (0, 6, 2)])
    logp = -rng.uniform(0.5, 12, size=seg.shape[0])
    for scope in (O.SCOPE_FULL, O.SCOPE_RESPONSE):
        ep = O.epilogue(logp, seg, 2, 0.2, scope)
        # row permutation within a pair's span leaves everything unchanged
        perm = np.arange(len(seg))
        perm[3:8] = perm[3:8][::-1]
        ep2 = O.epilogue(logp[perm], seg[perm], 2, 0.2, scope)
        assert ep2["loss"] == pytest.approx(ep["loss"], rel=1e-14)
        # duplicating every pair leaves the batch means unchanged
        seg_dup = np.concatenate([seg, seg + (2 << 2)])
        ep3 = O.epilogue(np.concatenate([logp, logp]), seg_dup, 4, 0.2, scope)
        for k in ("loss", "nll", "orv", "margin", "accuracy"):
            assert ep3[k] == pytest.approx(ep[k], rel=1e-14)
        # ignore rows carry no weight, and changing their logp changes nothing
        ign = (seg & 3) == WL.KIND_IGNORE
        assert np.all(ep["coef"][ign] == 0.0)
        lp4 = logp.copy()
        lp4[ign] = -99.0
        assert O.epilogue(lp4, seg, 2, 0.2, scope)["loss"] == ep["loss"]
        # prompt rows carry no weight in response scope
        prm = (seg & 3) == WL.KIND_PROMPT
        if scope == O.SCOPE_RESPONSE:
            assert np.all(ep["coef"][prm] == 0.0)
        else:
            assert np.all(ep["coef"][prm] > 0.0)
        # sign convention: chosen coef > 0, rejected coef < 0
        assert np.all(ep["coef"][(seg & 3) == WL.KIND_CHOSEN] > 0)
        assert np.all(ep["coef"][(seg & 3) == WL.KIND_REJECTED] < 0)


def test_p6_accuracy_and_margin():
    seg = WL.layout_pairs([(0, 1, 1), (0, 1, 1), (0, 1, 1)])
    logp = np.array([-1.0, -2.0, -3.0, -3.0, -4.0, -1.0])
    ep = O.epilogue(logp, seg, 3, 0.1, O.SCOPE_RESPONSE)
    assert ep["accuracy"] == pytest.approx(1.0 / 3.0)       # strict >, tie is a miss
    lo = [odds_ratio_log(-1, -2), 0.0, odds_ratio_log(-4, -1)]
    assert ep["margin"] == pytest.approx(np.mean(lo), rel=1e-12)


# ----------------------------------------------------------------------------
# P7: finite differences of the whole chain (H, W -> loss)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("scope", [O.SCOPE_FULL, O.SCOPE_RESPONSE])
def test_p7_finite_differences(scope):
    spans = [(2, 3, 2, 1), (1, 2, 3), (0, 1, 1)]          # M = 16, all four kinds
    wl = WL.make_custom(spans, D=6, V=11, seed=21, hidden_scale=1.3, w_std=0.6, lam=0.35)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    B = len(spans)

    def L(Hx, Wx):
        lp, _ = O.forward(Hx, Wx, y)
        return O.epilogue(lp, seg, B, wl.lam, scope)["loss"]

    logp, lse = O.forward(H, W, y)
    ep = O.epilogue(logp, seg, B, wl.lam, scope)
    dh, dW = O.backward(H, W, y, lse, ep["coef"])
    eps = 1e-6
    fdH = np.zeros_like(H)
    for i in range(H.shape[0]):
        for d in range(H.shape[1]):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, d] += eps
            Hm[i, d] -= eps
            fdH[i, d] = (L(Hp, W) - L(Hm, W)) / (2 * eps)
    fdW = np.zeros_like(W)
    for v in range(W.shape[0]):
        for d in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, d] += eps
            Wm[v, d] -= eps
            fdW[v, d] = (L(H, Wp) - L(H, Wm)) / (2 * eps)
    assert np.linalg.norm(dh - fdH) / np.linalg.norm(fdH) < 1e-6
    assert np.linalg.norm(dW - fdW) / np.linalg.norm(fdW) < 1e-6


def test_p7_finite_differences_of_coef():
    """coef_i = -dL/dlogp_i, by central differences on the epilogue alone."""
    seg = WL.layout_pairs([(2, 3, 2, 1), (1, 2, 3)])
    rng = np.random.default_rng(8)
    logp = -rng.uniform(0.3, 4.0, size=seg.shape[0])
    for scope in (O.SCOPE_FULL, O.SCOPE_RESPONSE):
        ep = O.epilogue(logp, seg, 2, 0.6, scope)
        for i in range(len(logp)):
            e = 1e-6
            lp, lm = logp.copy(), logp.copy()
            lp[i] += e
            lm[i] -= e
            fd = (O.loss_from_logp(lp, seg, 2, 0.6, scope) - O.loss_from_logp(lm, seg, 2, 0.6, scope)) / (2 * e)
            assert -fd == pytest.approx(ep["coef"][i], rel=1e-6, abs=1e-10)


# ----------------------------------------------------------------------------
# P8: brute force with per-element loops (no matmul, no vector logsumexp)
# ----------------------------------------------------------------------------
def test_p8_brute_force():
    spans = [(1, 2, 1, 1)]          # M = 5
    wl = WL.make_custom(spans, D=3, V=7, seed=2, hidden_scale=1.0, w_std=0.8, lam=0.25)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    M, V, D = wl.M, wl.V, wl.D
    z = [[sum(H[i][d] * W[v][d] for d in range(D)) for v in range(V)] for i in range(M)]
    lse = [math.log(sum(math.exp(z[i][v]) for v in range(V))) for i in range(M)]
    logp = [(z[i][y[i]] - lse[i]) if y[i] >= 0 else 0.0 for i in range(M)]
    lp_o, lse_o = O.forward(H, W, y)
    np.testing.assert_allclose(lp_o, logp, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse_o, lse, rtol=1e-12)
    ep = O.epilogue(lp_o, seg, 1, wl.lam, O.SCOPE_FULL)
    coef = ep["coef"]
    dh = [[0.0] * D for _ in range(M)]
    dW = [[0.0] * D for _ in range(V)]
    for i in range(M):
        for v in range(V):
            g = coef[i] * (math.exp(z[i][v] - lse[i]) - (1.0 if v == y[i] else 0.0))
            for d in range(D):
                dh[i][d] += g * W[v][d]
                dW[v][d] += g * H[i][d]
    dh_o, dW_o = O.backward(H, W, y, lse_o, coef)
    np.testing.assert_allclose(dh_o, dh, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(dW_o, dW, rtol=1e-11, atol=1e-15)


# ----------------------------------------------------------------------------
# P9: integer handling
# ----------------------------------------------------------------------------
def test_p9_counts_and_zero_coef():
    spans = [(7, 11, 5, 3), (0, 2, 9, 4), (1, 1, 1)]
    seg = WL.layout_pairs(spans)
    logp = -np.linspace(1, 5, seg.shape[0])
    ep = O.epilogue(logp, seg, 3, 0.1, O.SCOPE_RESPONSE)
    assert list(ep["Pm1"]) == [7, 0, 1]
    assert list(ep["Mw"]) == [11, 2, 1]
    assert list(ep["Mr"]) == [5, 9, 1]
    kind = seg & 3
    assert np.all(ep["coef"][(kind == WL.KIND_IGNORE) | (kind == WL.KIND_PROMPT)] == 0.0)
    with pytest.raises(ValueError):
        O.epilogue(logp, WL.layout_pairs([(1, 3, 0, 0)] + spans[1:])[: len(logp)], 3, 0.1, O.SCOPE_FULL)


def test_p9_target_gather_index():
    """The gathered logit is z[i, y_i] exactly (not a neighbour, not transposed)."""
    M, V, D = 6, 9, 4
    H = np.eye(M, D) * 3.0
    W = np.zeros((V, D))
    for v in range(V):
        W[v, v % D] = float(v)           # z[i, v] = 3 * v if v % D == i else 0
    y = np.array([0, 5, 2, 7, -1, 3])
    logp, lse = O.forward(H, W, y)
    Z = H @ W.T
    for i in range(M):
        if y[i] >= 0:
            assert logp[i] == Z[i, y[i]] - lse[i]


# ----------------------------------------------------------------------------
# filter mode (reported, not gated): it only drops sub-eps softmax entries
# ----------------------------------------------------------------------------
def test_filter_mode_drops_only_small_entries():
    wl = WL.make_custom([(2, 6, 6)], D=8, V=200, seed=13, hidden_scale=3.0, w_std=1.0)
    H, W, y = wl.h64(), wl.W64(), wl.y
    logp, lse = O.forward(H, W, y)
    coef = O.epilogue(logp, wl.seg, 1, 0.1, O.SCOPE_FULL)["coef"]
    Z = H @ W.T
    G0 = O.grad_logits(Z, lse, y, coef, 0.0)
    G1 = O.grad_logits(Z, lse, y, coef, 1e-3)
    P = np.exp(Z - lse[:, None])
    changed = G0 != G1
    assert np.all(P[changed] < 1e-3)
    for i in range(wl.M):
        assert G1[i, y[i]] == G0[i, y[i]]
    assert changed.sum() > 0


def test_filter_mode_brute_force():
    """The filtered gradient on a tiny case, written out with scalar loops: a
    non-target entry whose softmax value is below eps contributes nothing, every
    other entry is coef * (p - onehot).  Drops exactly that set (an entry at
    p >= eps stays), and the target is kept however small its p."""
    rng = np.random.default_rng(21)
    M, V, D, eps = 5, 40, 6, 2e-2
    H = rng.normal(size=(M, D)) * 1.5
    W = rng.normal(size=(V, D))
    y = np.array([3, 17, -1, 39, 0])
    coef = np.array([0.7, -1.3, 0.4, 2.0, -0.2])
    Z = H @ W.T
    # make row 0's target tiny (it must survive the filter) and put one entry
    # of row 1 exactly at the threshold (it must survive too: only p < eps drops)
    Z[0, 3] = Z[0].max() - 30.0
    zmax1 = Z[1].max()
    ssum = sum(math.exp(Z[1, v] - zmax1) for v in range(V) if v != 5)
    Z[1, 5] = zmax1 + math.log(eps * ssum / (1.0 - eps))
    lse = np.array([max(Z[i]) + math.log(sum(math.exp(Z[i, v] - max(Z[i])) for v in range(V)))
                    for i in range(M)])
    G = O.grad_logits(Z, lse, y, coef, eps)
    dropped = 0
    for i in range(M):
        for v in range(V):
            p = math.exp(Z[i, v] - lse[i])
            tgt = 1.0 if v == y[i] else 0.0
            want = 0.0 if (p < eps and tgt == 0.0) else coef[i] * (p - tgt)
            dropped += p < eps and tgt == 0.0
            assert abs(G[i, v] - want) <= 1e-12 * max(1.0, abs(want)), (i, v)
    assert math.exp(Z[1, 5] - lse[1]) == eps  # exactly at the threshold in this seeded case
    assert G[1, 5] != 0.0 and G[0, 3] != 0.0
    assert 0 < dropped < M * V


# ----------------------------------------------------------------------------
# input generators
# ----------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10 ** rng.uniform(-5, 5, 10000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00390625, 0.0, -0.0], np.float32)])
    ours = WL.f32_to_bf16_bits(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(WL.bf16_bits_to_f32(ours), torch.tensor(x).to(torch.bfloat16).float().numpy())


def test_workload_determinism_and_layouts():
    a = WL.make_workload("tiny")
    b = WL.make_workload("tiny")
    assert np.array_equal(a.h_bits, b.h_bits) and np.array_equal(a.W_bits, b.W_bits)
    assert np.array_equal(a.y, b.y) and np.array_equal(a.seg, b.seg)
    assert (a.M, a.D, a.V) == (287, 256, 4096)
    kinds = np.bincount(a.seg & 3, minlength=4)
    assert list(kinds) == [0, 31, 128, 128]
    assert a.h_f32_raw is not None


def test_stress_layout():
    rng = np.random.default_rng(np.random.SeedSequence(WL.BASE_SEED + 4).spawn(4)[3])
    spans = WL.stress_spans(rng)
    seg = WL.layout_pairs(spans)
    kinds = np.bincount(seg & 3, minlength=4)
    assert seg.shape[0] == 16384
    assert kinds[WL.KIND_IGNORE] == 1638 and kinds[WL.KIND_PROMPT] == 3277
    assert kinds[WL.KIND_CHOSEN] + kinds[WL.KIND_REJECTED] == 11469
    lens = [s[1] for s in spans] + [s[2] for s in spans]
    assert min(lens) >= 64 and max(lens) <= 4096 and len(spans) == 8


def test_zipf_histogram():
    rng = np.random.default_rng(3)
    V = 1000
    ids = WL.zipf_ids(rng, 200000, V)
    p = np.arange(1, V + 1, dtype=float) ** -1.1
    p /= p.sum()
    counts = np.bincount(ids, minlength=V)
    for k in (0, 1, 2, 9, 99):
        expect = p[k] * 200000
        assert abs(counts[k] - expect) < 4.0 * math.sqrt(expect)     # 4 sigma
    assert ids.min() >= 0 and ids.max() < V


# ----------------------------------------------------------------------------
# P10: final-logit softcap ([P1] §5.1, the e4b head with cap 30; [P2] lever 1
# "Implementation spec": logit = cap * tanh(raw / cap), folded into both the
# log-sum-exp and the backward, d logit / d raw = sech^2(raw / cap))
# ----------------------------------------------------------------------------
def test_p10_softcap_binds_closed_form():
    """One raw logit far above the cap: the capped logit is the cap itself, so
    logp = cap - log(e^cap + (V - 1)) for that target and -log(e^cap + V - 1)
    for any other (an uncapped head would give about 0 and about -1e4)."""
    V, cap = 5, 30.0
    H = np.array([[1.0], [1.0]])
    W = np.array([[1.0e4], [0.0], [0.0], [0.0], [0.0]])
    y = np.array([0, 3])
    logp, lse = O.forward(H, W, y, softcap=cap)
    den = math.log(math.exp(cap) + (V - 1))
    assert logp[0] == pytest.approx(cap - den, rel=1e-14, abs=1e-15)
    assert logp[1] == pytest.approx(-den, rel=1e-14)
    assert lse[0] == pytest.approx(den, rel=1e-14)


def test_p10_softcap_large_cap_is_uncapped():
    wl = _case()
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    lp0, ls0 = O.forward(H, W, y)
    lp1, ls1 = O.forward(H, W, y, softcap=1.0e7)
    np.testing.assert_allclose(lp1, lp0, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ls1, ls0, rtol=1e-9)
    coef = O.epilogue(lp0, seg, 2, wl.lam, O.SCOPE_FULL)["coef"]
    dh0, dW0 = O.backward(H, W, y, ls0, coef)
    dh1, dW1 = O.backward(H, W, y, ls1, coef, softcap=1.0e7)
    np.testing.assert_allclose(dh1, dh0, rtol=1e-8, atol=1e-14)
    np.testing.assert_allclose(dW1, dW0, rtol=1e-8, atol=1e-14)


def test_p10_softcap_torch_autograd():
    """Forward and the analytic backward with a cap that binds (logit scale
    several times the cap) equal torch fp64 autograd through cap * tanh."""
    torch = pytest.importorskip("torch")
    spans = [(3, 6, 5, 2), (1, 4, 4)]
    wl = WL.make_custom(spans, D=12, V=23, seed=17, hidden_scale=3.0, w_std=1.0, lam=0.5)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    cap = 2.5
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    Z = cap * torch.tanh((Ht @ Wt.T) / cap)
    lsm = torch.log_softmax(Z, dim=1)
    lp_t = lsm[torch.arange(len(y)), torch.tensor(np.maximum(y, 0))] * torch.tensor(y >= 0)
    logp, lse = O.forward(H, W, y, softcap=cap)
    np.testing.assert_allclose(logp, lp_t.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(Z, 1).detach().numpy(), rtol=1e-13)
    ep = O.epilogue(logp, seg, 2, wl.lam, O.SCOPE_FULL)
    # the loss as a function of lp_t, through the oracle's coef (dL/dlogp = -coef)
    (-(torch.tensor(ep["coef"]) * lp_t).sum()).backward()
    dh, dW = O.backward(H, W, y, lse, ep["coef"], softcap=cap)
    np.testing.assert_allclose(dh, Ht.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_p10_softcap_finite_differences():
    spans = [(2, 3, 2, 1), (1, 2, 3)]
    wl = WL.make_custom(spans, D=5, V=9, seed=23, hidden_scale=2.5, w_std=1.2, lam=0.3)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    cap = 1.5

    def L(Hx, Wx):
        lp, _ = O.forward(Hx, Wx, y, softcap=cap)
        return O.epilogue(lp, seg, 2, wl.lam, O.SCOPE_FULL)["loss"]

    logp, lse = O.forward(H, W, y, softcap=cap)
    ep = O.epilogue(logp, seg, 2, wl.lam, O.SCOPE_FULL)
    dh, dW = O.backward(H, W, y, lse, ep["coef"], softcap=cap)
    eps = 1e-6
    fdH = np.zeros_like(H)
    for i in range(H.shape[0]):
        for d in range(H.shape[1]):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, d] += eps
            Hm[i, d] -= eps
            fdH[i, d] = (L(Hp, W) - L(Hm, W)) / (2 * eps)
    fdW = np.zeros_like(W)
    for v in range(W.shape[0]):
        for d in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, d] += eps
            Wm[v, d] -= eps
            fdW[v, d] = (L(H, Wp) - L(H, Wm)) / (2 * eps)
    assert np.linalg.norm(dh - fdH) / np.linalg.norm(fdH) < 1e-6
    assert np.linalg.norm(dW - fdW) / np.linalg.norm(fdW) < 1e-6
    # the cap matters here: the same gradient with the sech^2 factor dropped
    # (softmax of the capped logits, no chain rule through the cap) is far off
    Zc = cap * np.tanh((H @ W.T) / cap)
    onehot = np.zeros_like(Zc)
    onehot[np.nonzero(y >= 0)[0], y[y >= 0]] = 1.0
    dh_nosech = (ep["coef"][:, None] * (np.exp(Zc - lse[:, None]) - onehot)) @ W
    assert np.linalg.norm(dh_nosech - fdH) / np.linalg.norm(fdH) > 1e-2


# ----------------------------------------------------------------------------
# P11: the preference-objective family ([P1] §8.3; "ORPO from-base on
# UltraFeedback — results + research directions" §6.1-6.3)
# ----------------------------------------------------------------------------
OBJECTIVES = [O.OBJ_ORPO, O.OBJ_SIGMOID, O.OBJ_IPO, O.OBJ_HINGE]


def test_p11_orpo_member_is_the_orpo_epilogue():
    seg = WL.layout_pairs([(2, 3, 2, 1), (1, 2, 3), (0, 4, 2)])
    rng = np.random.default_rng(31)
    logp = -rng.uniform(0.3, 4.0, size=seg.shape[0])
    for scope in (O.SCOPE_FULL, O.SCOPE_RESPONSE):
        a = O.epilogue(logp, seg, 3, 0.45, scope)
        b = O.pref_epilogue(logp, seg, 3, O.OBJ_ORPO, 1.0, 0.45, 7.0, 9.0, scope)
        assert b["loss"] == a["loss"] and b["nll"] == a["nll"] and b["pref"] == a["orv"]
        assert b["margin"] == a["margin"] and b["accuracy"] == a["accuracy"]
        np.testing.assert_array_equal(b["coef"], a["coef"])
        np.testing.assert_array_equal(b["s"], a["log_odds"])


def _dec_softplus_neg(x):
    """softplus(-x) = log(1 + e^-x) in 50-digit decimal arithmetic."""
    getcontext().prec = 50
    return float((Decimal(1) + (-Decimal(x)).exp()).ln())


@pytest.mark.parametrize("lw,lr,beta,gamma", [(-1.2, -1.5, 2.0, 0.5), (-3.0, -2.1, 0.7, 0.1),
                                               (-0.4, -0.4, 3.0, 0.0)])
def test_p11_closed_forms_one_pair(lw, lr, beta, gamma):
    """One pair, one chosen and one rejected row, response scope: every term
    evaluated independently by hand (decimal arithmetic for the softplus)."""
    seg = WL.layout_pairs([(0, 1, 1)])
    logp = np.array([lw, lr])
    s = beta * (lw - lr) - gamma
    want = {O.OBJ_SIGMOID: _dec_softplus_neg(s), O.OBJ_IPO: s * s, O.OBJ_HINGE: max(0.0, gamma - beta * (lw - lr))}
    for obj, P in want.items():
        for w_nll, lam in ((0.0, 1.0), (1.0, 0.3)):
            ep = O.pref_epilogue(logp, seg, 1, obj, w_nll, lam, beta, gamma, O.SCOPE_RESPONSE)
            assert ep["pref"] == pytest.approx(P, rel=1e-14, abs=1e-15)
            assert ep["loss"] == pytest.approx(w_nll * (-lw) + lam * P, rel=1e-14, abs=1e-15)
            assert ep["margin"] == pytest.approx(s, rel=1e-15, abs=1e-15)


@pytest.mark.parametrize("objective", OBJECTIVES)
def test_p11_finite_differences_of_coef(objective):
    """coef_i = -dL/dlogp_i for every member, by central differences."""
    seg = WL.layout_pairs([(2, 3, 2, 1), (1, 2, 3)])
    rng = np.random.default_rng(40 + objective)
    logp = -rng.uniform(0.3, 4.0, size=seg.shape[0])
    for scope in (O.SCOPE_FULL, O.SCOPE_RESPONSE):
        for w_nll, lam, beta, gamma in ((1.0, 0.6, 1.7, 0.3), (0.0, 1.0, 2.5, -0.4)):
            def L(lp):
                return O.pref_epilogue(lp, seg, 2, objective, w_nll, lam, beta, gamma, scope)["loss"]
            ep = O.pref_epilogue(logp, seg, 2, objective, w_nll, lam, beta, gamma, scope)
            for i in range(len(logp)):
                e = 1e-6
                lp, lm = logp.copy(), logp.copy()
                lp[i] += e
                lm[i] -= e
                fd = (L(lp) - L(lm)) / (2 * e)
                assert -fd == pytest.approx(ep["coef"][i], rel=1e-6, abs=1e-9), (scope, i)


def test_p11_gamma_hybrid_torch_autograd():
    """The gamma-hybrid (NLL + lambda * -log sigmoid(beta (lw - lr) - gamma))
    through torch fp64 autograd, from H and W to the loss, against the oracle's
    forward, coefficients and analytic backward."""
    torch = pytest.importorskip("torch")
    spans = [(4, 6, 5, 1), (0, 3, 4), (2, 5, 5, 3)]
    wl = WL.make_custom(spans, D=16, V=29, seed=55, hidden_scale=1.5, w_std=0.4, lam=0.7)
    H, W, y, seg = wl.h64(), wl.W64(), wl.y, wl.seg
    kind, pair = seg & 3, seg >> 2
    beta, gamma, lam = 2.0, 0.25, 0.7
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    lsm = torch.log_softmax(Ht @ Wt.T, dim=1)
    lp = lsm[torch.arange(len(y)), torch.tensor(np.maximum(y, 0))] * torch.tensor(y >= 0)
    terms = []
    for b in range(len(spans)):
        C = torch.tensor((pair == b) & (kind == WL.KIND_CHOSEN))
        R = torch.tensor((pair == b) & (kind == WL.KIND_REJECTED))
        Q = torch.tensor((pair == b) & (kind == WL.KIND_PROMPT))
        lw, lr = lp[C].mean(), lp[R].mean()
        nll = -(lp[Q].sum() + lp[C].sum()) / (int(Q.sum()) + int(C.sum()))
        terms.append(nll - lam * torch.nn.functional.logsigmoid(beta * (lw - lr) - gamma))
    loss = torch.stack(terms).mean()
    loss.backward()
    logp, lse = O.forward(H, W, y)
    ep = O.pref_epilogue(logp, seg, len(spans), O.OBJ_SIGMOID, 1.0, lam, beta, gamma, O.SCOPE_FULL)
    assert ep["loss"] == pytest.approx(loss.item(), rel=1e-12)
    dh, dW = O.backward(H, W, y, lse, ep["coef"])
    np.testing.assert_allclose(dh, Ht.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-15)


# ----------------------------------------------------------------------------
# P12: the affine-quantised head ([P1] §5.1, §5.6)
# ----------------------------------------------------------------------------
def test_p12_dequantize_hand_example():
    """4-bit codes 0..7 in one word (code j at bits 4j), then 15..8 in the next;
    8-bit codes 1, 2, 3, 250 in one word; values by hand."""
    Wq = np.array([[0x76543210, 0x89ABCDEF]], np.uint32)
    W = O.dequantize(Wq, np.array([[2.0]]), np.array([[-1.0]]), 4, 16)
    assert W.tolist() == [[-1.0, 1.0, 3.0, 5.0, 7.0, 9.0, 11.0, 13.0,
                           29.0, 27.0, 25.0, 23.0, 21.0, 19.0, 17.0, 15.0]]
    Wq8 = np.array([[0xFA030201]], np.uint32)
    W8 = O.dequantize(Wq8, np.array([[0.5, 0.25]]), np.array([[1.0, -2.0]]), 8, 2)
    assert W8.tolist() == [[1.5, 2.0, -1.25, 60.5]]


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 32), (8, 64), (8, 128)])
def test_p12_dequantize_round_trip(bits, group):
    """dequantize(quantize(W)) lies within half a code step (plus the bf16
    rounding of the stored bias) of W, and reproduces the group extremes' span:
    the quantiser (input preparation) and the oracle's dequantiser agree on
    the format."""
    rng = np.random.default_rng(bits * 1000 + group)
    W = rng.standard_normal((37, 256)) * 0.05
    qh = WL.quantize_affine(W, bits, group)
    s = WL.bf16_bits_to_f32(qh.scale_bits).astype(np.float64)
    b = WL.bf16_bits_to_f32(qh.bias_bits).astype(np.float64)
    Wd = O.dequantize(qh.Wq, s, b, bits, group)
    g = np.arange(256) // group
    step = s[:, g]
    err = np.abs(Wd - W)
    # rounding to the nearest code: half a step, plus what bf16 rounding of the
    # stored scale and bias shifts (the bias by its own rounding, the scale by
    # up to 2^-8 relative times the largest code)
    tol = 0.5 * step + np.abs(b[:, g]) * 2.0 ** -8 + step * 2.0 ** -8 * ((1 << bits) - 1) + 1e-12
    assert np.all(err <= tol)
    levels = (1 << bits) - 1
    codes = np.rint((Wd - b[:, g]) / step)
    assert codes.min() >= 0 and codes.max() <= levels
    assert np.allclose(codes, (Wd - b[:, g]) / step, atol=1e-9)


# ----------------------------------------------------------------------------
# P13: bf16 rounding of the dequantised head (the quantised path's operands)
# ----------------------------------------------------------------------------
def test_p13_round_bf16_hand_values():
    """Ties go to the even significand; anything past a tie goes up; the bf16
    grid (8 significant bits) is fixed."""
    u = 2.0 ** -7                                    # one bf16 ulp at 1
    vals = np.array([1.0, 1 + u / 2, 1 + 1.5 * u, 1 + u / 2 + 2.0 ** -30, 1 + u / 2 - 2.0 ** -30,
                     -(1 + 1.5 * u), 3.0 * 2.0 ** -140 * 2 ** 20, 0.0, 255.0, 257.0, 259.0])
    want = [1.0, 1.0, 1 + 2 * u, 1 + u, 1.0, -(1 + 2 * u), 3.0 * 2.0 ** -120, 0.0, 255.0, 256.0,
            260.0]
    assert O.round_bf16(vals).tolist() == want


def test_p13_round_bf16_matches_torch_on_fp32_values():
    """On values exactly representable in fp32 the rounding equals torch's own
    fp32 -> bfloat16 conversion (round to nearest even), a library routine."""
    import torch
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # plant exact ties: the low 16 bits 0x8000 with even and odd kept parts
    xi = x.view(np.uint32).copy()
    xi[:2000] = (xi[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = xi.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


# ----------------------------------------------------------------------------
# P14: the forward-saved block maximum and the block skip ([P1] §5.1 backward
# skips)
# ----------------------------------------------------------------------------
def test_p14_block_max_brute_force():
    rng = np.random.default_rng(14)
    M, V, D, blk = 7, 23, 5, 4
    H, W = rng.standard_normal((M, D)), rng.standard_normal((V, D))
    for cap in (0.0, 1.5):
        got = O.block_max(H, W, cap, block=blk)
        assert got.shape == (6, M)
        for b in range(6):
            for i in range(M):
                best = -math.inf
                for v in range(b * blk, min(V, (b + 1) * blk)):
                    z = sum(H[i, d] * W[v, d] for d in range(D))
                    if cap:
                        z = cap * math.tanh(z / cap)
                    best = max(best, z)
                assert got[b, i] == pytest.approx(best, rel=1e-12, abs=1e-12)


def test_p14_block_max_bounds_the_lse():
    """max over blocks of block_max is the row max, so it is <= lse <= that + log V."""
    rng = np.random.default_rng(15)
    H, W = rng.standard_normal((40, 16)), rng.standard_normal((1000, 16))
    y = rng.integers(0, 1000, 40)
    _, lse = O.forward(H, W, y)
    top = O.block_max(H, W).max(axis=0)
    assert np.allclose(top, O.logits(H, W).max(axis=1), rtol=0, atol=1e-12)
    assert np.all(top <= lse + 1e-12) and np.all(lse <= top + math.log(1000) + 1e-12)


def test_p14_block_skip_equals_filter_when_eps_match():
    """Every entry of a dead block is below eps and not a target, so with
    block_eps = filter_eps the skip removes nothing the filter keeps."""
    rng = np.random.default_rng(16)
    M, V, D, blk = 20, 64, 6, 8
    H = rng.standard_normal((M, D))
    H[:, 0] = 3.0
    W = rng.standard_normal((V, D)) * 0.5
    W[16:40, 0] = -5.0                        # vocab blocks 2..4 far down for every row
    y = rng.integers(0, 16, M)
    coef = rng.standard_normal(M)
    _, lse = O.forward(H, W, y)
    eps = 1e-3
    dead = O.dead_blocks(O.block_max(H, W, block=blk), lse, y, eps, block=blk)
    assert dead.any() and not dead.all()
    a = O.backward(H, W, y, lse, coef, filter_eps=eps, block_eps=eps, block=blk)
    b = O.backward(H, W, y, lse, coef, filter_eps=eps)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_p14_block_skip_zeroes_exactly_the_dead_blocks():
    """Without the filter, the skip removes exactly the dead blocks' terms:
    dW rows of a vocab block dead for every row block are 0, and the dh
    difference equals the dead entries' contribution computed directly."""
    rng = np.random.default_rng(17)
    M, V, D, blk = 16, 32, 4, 8
    H = np.abs(rng.standard_normal((M, D))) + 1.0
    W = rng.standard_normal((V, D)) * 0.1
    W[8:16] = -4.0                             # vocab block 1 far below for every row
    y = rng.integers(16, 32, M)
    coef = rng.standard_normal(M)
    _, lse = O.forward(H, W, y)
    dead = O.dead_blocks(O.block_max(H, W, block=blk), lse, y, 1e-4, block=blk)
    assert dead[:, 1].all() and not dead[:, [0, 2, 3]].any()
    dh_s, dW_s = O.backward(H, W, y, lse, coef, block_eps=1e-4, block=blk)
    dh, dW = O.backward(H, W, y, lse, coef)
    assert np.all(dW_s[8:16] == 0.0)
    assert np.array_equal(dW_s[:8], dW[:8]) and np.array_equal(dW_s[16:], dW[16:])
    P = np.exp(O.logits(H, W[8:16]) - lse[:, None])
    assert np.allclose(dh - dh_s, (coef[:, None] * P) @ W[8:16], rtol=1e-10, atol=1e-14)
    # target inside the block keeps it alive for that row block
    y2 = y.copy()
    y2[3] = 9
    dead2 = O.dead_blocks(O.block_max(H, W, block=blk), lse, y2, 1e-4, block=blk)
    assert not dead2[0, 1] and dead2[1, 1]


# ----------------------------------------------------------------------------
# Row helpers (sampled checks at sizes where the whole oracle is too slow): each
# equals the matching rows of the whole-matrix functions above, which the pins
# above fix.  Subsets are unsorted, with a repeated index, so that an indexing
# mistake (rows of one array taken against another's order) shows.
# ----------------------------------------------------------------------------
def _helper_case(seed):
    rng = np.random.default_rng(seed)
    M, V, D = 37, 53, 9
    H = rng.standard_normal((M, D)) * 1.5
    W = rng.standard_normal((V, D)) * 0.7
    y = rng.integers(0, V, M)
    y[[4, 11]] = -1
    coef = rng.standard_normal(M)
    coef[[4, 11]] = 0.0
    rows = np.array([30, 2, 17, 4, 2, 36, 0, 11, 23])
    vrows = np.array([52, 7, 0, 31, 7, 19, int(y[5]), int(y[6])])
    return H, W, y, coef, rows, vrows


@pytest.mark.parametrize("softcap,feps", [(0.0, 0.0), (0.0, 2e-2), (1.7, 0.0), (1.7, 2e-2)])
def test_row_helpers_equal_the_whole_oracle(softcap, feps):
    H, W, y, coef, rows, vrows = _helper_case(31)
    logp, lse = O.forward(H, W, y, softcap)
    lp_r, ls_r = O.forward_rows(H, W, y, rows, softcap)
    np.testing.assert_allclose(lp_r, logp[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ls_r, lse[rows], rtol=1e-12)
    dh, dW = O.backward(H, W, y, lse, coef, filter_eps=feps, softcap=softcap)
    dh_r = O.backward_dh_rows(H, W, y, lse, coef, rows, filter_eps=feps, softcap=softcap)
    np.testing.assert_allclose(dh_r, dh[rows], rtol=1e-12, atol=1e-15)
    dW_r = O.backward_dW_rows(H, W, y, lse, coef, vrows, filter_eps=feps, softcap=softcap)
    np.testing.assert_allclose(dW_r, dW[vrows], rtol=1e-12, atol=1e-15)
    # the filter changes something in these cases (so the filtered branch is exercised)
    if feps:
        dh0, dW0 = O.backward(H, W, y, lse, coef, softcap=softcap)
        assert not np.allclose(dh0[rows], dh_r) and not np.allclose(dW0[vrows], dW_r)


# ----------------------------------------------------------------------------
# P15: the softmax part of the gradient on its own.  With every target -1 the
# gradient is G = coef * softmax (times sech^2 under a cap), which is the
# gradient of sum_i coef_i lse_i: d lse_i / d z_iv = softmax_iv.  Pinned
# against torch autograd (fp64, CPU) of that sum, written with logsumexp.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("softcap", [0.0, 2.5])
def test_p15_softmax_part_is_the_gradient_of_weighted_lse(softcap):
    import torch
    rng = np.random.default_rng(41)
    M, V, D = 13, 29, 7
    H = rng.standard_normal((M, D)) * 1.3
    W = rng.standard_normal((V, D)) * 0.8
    coef = rng.standard_normal(M)
    y = -np.ones(M, np.int64)
    _, lse = O.forward(H, W, y, softcap)
    dh, dW = O.backward(H, W, y, lse, coef, softcap=softcap)
    Ht = torch.tensor(H, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    Z = Ht @ Wt.T
    if softcap:
        Z = softcap * torch.tanh(Z / softcap)
    (torch.tensor(coef) * torch.logsumexp(Z, dim=1)).sum().backward()
    np.testing.assert_allclose(dh, Ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)
    # and the whole gradient with targets is this part minus the onehot part
    y2 = rng.integers(0, V, M)
    dh2, dW2 = O.backward(H, W, y2, lse, coef, softcap=softcap)
    sech2 = O.dcapped(H @ W.T, softcap)[np.arange(M), y2]
    onehot_dh = (coef * sech2)[:, None] * W[y2]
    onehot_dW = np.zeros_like(W)
    np.add.at(onehot_dW, y2, (coef * sech2)[:, None] * H)
    np.testing.assert_allclose(dh2, dh - onehot_dh, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW2, dW - onehot_dW, rtol=1e-11, atol=1e-14)
