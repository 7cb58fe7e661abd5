"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Gates (per the head's stated tolerances): per-row logp and lse relative error
<= 1e-3 (absolute 1e-6 where |ref| < 1e-3); loss, nll and or relative <= 1e-3;
dh and dW relative L2 <= 1e-2 with the filter off; integer handling (span
counts, ignore rows, status bits) bit-exact.  The oracle only ever sees the
seeded inputs, never a value the GPU produced.
"""
import math
import sys

import numpy as np
import pytest
import torch

from linear_cross_entropy_forward_amd import binding as B
from linear_cross_entropy_forward_amd import workloads as WL
from oracle import cce_oracle as O

pytestmark = pytest.mark.gpu

RTOL_ROW = 1e-3
RTOL_SCALAR = 1e-3
RTOL_GRAD = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(wl, device):
    h = B.to_device_bits(wl.h_bits, device)
    W = B.to_device_bits(wl.W_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    seg = torch.from_numpy(wl.seg).to(device)
    return h, W, y, seg


def run_gpu(wl, device, filter_eps=0.0, block_eps=0.0, W_override=None, softcap=0.0):
    head = B.Head(wl.M, wl.V, wl.D, device)
    h, W, y, seg = upload(wl, device)
    if W_override is not None:
        W = W_override
    head.clear_status()
    out = B.step(head, h, W, y, seg, wl.n_pairs, wl.lam, wl.scope, filter_eps, block_eps,
                 softcap=softcap)
    torch.cuda.synchronize()
    status = head.read_status()
    res = {k: v.detach().cpu().numpy() for k, v in out.items()}
    del head, h, W, y, seg, out
    torch.cuda.empty_cache()
    return res, status


def rel_l2(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(np.asarray(a, np.float64) - b) / (nb if nb > 0 else 1.0)


def check_rows(got, ref, name):
    got = np.asarray(got, np.float64)
    big = np.abs(ref) >= 1e-3
    err = np.where(big, np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300), np.abs(got - ref))
    lim = np.where(big, RTOL_ROW, 1e-6)
    worst = int(np.argmax(err / lim))
    assert np.all(err <= lim), f"{name}: row {worst} got {got[worst]} ref {ref[worst]}"


def check_full(wl, g, o, scope, grads=True, tag=""):
    valid = wl.y >= 0
    check_rows(g["logp"][valid], o["logp"][valid], f"{tag} logp")
    assert np.all(g["logp"][~valid] == 0.0)
    check_rows(g["lse"], o["lse"], f"{tag} lse")
    out5 = g["out5"]
    for k, idx in (("loss", 0), ("nll", 1), ("orv", 2)):
        assert abs(out5[idx] - o[k]) <= RTOL_SCALAR * abs(o[k]), f"{tag} {k}: {out5[idx]} vs {o[k]}"
    assert abs(out5[3] - o["margin"]) <= 1e-3 * max(1.0, abs(o["margin"]))
    if np.all(np.abs(o["lw"] - o["lr"]) > 1e-4):
        assert out5[4] == pytest.approx(o["accuracy"], abs=1e-7)
    ps = g["pair_stats"]
    assert np.array_equal(ps[:, 5].astype(np.int64), o["Mw"])
    assert np.array_equal(ps[:, 6].astype(np.int64), o["Mr"])
    assert np.array_equal(ps[:, 7].astype(np.int64), o["Pm1"])
    np.testing.assert_allclose(ps[:, 0], o["lw"], rtol=RTOL_ROW)
    np.testing.assert_allclose(ps[:, 1], o["lr"], rtol=RTOL_ROW)
    kind = wl.seg & 3
    zero_rows = (kind == WL.KIND_IGNORE) | ((kind == WL.KIND_PROMPT) & (scope == WL.SCOPE_RESPONSE))
    assert np.all(g["coef"][zero_rows] == 0.0)
    nz = ~zero_rows
    np.testing.assert_allclose(g["coef"][nz], o["coef"][nz], rtol=RTOL_SCALAR)
    if grads:
        e_dh, e_dW = rel_l2(g["dh"], o["dh"]), rel_l2(g["dW"], o["dW"])
        say(f"  {tag} dh rel L2 {e_dh:.3e}  dW rel L2 {e_dW:.3e}")
        assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD
        assert np.all(g["dh"][kind == WL.KIND_IGNORE] == 0.0)


# ----------------------------------------------------------------------------
# full comparisons at sizes the oracle finishes in seconds
# ----------------------------------------------------------------------------
def test_tiny_config(device):
    wl = WL.make_workload("tiny")
    say(f"[gpu] tiny M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="tiny")
    # the fp32 inputs before bf16 rounding: gap reported, not gated
    o32 = O.step(wl.h_f32_raw.astype(np.float64), wl.W_f32_raw.astype(np.float64), wl.y, wl.seg,
                 wl.n_pairs, wl.lam, wl.scope)
    say(f"  tiny fp32-input gap: loss {abs(g['out5'][0] - o32['loss']) / abs(o32['loss']):.2e} "
        f"dh {rel_l2(g['dh'], o32['dh']):.2e}")


RAGGED = [
    # spans, D, V, targets, hidden_scale, scope   (multi-pair, all kinds)
    ([(13, 40, 37, 5), (0, 21, 19), (7, 3, 9, 2)], 200, 17000, "uniform", 1.0, WL.SCOPE_FULL),
    ([(13, 40, 37, 5), (0, 21, 19), (7, 3, 9, 2)], 200, 17000, "zipf", 1.0, WL.SCOPE_RESPONSE),
    ([(5, 30, 30, 5)], 77, 1000, "uniform", 2.0, WL.SCOPE_FULL),          # D % 8 != 0: slow loads
    ([(100, 250, 240, 10)], 128, 33000, "zipf", 1.0, WL.SCOPE_FULL),     # 3 M tiles, 3 chunks
    ([(0, 1, 1)], 8, 1, "uniform", 1.0, WL.SCOPE_FULL),                  # V = 1, M = 2
    ([(3, 2, 2, 1)] * 40, 64, 300, "uniform", 1.0, WL.SCOPE_RESPONSE),   # many pairs
    # pipelined backward (two gradient buffers), 384-row vocab tiles ragged in every chunk:
    # chunks 16384 + 15353, one partial D tile
    ([(13, 40, 37, 5), (0, 21, 19)], 96, 31737, "zipf", 1.0, WL.SCOPE_FULL),
    # 32 token tiles: 15360-wide chunk step (whole rounds of tall recompute tiles), the last
    # chunk takes the 16377-entry remainder
    ([(2047, 3072, 3072, 1)], 32, 31737, "zipf", 1.0, WL.SCOPE_FULL),
]


@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_and_edge_shapes(device, case):
    spans, D, V, tg, hs, scope = RAGGED[case]
    wl = WL.make_custom(spans, D=D, V=V, seed=100 + case, hidden_scale=hs, w_std=0.05,
                        targets=tg, lam=0.3, scope=scope)
    say(f"[gpu] ragged case {case}: M={wl.M} V={wl.V} D={wl.D} pairs={wl.n_pairs}")
    g, st = run_gpu(wl, device)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, scope)
    check_full(wl, g, o, scope, tag=f"ragged{case}")


def test_forward_many_tiles_per_workgroup(device):
    """The forward at a shape where every workgroup runs 32 vocab tiles (8192
    rows, 65613 vocab entries with a ragged tail tile, D = 64): the 256x256 tiles
    with 64-wide K-slices, against the oracle's forward on every row, and with the
    softcap; the same head at D = 96 (D % 64 != 0) takes the tall tiles."""
    for D, cap in ((64, 0.0), (64, 25.0), (96, 0.0)):
        wl = WL.make_custom([(2047, 3072, 3072, 1)], D=D, V=65613, seed=470 + D, hidden_scale=2.0,
                            w_std=0.05, targets="zipf")
        say(f"[gpu] forward, many tiles per workgroup: M={wl.M} V={wl.V} D={D} softcap={cap}")
        head = B.Head(wl.M, wl.V, wl.D, device)
        h, W, y, seg = upload(wl, device)
        head.clear_status()
        logp, lse = head.forward(h, W, y, softcap=cap)
        torch.cuda.synchronize()
        assert head.read_status() == 0
        ref_logp, ref_lse = O.forward(wl.h64(), wl.W64(), wl.y, softcap=cap)
        valid = wl.y >= 0
        check_rows(lse.cpu().numpy(), ref_lse, f"D={D} cap={cap} lse")
        check_rows(logp.cpu().numpy()[valid], ref_logp[valid], f"D={D} cap={cap} logp")
        del head, h, W, y, seg
        torch.cuda.empty_cache()


def test_small_config_full(device):
    wl = WL.make_workload("small_1b")
    say(f"[gpu] small_1b M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="small")


def test_long_config_reduced_rows_filter(device):
    """Long-context config (peaked softmax, x4 hidden) at a quarter of the rows:
    exact mode gated; filter eps=1e-6 reported against the exact oracle and
    gated against the oracle's own filtered gradient."""
    wl = WL.make_workload("long_1b", M_scale=0.25)
    say(f"[gpu] long_1b reduced M={wl.M} V={wl.V} D={wl.D}")
    H, W = wl.h64(), wl.W64()
    g, st = run_gpu(wl, device)
    assert st == 0
    o = O.step(H, W, wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="long")
    eps = wl.filter_eps
    gf, st = run_gpu(wl, device, filter_eps=eps, block_eps=eps)
    assert st == 0
    dh_f, dW_f = O.backward(H, W, wl.y, o["lse"], o["coef"], filter_eps=eps)
    e_dh, e_dW = rel_l2(gf["dh"], dh_f), rel_l2(gf["dW"], dW_f)
    say(f"  long filter eps={eps}: vs filtered oracle dh {e_dh:.3e} dW {e_dW:.3e}; "
        f"vs exact dh {rel_l2(gf['dh'], o['dh']):.3e} dW {rel_l2(gf['dW'], o['dW']):.3e}")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD


def test_block_skip_matches_filtered_oracle(device):
    """A vocab tile whose logits are far below the others is skipped; the result
    equals the oracle's filtered gradient at the same eps."""
    spans = [(10, 120, 110, 16)]
    wl = WL.make_custom(spans, D=64, V=1024, seed=7, hidden_scale=1.0, w_std=0.05, lam=0.2)
    # hidden coordinate 0 is 4 on every row and vocab rows 256..511 weigh it by
    # -4, so their logits sit near -16 while the rest stay near 0
    Hf = WL.bf16_bits_to_f32(wl.h_bits).copy()
    Hf[:, 0] = 4.0
    Wf = WL.bf16_bits_to_f32(wl.W_bits).copy()
    Wf[256:512, 0] = -4.0
    wl.h_bits = WL.f32_to_bf16_bits(Hf)
    wl.W_bits = WL.f32_to_bf16_bits(Wf)
    wl.y = np.where((wl.y >= 256) & (wl.y < 512), wl.y - 256, wl.y).astype(np.int32)
    eps = 1e-6
    say(f"[gpu] block skip M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device, filter_eps=eps, block_eps=eps)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, 1, wl.lam, wl.scope)
    dh_f, dW_f = O.backward(wl.h64(), wl.W64(), wl.y, o["lse"], o["coef"], filter_eps=eps)
    assert rel_l2(g["dh"], dh_f) <= RTOL_GRAD and rel_l2(g["dW"], dW_f) <= RTOL_GRAD
    assert np.all(g["dW"][256:512] == 0.0)           # the skipped tile contributes nothing


# ----------------------------------------------------------------------------
# status bits and determinism
# ----------------------------------------------------------------------------
def test_status_bits(device):
    wl = WL.make_custom([(2, 5, 5, 1), (1, 4, 3)], D=32, V=100, seed=3)
    # bad target on a chosen row, and a pair index beyond n_pairs
    y = wl.y.copy()
    y[3] = 100
    wl2 = WL.make_custom([(2, 5, 5, 1), (1, 4, 3)], D=32, V=100, seed=3)
    wl2.y = y
    g, st = run_gpu(wl2, device)
    assert st & B.DERR_TARGET
    seg = wl.seg.copy()
    seg[0] = (7 << 2) | WL.KIND_PROMPT
    wl3 = WL.make_custom([(2, 5, 5, 1), (1, 4, 3)], D=32, V=100, seed=3)
    wl3.seg = seg
    g, st = run_gpu(wl3, device)
    assert st & B.DERR_PAIR and not (st & B.DERR_TARGET)
    # empty rejected span
    wl4 = WL.make_custom([(2, 5, 0, 1), (1, 4, 3)], D=32, V=100, seed=3)
    g, st = run_gpu(wl4, device)
    assert st & B.DERR_EMPTY_SPAN
    assert np.all(g["coef"][wl4.seg >> 2 == 0] == 0.0)
    # y = -1 on a chosen row
    wl5 = WL.make_custom([(2, 5, 5, 1), (1, 4, 3)], D=32, V=100, seed=3)
    wl5.y = wl5.y.copy()
    wl5.y[4] = -1
    g, st = run_gpu(wl5, device)
    assert st & B.DERR_TARGET


def test_run_to_run_bytes_identical(device):
    wl = WL.make_custom([(30, 300, 280, 20)], D=256, V=20000, seed=5, targets="zipf")
    a, _ = run_gpu(wl, device)
    b, _ = run_gpu(wl, device)
    for k in ("logp", "lse", "out5", "coef", "dh", "dW"):
        assert a[k].tobytes() == b[k].tobytes(), k


# ----------------------------------------------------------------------------
# full-size configs in the benchmark's launch configuration: sampled rows,
# closed forms and invariants (the full fp64 oracle would take minutes)
# ----------------------------------------------------------------------------
def _sampled_full_size(name, device, n_rows=24, softcap=0.0):
    wl = WL.make_workload(name)
    say(f"[gpu] {name} full size M={wl.M} V={wl.V} D={wl.D} softcap={softcap}: sampled rows")
    head = B.Head(wl.M, wl.V, wl.D, device)
    h, W, y, seg = upload(wl, device)
    head.clear_status()
    logp, lse = head.forward(h, W, y, softcap=softcap)
    # backward with a seeded coefficient (an input here, drawn like the others)
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, 77]))
    coef = (rng.standard_normal(wl.M) * 1e-4).astype(np.float32)
    coef[wl.y < 0] = 0.0
    dh, dW = head.backward(h, W, y, lse, torch.from_numpy(coef).to(device), softcap=softcap)
    torch.cuda.synchronize()
    assert head.read_status() == 0
    rows = np.sort(rng.choice(wl.M, size=n_rows, replace=False))
    H64 = WL.bf16_bits_to_f32(wl.h_bits[rows]).astype(np.float64)
    W64 = wl.W64()
    lp_o, lse_o = O.forward(H64, W64, wl.y[rows], softcap)
    ok = wl.y[rows] >= 0
    check_rows(logp.cpu().numpy()[rows][ok], lp_o[ok], f"{name} logp")
    check_rows(lse.cpu().numpy()[rows], lse_o, f"{name} lse")
    dh_o = O.backward_dh_rows(H64, W64, wl.y[rows], lse_o, coef[rows].astype(np.float64),
                              np.arange(n_rows), softcap=softcap)
    dh_g = dh.cpu().numpy()[rows]
    nzr = coef[rows] != 0
    e = rel_l2(dh_g[nzr], dh_o[nzr])
    say(f"  {name} sampled dh rel L2 {e:.3e}")
    assert e <= RTOL_GRAD
    assert np.all(dh_g[~nzr] == 0.0)
    assert np.isfinite(dW.sum().item())
    del head, h, W, y, seg, logp, lse, dh, dW
    torch.cuda.empty_cache()


def test_stress_filter_sampled(device):
    """Stress config with its filter (eps 1e-5, response scope, lambda 0.5):
    sampled dh rows against the oracle's filtered gradient (gated) and against
    the exact one (reported)."""
    wl = WL.make_workload("stress")
    eps = wl.filter_eps
    say(f"[gpu] stress filter eps={eps}: sampled rows")
    head = B.Head(wl.M, wl.V, wl.D, device)
    h, W, y, seg = upload(wl, device)
    head.clear_status()
    logp, lse = head.forward(h, W, y)
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, 78]))
    coef = (rng.standard_normal(wl.M) * 1e-4).astype(np.float32)
    coef[wl.y < 0] = 0.0
    dh, dW = head.backward(h, W, y, lse, torch.from_numpy(coef).to(device), eps, eps)
    torch.cuda.synchronize()
    assert head.read_status() == 0
    rows = np.sort(rng.choice(np.nonzero(coef != 0)[0], size=16, replace=False))
    H64 = WL.bf16_bits_to_f32(wl.h_bits[rows]).astype(np.float64)
    W64 = wl.W64()
    _, lse_o = O.forward(H64, W64, wl.y[rows])
    c = coef[rows].astype(np.float64)
    dh_f = O.backward_dh_rows(H64, W64, wl.y[rows], lse_o, c, np.arange(16), filter_eps=eps)
    dh_x = O.backward_dh_rows(H64, W64, wl.y[rows], lse_o, c, np.arange(16))
    g = dh.cpu().numpy()[rows]
    e_f, e_x = rel_l2(g, dh_f), rel_l2(g, dh_x)
    say(f"  stress filter: vs filtered oracle {e_f:.3e}, vs exact {e_x:.3e}")
    assert e_f <= RTOL_GRAD
    del head, h, W, y, seg, logp, lse, dh, dW
    torch.cuda.empty_cache()


def _zero_head_full_size(name, device):
    """W = 0 at full size: lse = ln V, logp = -ln V, dh = 0 and
    dW_v = sum_i coef_i (1/V - [y_i = v]) h_i (closed form)."""
    wl = WL.make_workload(name)
    say(f"[gpu] {name} full size, W = 0 closed form")
    Wz = torch.zeros((wl.V, wl.D), dtype=torch.bfloat16, device=device)
    g, st = run_gpu(wl, device, W_override=Wz)
    assert st == 0
    lnV = math.log(wl.V)
    np.testing.assert_allclose(g["lse"], lnV, rtol=1e-6)
    valid = wl.y >= 0
    np.testing.assert_allclose(g["logp"][valid], -lnV, rtol=1e-6)
    lp = np.where(valid, -lnV, 0.0)
    o = O.epilogue(lp, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    nz = o["coef"] != 0
    np.testing.assert_allclose(g["coef"][nz], o["coef"][nz], rtol=RTOL_SCALAR)
    assert abs(g["out5"][0] - o["loss"]) <= RTOL_SCALAR * abs(o["loss"])
    assert np.all(g["dh"] == 0.0)
    H = wl.h64()
    c = o["coef"]
    ref = np.tile((c @ H) / wl.V, (wl.V, 1))
    np.subtract.at(ref, wl.y[valid], c[valid, None] * H[valid])
    e = rel_l2(g["dW"], ref)
    say(f"  {name} W=0 dW rel L2 {e:.3e}")
    assert e <= RTOL_GRAD


@pytest.mark.parametrize("name", ["gemma4b_head", "stress"])
def test_full_size_sampled(device, name):
    _sampled_full_size(name, device)


@pytest.mark.parametrize("name", ["gemma4b_head"])
def test_full_size_zero_head(device, name):
    _zero_head_full_size(name, device)


# ----------------------------------------------------------------------------
# final-logit softcap: cap * tanh(z / cap) in the forward, sech^2 in the
# backward ("Training — design …" §5.1, the e4b head; "ORPO training —
# design", lever 1 spec).  Caps are chosen so that tanh is far from linear on
# these logits (raw logit scale several times the cap in the first cases).
# ----------------------------------------------------------------------------
SOFTCAP = [
    # spans, D, V, targets, hidden_scale, w_std, cap, filter/block eps
    ([(31, 128, 128)], 256, 4096, "uniform", 3.0, 0.3, 5.0, 0.0),            # cap binds hard
    ([(5, 30, 30, 5)], 77, 1000, "uniform", 2.0, 0.4, 2.0, 0.0),             # D % 8 != 0: slow loads
    ([(100, 250, 240, 10)], 128, 33000, "zipf", 2.0, 0.2, 3.0, 0.0),         # 3 chunks, ragged V
    ([(20, 100, 90, 4), (3, 40, 50)], 192, 20000, "zipf", 4.0, 0.25, 8.0, 1e-6),  # filter + block skip
]


@pytest.mark.parametrize("case", range(len(SOFTCAP)))
def test_softcap_full(device, case):
    spans, D, V, tg, hs, ws, cap, eps = SOFTCAP[case]
    wl = WL.make_custom(spans, D=D, V=V, seed=300 + case, hidden_scale=hs, w_std=ws, targets=tg,
                        lam=0.4, scope=WL.SCOPE_FULL)
    say(f"[gpu] softcap case {case}: M={wl.M} V={wl.V} D={wl.D} cap={cap} eps={eps}")
    g, st = run_gpu(wl, device, eps, eps, softcap=cap)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope, filter_eps=eps,
               softcap=cap)
    check_full(wl, g, o, wl.scope, tag=f"softcap{case}")
    if eps == 0.0:
        # the same inputs without the cap differ clearly: the cap is really applied
        o0 = O.forward(wl.h64(), wl.W64(), wl.y)[0]
        valid = wl.y >= 0
        assert np.max(np.abs(o0[valid] - o["logp"][valid])) > 1e-2


def test_softcap_full_size_sampled(device):
    """The Gemma-4B head at full size with the pages' e4b cap of 30."""
    _sampled_full_size("gemma4b_head", device, softcap=30.0)


# ----------------------------------------------------------------------------
# preference-objective epilogue ("Training — design …" §8.3; "ORPO from-base
# on UltraFeedback — results + research directions" §6.1-6.3)
# ----------------------------------------------------------------------------
PREF = [
    # objective, nll_weight, lambda, beta, gamma, scope
    (B.OBJ_SIGMOID, 0.0, 1.0, 2.0, 0.5, WL.SCOPE_RESPONSE),   # SimPO
    (B.OBJ_SIGMOID, 1.0, 0.3, 2.5, 1.0, WL.SCOPE_FULL),       # gamma-hybrid
    (B.OBJ_IPO, 0.0, 1.0, 1.0, 0.25, WL.SCOPE_RESPONSE),      # IPO, tau = 2
    (B.OBJ_HINGE, 1.0, 0.5, 1.5, 0.2, WL.SCOPE_FULL),         # hinge + NLL
    (B.OBJ_ORPO, 0.5, 0.2, 0.0, 0.0, WL.SCOPE_FULL),          # ORPO with a half NLL weight
]


@pytest.mark.parametrize("case", range(len(PREF)))
def test_pref_epilogue_full(device, case):
    obj, w_nll, lam, beta, gamma, scope = PREF[case]
    spans = [(13, 40, 37, 5), (0, 21, 19), (7, 3, 9, 2), (4, 17, 22, 1)]
    wl = WL.make_custom(spans, D=200, V=9000, seed=400 + case, hidden_scale=1.5, w_std=0.1,
                        targets="zipf", lam=lam, scope=scope)
    say(f"[gpu] pref epilogue case {case}: objective {obj} M={wl.M} pairs={wl.n_pairs}")
    head = B.Head(wl.M, wl.V, wl.D, device)
    h, W, y, seg = upload(wl, device)
    head.clear_status()
    logp, lse = head.forward(h, W, y)
    out5, ps, coef = head.pref_epilogue(logp, y, seg, wl.n_pairs, obj, w_nll, lam, beta, gamma, scope)
    dh, dW = head.backward(h, W, y, lse, coef)
    torch.cuda.synchronize()
    assert head.read_status() == 0
    H, Wm = wl.h64(), wl.W64()
    lp_o, lse_o = O.forward(H, Wm, wl.y)
    o = O.pref_epilogue(lp_o, wl.seg, wl.n_pairs, obj, w_nll, lam, beta, gamma, scope)
    out5, ps, coef_g = out5.cpu().numpy(), ps.cpu().numpy(), coef.cpu().numpy()
    for k, idx in (("loss", 0), ("nll", 1), ("pref", 2)):
        assert abs(out5[idx] - o[k]) <= RTOL_SCALAR * max(abs(o[k]), 1e-3), (k, out5[idx], o[k])
    assert abs(out5[3] - o["margin"]) <= 1e-3 * max(1.0, abs(o["margin"]))
    if np.all(np.abs(o["lw"] - o["lr"]) > 1e-4):
        assert out5[4] == pytest.approx(o["accuracy"], abs=1e-7)
    np.testing.assert_allclose(ps[:, 2], o["s"], rtol=1e-3, atol=1e-4)
    np.testing.assert_allclose(ps[:, 4], o["pref_b"], rtol=1e-3, atol=1e-5)
    assert np.array_equal(ps[:, 5].astype(np.int64), o["Mw"])
    nz = o["coef"] != 0
    np.testing.assert_allclose(coef_g[nz], o["coef"][nz], rtol=RTOL_SCALAR)
    assert np.all(coef_g[~nz] == 0.0)
    dh_o, dW_o = O.backward(H, Wm, wl.y, lse_o, o["coef"])
    e_dh, e_dW = rel_l2(dh.cpu().numpy(), dh_o), rel_l2(dW.cpu().numpy(), dW_o)
    say(f"  pref{case} dh rel L2 {e_dh:.3e}  dW rel L2 {e_dW:.3e}")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD
    del head, h, W, y, seg, logp, lse, dh, dW
    torch.cuda.empty_cache()


def test_orpo_epilogue_is_pref_orpo(device):
    """orpo_epilogue and pref_epilogue(ORPO, nll_weight 1) give identical bytes."""
    wl = WL.make_custom([(13, 40, 37, 5), (0, 21, 19)], D=64, V=3000, seed=450, lam=0.35)
    head = B.Head(wl.M, wl.V, wl.D, device)
    h, W, y, seg = upload(wl, device)
    logp, _ = head.forward(h, W, y)
    a = head.epilogue(logp, y, seg, wl.n_pairs, wl.lam, wl.scope)
    b = head.pref_epilogue(logp, y, seg, wl.n_pairs, B.OBJ_ORPO, 1.0, wl.lam, 3.0, 1.0, wl.scope)
    torch.cuda.synchronize()
    for x, z in zip(a, b):
        assert x.cpu().numpy().tobytes() == z.cpu().numpy().tobytes()
