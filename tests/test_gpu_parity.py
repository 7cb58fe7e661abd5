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


def soft_coef(wl):
    """Seeded per-row coefficients for the softmax-only backward (an input drawn
    like the others, nonzero on every row)."""
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, 500, wl.M, wl.V, wl.D]))
    return (rng.standard_normal(wl.M) * 1e-3).astype(np.float32)


def run_gpu(wl, device, filter_eps=0.0, block_eps=0.0, W_override=None, softcap=0.0, soft=False):
    """One step through the C-ABI.  soft: also the backward with every target
    -1 and the seeded soft_coef(wl) (same lse), whose gradient is the softmax
    part alone, coef * softmax: returned as dh_s, dW_s."""
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
    if soft:
        y_neg = torch.full_like(y, -1)
        cs = torch.from_numpy(soft_coef(wl)).to(device)
        dh_s, dW_s = head.backward(h, W, y_neg, out["lse"], cs, filter_eps, block_eps,
                                   softcap=softcap)
        torch.cuda.synchronize()
        status |= head.read_status()
        res["dh_s"], res["dW_s"] = dh_s.cpu().numpy(), dW_s.cpu().numpy()
        del dh_s, dW_s, y_neg, cs
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


def check_full(wl, g, o, scope, grads=True, tag="", filtered=False, capped=False):
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
        if not filtered and not capped:
            # P6: each row's softmax sums to its onehot, so sum_v dW[v, :] = 0; the test
            # scale is the size of sum_i coef_i h_i (the onehot part summed over v).  Each
            # dW entry is an fp32 sum over the M rows (MFMA accumulation), whose rounding
            # error is typically 2^-24 sqrt(M) of the entry; summed over V rows that allows
            # 2^-24 sqrt(M V) |dW| on top (it matters only where M is huge and dW's rows are
            # far larger than their sum: the 2^21-row limit case)
            scale = np.linalg.norm(o["coef"] @ wl.h64())
            acc_err = 2.0 ** -24 * math.sqrt(wl.M * wl.V) * np.linalg.norm(o["dW"])
            e_sum = np.linalg.norm(g["dW"].astype(np.float64).sum(axis=0))
            say(f"  {tag} |sum_v dW| / |sum_i coef_i h_i| {e_sum / max(scale, 1e-300):.3e} "
                f"(fp32 accumulation allowance {acc_err / max(scale, 1e-300):.3e})")
            assert e_sum <= RTOL_GRAD * scale + acc_err


def check_softmax_part(wl, g, lse_o, tag, filter_eps=0.0, block_eps=0.0, softcap=0.0,
                       H=None, W=None):
    """The softmax-only backward (every target -1, seeded coefficients) against the
    oracle's at rel L2 <= 1e-2: with no onehot term the whole gradient is
    coef * softmax, so a dropped, misplaced or mis-normalised softmax entry shows
    at full weight."""
    H = wl.h64() if H is None else H
    W = wl.W64() if W is None else W
    y_neg = -np.ones(wl.M, np.int64)
    dh_o, dW_o = O.backward(H, W, y_neg, lse_o, soft_coef(wl).astype(np.float64), filter_eps,
                            softcap, block_eps)
    e_dh, e_dW = rel_l2(g["dh_s"], dh_o), rel_l2(g["dW_s"], dW_o)
    say(f"  {tag} softmax-only backward: dh rel L2 {e_dh:.3e}  dW rel L2 {e_dW:.3e}")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD


def softmax_share_gate(wl, g, o, tag, softcap=0.0):
    """Where the softmax part is a large share of the gradient (peaked logits):
    the with-target gradient's error measured against the size of the oracle's
    softmax part alone, |G - O| <= 1e-2 |O + onehot part|."""
    H, W = wl.h64(), wl.W64()
    ok = wl.y >= 0
    yy = np.where(ok, wl.y, 0)
    t = o["coef"] * ok
    if softcap:
        zt = np.einsum("ij,ij->i", H, W[yy])
        t = t * (1.0 - np.tanh(zt / softcap) ** 2)
    on_dh = t[:, None] * W[yy]
    on_dW = np.zeros_like(W)
    np.add.at(on_dW, yy[ok], t[ok, None] * H[ok])
    soft_dh, soft_dW = o["dh"] + on_dh, o["dW"] + on_dW
    share_dh = np.linalg.norm(soft_dh) / np.linalg.norm(o["dh"])
    share_dW = np.linalg.norm(soft_dW) / np.linalg.norm(o["dW"])
    e_dh = np.linalg.norm(g["dh"] - o["dh"]) / np.linalg.norm(soft_dh)
    e_dW = np.linalg.norm(g["dW"] - o["dW"]) / np.linalg.norm(soft_dW)
    say(f"  {tag} softmax share dh {share_dh:.3f} dW {share_dW:.3f}; error / softmax part: "
        f"dh {e_dh:.3e} dW {e_dW:.3e}")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD
    return share_dh, share_dW


# ----------------------------------------------------------------------------
# full comparisons at sizes the oracle finishes in seconds
# ----------------------------------------------------------------------------
def test_tiny_config(device):
    wl = WL.make_workload("tiny")
    say(f"[gpu] tiny M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device, soft=True)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="tiny")
    check_softmax_part(wl, g, o["lse"], "tiny")
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
    g, st = run_gpu(wl, device, soft=True)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, scope)
    check_full(wl, g, o, scope, tag=f"ragged{case}")
    check_softmax_part(wl, g, o["lse"], f"ragged{case}")


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
    g, st = run_gpu(wl, device, soft=True)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="small")
    check_softmax_part(wl, g, o["lse"], "small")


def report(kind, **fields):
    """Deviation figures for the repository's profile tables: appended as one
    JSON line to the file named by CCE_REPORT when it is set (they are also
    printed)."""
    import json
    import os
    path = os.environ.get("CCE_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(kind=kind, **fields)) + "\n")


def test_long_config_full_filter(device):
    """Long-context config (x4 hidden: a peaked softmax) at all 5119 rows: exact
    mode gated, including the softmax part at its own scale; the filter at eps
    1e-6 (with the block skip at the same eps) gated against the oracle's own
    filtered gradient and reported against the exact one."""
    wl = WL.make_workload("long_1b")
    say(f"[gpu] long_1b M={wl.M} V={wl.V} D={wl.D}")
    H, W = wl.h64(), wl.W64()
    g, st = run_gpu(wl, device, soft=True)
    assert st == 0
    o = O.step(H, W, wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="long")
    check_softmax_part(wl, g, o["lse"], "long", H=H, W=W)
    softmax_share_gate(wl, g, o, "long")
    eps = wl.filter_eps
    gf, st = run_gpu(wl, device, filter_eps=eps, block_eps=eps, soft=True)
    assert st == 0
    dh_f, dW_f = O.backward(H, W, wl.y, o["lse"], o["coef"], filter_eps=eps)
    e_dh, e_dW = rel_l2(gf["dh"], dh_f), rel_l2(gf["dW"], dW_f)
    x_dh, x_dW = rel_l2(gf["dh"], o["dh"]), rel_l2(gf["dW"], o["dW"])
    o_dh, o_dW = rel_l2(dh_f, o["dh"]), rel_l2(dW_f, o["dW"])
    say(f"  long filter eps={eps}: vs filtered oracle dh {e_dh:.3e} dW {e_dW:.3e}; "
        f"vs exact dh {x_dh:.3e} dW {x_dW:.3e} (filtered oracle vs exact: {o_dh:.3e} / {o_dW:.3e})")
    report("filter_deviation", workload="long_1b", rows="all 5119", eps=eps,
           gpu_vs_filtered_dh=e_dh, gpu_vs_filtered_dW=e_dW, gpu_vs_exact_dh=x_dh,
           gpu_vs_exact_dW=x_dW, filtered_oracle_vs_exact_dh=o_dh, filtered_oracle_vs_exact_dW=o_dW)
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD
    check_softmax_part(wl, gf, o["lse"], "long filtered", filter_eps=eps, block_eps=eps, H=H, W=W)


def test_peaked_pipelined_8192_rows(device):
    """8192 rows (32 token tiles: the 15360-wide chunk step of the pipelined
    backward, its fused launch and the last chunk's contractions alone) with a
    peaked softmax (hidden x4, head std 0.08, logit std about 3.6), where the
    softmax part is about a third of dh and a quarter of dW: the whole gradient
    is gated at the scale of its softmax part, as well as the softmax-only
    backward."""
    wl = WL.make_custom([(2047, 3072, 3072, 1)], D=128, V=31737, seed=480, hidden_scale=4.0,
                        w_std=0.08, targets="zipf", lam=0.3)
    say(f"[gpu] peaked pipelined M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device, soft=True)
    assert st == 0
    H, W = wl.h64(), wl.W64()
    o = O.step(H, W, wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag="peaked8192")
    check_softmax_part(wl, g, o["lse"], "peaked8192", H=H, W=W)
    sh_dh, sh_dW = softmax_share_gate(wl, g, o, "peaked8192")
    assert sh_dh >= 0.2 and sh_dW >= 0.2


def test_block_skip_past_64_token_blocks(device):
    """Block skip with more than 64 token blocks in the dW contraction's K
    (17100 rows: 67 blocks), the path that streams every K slice and branches
    around the skipped blocks' MFMAs; against the oracle's filtered gradient,
    and a vocab tile dead for every row block contributes nothing."""
    spans = [(1000, 8000, 7900, 200)]
    wl = WL.make_custom(spans, D=64, V=1024, seed=8, hidden_scale=1.0, w_std=0.05, lam=0.2)
    Hf = WL.bf16_bits_to_f32(wl.h_bits).copy()
    Hf[:, 0] = 4.0
    Wf = WL.bf16_bits_to_f32(wl.W_bits).copy()
    Wf[256:768, 0] = -4.0
    # vocab tiles 1 and 2 sit near -16; token block 3 (rows 768..1023) is lifted on
    # tile 2 (to about -4), so that tile is live for that block only: a mixed
    # K-block mask in tile 2's dW contraction
    Hf[768:1024, 1] = 8.0
    Wf[512:768, 1] = 1.5
    wl.h_bits = WL.f32_to_bf16_bits(Hf)
    wl.W_bits = WL.f32_to_bf16_bits(Wf)
    wl.y = np.where((wl.y >= 256) & (wl.y < 768), wl.y % 256, wl.y).astype(np.int32)
    eps = 1e-6
    say(f"[gpu] block skip, {wl.M} rows ({(wl.M + 255) // 256} token blocks), V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device, filter_eps=eps, block_eps=eps)
    assert st == 0
    H, W = wl.h64(), wl.W64()
    o = O.step(H, W, wl.y, wl.seg, 1, wl.lam, wl.scope)
    dead = O.dead_blocks(O.block_max(H, W), o["lse"], wl.y, eps)
    assert dead[:, 1].all() and dead[:, 2].any() and not dead[:, 2].all()
    dh_f, dW_f = O.backward(H, W, wl.y, o["lse"], o["coef"], filter_eps=eps, block_eps=eps)
    e_dh, e_dW = rel_l2(g["dh"], dh_f), rel_l2(g["dW"], dW_f)
    say(f"  vs the oracle's block-skip gradient: dh {e_dh:.3e} dW {e_dW:.3e}")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD
    assert np.all(g["dW"][256:512] == 0.0)


def test_block_skip_block_live_in_one_half(device):
    """A 256-entry vocab block that a 384-row recompute tile boundary cuts in
    two (block 1: rows 256..383 in the first tall tile, 384..511 in the
    second), live for token block 0 through its upper half only: the block's
    flag combines both tiles' votes, so it must stay live there (its entries
    reach the gradient) and be skipped for the other token blocks; against the
    oracle's block-skip gradient."""
    spans = [(100, 300, 290, 30)]
    wl = WL.make_custom(spans, D=64, V=1024, seed=9, hidden_scale=1.0, w_std=0.05, lam=0.2)
    Hf = WL.bf16_bits_to_f32(wl.h_bits).copy()
    Hf[:, 0] = 4.0
    Wf = WL.bf16_bits_to_f32(wl.W_bits).copy()
    Wf[256:512, 0] = -4.0            # block 1 near -16 on every row
    Hf[0:256, 1] = 8.0
    Wf[400:512, 1] = 1.5             # ... lifted to about -4 for token block 0, upper half only
    wl.h_bits = WL.f32_to_bf16_bits(Hf)
    wl.W_bits = WL.f32_to_bf16_bits(Wf)
    wl.y = np.where((wl.y >= 256) & (wl.y < 512), wl.y % 256, wl.y).astype(np.int32)
    eps = 1e-6
    say(f"[gpu] block skip, block live in one half: M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device, filter_eps=eps, block_eps=eps)
    assert st == 0
    H, W = wl.h64(), wl.W64()
    o = O.step(H, W, wl.y, wl.seg, 1, wl.lam, wl.scope)
    dead = O.dead_blocks(O.block_max(H, W), o["lse"], wl.y, eps)
    assert not dead[0, 1] and dead[1:, 1].all()
    dh_f, dW_f = O.backward(H, W, wl.y, o["lse"], o["coef"], filter_eps=eps, block_eps=eps)
    e_dh, e_dW = rel_l2(g["dh"], dh_f), rel_l2(g["dW"], dW_f)
    e_half = rel_l2(g["dW"][400:512], dW_f[400:512])
    say(f"  vs the oracle's block-skip gradient: dh {e_dh:.3e} dW {e_dW:.3e} "
        f"(rows 400..511: {e_half:.3e})")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD and e_half <= RTOL_GRAD
    assert np.abs(dW_f[400:512]).max() > 0.0
    assert np.all(g["dW"][256:400] == 0.0)           # filtered or skipped everywhere


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


@pytest.mark.parametrize("eps", [0.0, 1e-5])
def test_run_to_run_bytes_identical_work_queue(device, eps):
    """8192 rows (32 token tiles) over three vocab chunks: each pipelined
    launch hands 1280 recompute tiles to at most 256 workers through the
    per-XCD queues, so which workgroup computes which tile changes from run to
    run (stealing included); every output is still byte-identical, with and
    without the filter and block skip."""
    wl = WL.make_custom([(1000, 3600, 3500, 92)], D=64, V=40000, seed=6, targets="zipf",
                        hidden_scale=3.0)
    assert wl.M == 8192
    a, _ = run_gpu(wl, device, filter_eps=eps, block_eps=eps)
    b, _ = run_gpu(wl, device, filter_eps=eps, block_eps=eps)
    for k in ("logp", "lse", "out5", "coef", "dh", "dW"):
        assert a[k].tobytes() == b[k].tobytes(), k


def test_workspace_reuse_leaves_nothing_behind(device):
    """One head (one workspace) runs a step on one input and then on another:
    the second step's outputs are byte-identical to a fresh head's on that
    input (gradient buffers, block flags and work-queue counters are all
    rewritten or cleared by the step that uses them), with the block skip on
    and a first input whose vocab rows 10000..19999 are dead for every row."""
    eps = 1e-5
    wa = WL.make_custom([(1000, 3600, 3500, 92)], D=64, V=40000, seed=11, targets="zipf")
    wb = WL.make_custom([(1000, 3600, 3500, 92)], D=64, V=40000, seed=12, targets="zipf")
    # the first input: vocab rows 10000..19999 sink to about -16 on every row
    Hf = WL.bf16_bits_to_f32(wa.h_bits).copy()
    Hf[:, 0] = 4.0
    Wf = WL.bf16_bits_to_f32(wa.W_bits).copy()
    Wf[10000:20000, 0] = -4.0
    wa.h_bits = WL.f32_to_bf16_bits(Hf)
    wa.W_bits = WL.f32_to_bf16_bits(Wf)
    wa.y = np.where((wa.y >= 10000) & (wa.y < 20000), wa.y - 10000, wa.y).astype(np.int32)
    head = B.Head(wa.M, wa.V, wa.D, device)
    outs = []
    for wl in (wa, wb):
        h, W, y, seg = upload(wl, device)
        head.clear_status()
        out = B.step(head, h, W, y, seg, wl.n_pairs, wl.lam, wl.scope, eps, eps)
        torch.cuda.synchronize()
        assert head.read_status() == 0
        outs.append({k: v.detach().cpu().numpy() for k, v in out.items()})
    del head
    torch.cuda.empty_cache()
    fresh, st = run_gpu(wb, device, filter_eps=eps, block_eps=eps)
    assert st == 0
    for k in ("logp", "lse", "out5", "coef", "dh", "dW"):
        assert outs[1][k].tobytes() == fresh[k].tobytes(), k


# ----------------------------------------------------------------------------
# full-size configs in the benchmark's launch configuration: the oracle's
# forward and epilogue over every row (seconds to a minute of fp64 on the host
# cores), sampled dh rows and sampled dW vocab rows (each needs only its own
# logits), the softmax-only backward on the same samples, and closed forms
# ----------------------------------------------------------------------------
def _pick_vocab_rows(wl, n=64):
    """n vocab rows spread over the backward's chunks: the 16 most frequent
    targets (onehot-dominated rows) and rows drawn uniformly (nearly all of
    them nobody's target, i.e. pure softmax rows)."""
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, 601, wl.M, wl.V]))
    ids, cnt = np.unique(wl.y[wl.y >= 0], return_counts=True)
    top = ids[np.argsort(-cnt, kind="stable")[:16]]
    rest = rng.choice(np.setdiff1d(np.arange(wl.V), top), size=n - len(top), replace=False)
    return np.sort(np.concatenate([top, rest]))


def _full_size_against_oracle(name, device, softcap=0.0, filter_report=False):
    wl = WL.make_workload(name)
    say(f"[gpu] {name} full size M={wl.M} V={wl.V} D={wl.D} softcap={softcap}")
    head = B.Head(wl.M, wl.V, wl.D, device)
    h, W, y, seg = upload(wl, device)
    head.clear_status()
    out = B.step(head, h, W, y, seg, wl.n_pairs, wl.lam, wl.scope, softcap=softcap)
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, 77, wl.M]))
    rows = np.sort(rng.choice(wl.M, size=24, replace=False))
    vrows = _pick_vocab_rows(wl)
    rows_t, vrows_t = torch.from_numpy(rows).to(device), torch.from_numpy(vrows).to(device)
    g = {k: out[k].cpu().numpy() for k in ("logp", "lse", "out5", "pair_stats", "coef")}
    g["dh"], g["dW"] = out["dh"][rows_t].cpu().numpy(), out["dW"][vrows_t].cpu().numpy()
    lse_t = out["lse"]
    del out
    torch.cuda.empty_cache()
    cs = soft_coef(wl)
    dh_s, dW_s = head.backward(h, W, torch.full_like(y, -1), lse_t, torch.from_numpy(cs).to(device),
                               softcap=softcap)
    g["dh_s"], g["dW_s"] = dh_s[rows_t].cpu().numpy(), dW_s[vrows_t].cpu().numpy()
    del dh_s, dW_s
    torch.cuda.empty_cache()
    if filter_report:
        eps = wl.filter_eps
        dh_f, dW_f = head.backward(h, W, y, lse_t, torch.from_numpy(g["coef"]).to(device), eps, eps,
                                   softcap=softcap)
        g["dh_f"], g["dW_f"] = dh_f[rows_t].cpu().numpy(), dW_f[vrows_t].cpu().numpy()
        del dh_f, dW_f
    torch.cuda.synchronize()
    assert head.read_status() == 0
    del head, h, W, y, seg, lse_t
    torch.cuda.empty_cache()

    H, Wm = wl.h64(), wl.W64()
    logp_o, lse_o = O.forward(H, Wm, wl.y, softcap)
    valid = wl.y >= 0
    check_rows(g["logp"][valid], logp_o[valid], f"{name} logp (every row)")
    check_rows(g["lse"], lse_o, f"{name} lse (every row)")
    o = O.epilogue(logp_o, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    out5 = g["out5"]
    for k, idx in (("loss", 0), ("nll", 1), ("orv", 2)):
        assert abs(out5[idx] - o[k]) <= RTOL_SCALAR * abs(o[k]), f"{name} {k}: {out5[idx]} vs {o[k]}"
    assert abs(out5[3] - o["margin"]) <= 1e-3 * max(1.0, abs(o["margin"]))
    ps = g["pair_stats"]
    assert np.array_equal(ps[:, 5].astype(np.int64), o["Mw"])
    assert np.array_equal(ps[:, 6].astype(np.int64), o["Mr"])
    assert np.array_equal(ps[:, 7].astype(np.int64), o["Pm1"])
    np.testing.assert_allclose(ps[:, 0], o["lw"], rtol=RTOL_ROW)
    np.testing.assert_allclose(ps[:, 1], o["lr"], rtol=RTOL_ROW)
    nz = o["coef"] != 0
    assert np.all(g["coef"][~nz] == 0.0)
    np.testing.assert_allclose(g["coef"][nz], o["coef"][nz], rtol=RTOL_SCALAR)
    say(f"  {name}: logp / lse of every row, loss {out5[0]:.6f} (oracle {o['loss']:.6f}), "
        f"pair stats and every coef match")
    coef_o = o["coef"]
    dh_o = O.backward_dh_rows(H, Wm, wl.y, lse_o, coef_o, rows, softcap=softcap)
    dW_o = O.backward_dW_rows(H, Wm, wl.y, lse_o, coef_o, vrows, softcap=softcap)
    e_dh = rel_l2(g["dh"][nz[rows]], dh_o[nz[rows]])
    e_dW = rel_l2(g["dW"], dW_o)
    soft_rows = ~np.isin(vrows, wl.y)
    e_dWs = rel_l2(g["dW"][soft_rows], dW_o[soft_rows])
    say(f"  {name} sampled dh rel L2 {e_dh:.3e}; {len(vrows)} dW rows {e_dW:.3e} "
        f"({int(soft_rows.sum())} of them nobody's target: {e_dWs:.3e})")
    assert e_dh <= RTOL_GRAD and e_dW <= RTOL_GRAD and e_dWs <= RTOL_GRAD
    assert np.all(g["dh"][~nz[rows]] == 0.0)
    y_neg = -np.ones(wl.M, np.int64)
    c64 = cs.astype(np.float64)
    dh_so = O.backward_dh_rows(H, Wm, y_neg, lse_o, c64, rows, softcap=softcap)
    dW_so = O.backward_dW_rows(H, Wm, y_neg, lse_o, c64, vrows, softcap=softcap)
    e1, e2 = rel_l2(g["dh_s"], dh_so), rel_l2(g["dW_s"], dW_so)
    say(f"  {name} softmax-only backward: sampled dh {e1:.3e}, dW {e2:.3e}")
    assert e1 <= RTOL_GRAD and e2 <= RTOL_GRAD
    if filter_report:
        eps = wl.filter_eps
        dh_fo = O.backward_dh_rows(H, Wm, wl.y, lse_o, coef_o, rows, filter_eps=eps, softcap=softcap)
        dW_fo = O.backward_dW_rows(H, Wm, wl.y, lse_o, coef_o, vrows, filter_eps=eps,
                                   softcap=softcap)
        r = rows[nz[rows]]
        k = nz[rows]
        f_dh, f_dW = rel_l2(g["dh_f"][k], dh_fo[k]), rel_l2(g["dW_f"], dW_fo)
        x_dh, x_dW = rel_l2(g["dh_f"][k], dh_o[k]), rel_l2(g["dW_f"], dW_o)
        o_dh, o_dW = rel_l2(dh_fo[k], dh_o[k]), rel_l2(dW_fo, dW_o)
        say(f"  {name} filter eps={eps}: vs filtered oracle dh {f_dh:.3e} dW {f_dW:.3e}; vs exact "
            f"dh {x_dh:.3e} dW {x_dW:.3e} (filtered oracle vs exact {o_dh:.3e} / {o_dW:.3e})")
        report("filter_deviation", workload=name, rows=f"{len(r)} sampled dh rows, {len(vrows)} "
               f"sampled dW rows", eps=eps, gpu_vs_filtered_dh=f_dh, gpu_vs_filtered_dW=f_dW,
               gpu_vs_exact_dh=x_dh, gpu_vs_exact_dW=x_dW, filtered_oracle_vs_exact_dh=o_dh,
               filtered_oracle_vs_exact_dW=o_dW)
        assert f_dh <= RTOL_GRAD and f_dW <= RTOL_GRAD


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gemma4b_head", "stress"])
def test_full_size_against_oracle(device, name):
    _full_size_against_oracle(name, device, filter_report=(name == "stress"))


def _zero_head_full_size(name, device):
    """W = 0 at full size: lse = ln V, logp = -ln V, dh = 0 and
    dW_v = sum_i coef_i (1/V - [y_i = v]) h_i (closed form), with the uniform
    part (every row nobody targets: (sum_i coef_i h_i) / V) gated on its own."""
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
    u = (c @ H) / wl.V                                   # every row's uniform part
    tg = np.unique(wl.y[valid])
    ref_t = np.tile(u, (len(tg), 1))
    pos = np.searchsorted(tg, wl.y[valid])
    np.subtract.at(ref_t, pos, c[valid, None] * H[valid])
    # |dW - ref|^2 and |ref|^2 summed chunk by chunk over the non-target rows, then the targets
    others = np.ones(wl.V, bool)
    others[tg] = False
    err2 = ref2 = 0.0
    dW = g["dW"]
    for v0 in range(0, wl.V, 16384):
        sel = others[v0:v0 + 16384]
        d = dW[v0:v0 + 16384][sel].astype(np.float64) - u
        err2 += float((d * d).sum())
        ref2 += float(sel.sum()) * float(u @ u)
    e_u = math.sqrt(err2 / ref2)
    d = dW[tg].astype(np.float64) - ref_t
    e = math.sqrt((err2 + float((d * d).sum())) / (ref2 + float((ref_t * ref_t).sum())))
    say(f"  {name} W=0 dW rel L2 {e:.3e}; uniform part alone (rows nobody targets) {e_u:.3e}")
    assert e <= RTOL_GRAD and e_u <= RTOL_GRAD


@pytest.mark.parametrize("name", ["gemma4b_head", "stress", "long_1b"])
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
    g, st = run_gpu(wl, device, eps, eps, softcap=cap, soft=True)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope, filter_eps=eps,
               softcap=cap)
    check_full(wl, g, o, wl.scope, tag=f"softcap{case}", filtered=eps > 0, capped=True)
    check_softmax_part(wl, g, o["lse"], f"softcap{case}", filter_eps=eps, block_eps=eps,
                       softcap=cap)
    if eps == 0.0:
        # the same inputs without the cap differ clearly: the cap is really applied
        o0 = O.forward(wl.h64(), wl.W64(), wl.y)[0]
        valid = wl.y >= 0
        assert np.max(np.abs(o0[valid] - o["logp"][valid])) > 1e-2


@pytest.mark.timeout(900)
def test_softcap_full_size_against_oracle(device):
    """The Gemma-4B head at full size with the pages' e4b cap of 30."""
    _full_size_against_oracle("gemma4b_head", device, softcap=30.0)


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
