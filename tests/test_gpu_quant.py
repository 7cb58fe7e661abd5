"""GPU parity of the affine-quantised (frozen) head: cce_forward_q and
cce_backward_q through the C-ABI against the fp64 oracle.

The oracle's quantised head is round_bf16(dequantize(codes, scales, biases)):
the value s * q + b, taken in bf16 for the contractions.  Gates as for the bf16
head: logp / lse relative error <= 1e-3 per row, dh relative L2 <= 1e-2; the
quantised backward also equals the bf16 backward on the same (dequantised,
bf16) head up to the order of fp32 sums.
"""
import sys

import numpy as np
import pytest
import torch

from linear_cross_entropy_forward_amd import binding as B
from linear_cross_entropy_forward_amd import workloads as WL
from oracle import cce_oracle as O

pytestmark = pytest.mark.gpu

RTOL_ROW = 1e-3
RTOL_GRAD = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


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


def quant_upload(qh, device):
    Wq = torch.from_numpy(qh.Wq.view(np.int32)).to(device)
    s = B.to_device_bits(qh.scale_bits, device)
    b = B.to_device_bits(qh.bias_bits, device)
    return Wq, s, b


def oracle_head(qh, rows_per_part=16384):
    """round_bf16(dequantize(...)) of the whole head, built row block by row
    block (each row is independent) to bound the host memory."""
    s = WL.bf16_bits_to_f32(qh.scale_bits).astype(np.float64)
    b = WL.bf16_bits_to_f32(qh.bias_bits).astype(np.float64)
    V = qh.Wq.shape[0]
    return np.concatenate([
        O.round_bf16(O.dequantize(qh.Wq[v:v + rows_per_part], s[v:v + rows_per_part],
                                  b[v:v + rows_per_part], qh.bits, qh.group_size))
        for v in range(0, V, rows_per_part)])


def seeded_coef(wl, seed, scale=1e-3):
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, seed]))
    coef = (rng.standard_normal(wl.M) * scale).astype(np.float32)
    coef[wl.y < 0] = 0.0
    return coef


QUANT = [
    # spans, D, V, bits, group, softcap, filter_eps
    ([(13, 40, 37, 5), (0, 21, 19)], 256, 17000, 4, 64, 0.0, 0.0),      # 2 vocab chunks, ragged
    ([(100, 250, 240, 10)], 224, 33000, 8, 32, 0.0, 0.0),              # 3 M tiles, 3 chunks
    ([(5, 30, 30, 5)], 384, 1000, 4, 128, 30.0, 0.0),                  # softcap, one ragged chunk
    ([(7, 60, 50, 3)], 128, 16384 + 256, 8, 64, 0.0, 1e-6),            # filter; chunk + 1 tile
    ([(0, 1, 1)], 32, 1, 4, 32, 0.0, 0.0),                             # V = 1, M = 2
    ([(7, 30, 20, 3)], 32, 170001, 4, 32, 0.0, 0.0),                   # forward in 2 chunks, ragged
    ([(7, 30, 20, 3)], 64, 170001, 8, 64, 20.0, 1e-6),                 # the same with cap and filter
]


@pytest.mark.parametrize("case", range(len(QUANT)))
def test_quant_forward_backward(device, case):
    spans, D, V, bits, group, cap, feps = QUANT[case]
    wl = WL.make_custom(spans, D=D, V=V, seed=300 + case, w_std=0.05, targets="zipf")
    qh = WL.quantize_affine(WL.bf16_bits_to_f32(wl.W_bits), bits, group)
    say(f"[gpu] quant case {case}: M={wl.M} V={V} D={D} bits={bits} group={group} "
        f"softcap={cap} filter={feps}")
    Wo = oracle_head(qh)
    H = wl.h64()
    head = B.Head(wl.M, V, D, device, quantized=True)
    h = B.to_device_bits(wl.h_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    Wq, s, b = quant_upload(qh, device)
    head.clear_status()
    logp, lse = head.forward_q(h, Wq, s, b, bits, group, y, softcap=cap)
    coef = seeded_coef(wl, 400 + case)
    dh = head.backward_q(h, Wq, s, b, bits, group, y, lse, torch.from_numpy(coef).to(device),
                         filter_eps=feps, block_eps=feps, softcap=cap)
    torch.cuda.synchronize()
    assert head.read_status() == 0
    lp_o, lse_o = O.forward(H, Wo, wl.y, cap)
    ok = wl.y >= 0
    lp_g, lse_g = logp.cpu().numpy(), lse.cpu().numpy()
    check_rows(lp_g[ok], lp_o[ok], "logp")
    assert np.all(lp_g[~ok] == 0.0)
    check_rows(lse_g, lse_o, "lse")
    dh_o, _ = O.backward(H, Wo, wl.y, lse_o, coef.astype(np.float64), filter_eps=feps, softcap=cap)
    e = rel_l2(dh.cpu().numpy(), dh_o)
    say(f"  dh rel L2 {e:.3e}")
    assert e <= RTOL_GRAD
    assert np.all(dh.cpu().numpy()[~ok] == 0.0)

    # the bf16 path on the same head (uploaded as bf16) gives the same dh up to the
    # order of the fp32 sums (the frozen head's dh contraction may split K differently)
    Wb = B.to_device_bits(WL.f32_to_bf16_bits(Wo.astype(np.float32)), device)
    head_b = B.Head(wl.M, V, D, device)
    dh_b, _ = head_b.backward(h, Wb, y, lse, torch.from_numpy(coef).to(device), feps, feps,
                              softcap=cap)
    lp_b, lse_b = head_b.forward(h, Wb, y, softcap=cap)
    torch.cuda.synchronize()
    assert rel_l2(dh.cpu().numpy(), dh_b.cpu().numpy().astype(np.float64)) <= 1e-6
    # the forward folds chunks in another order: equal to rounding
    np.testing.assert_allclose(lse_b.cpu().numpy(), lse_g, rtol=1e-6, atol=1e-6)


def test_quant_target_logit_exact(device):
    """On one-hot hidden states the target logit is a single head value:
    logp + lse reproduces round_bf16(s * q + b) of the target row to fp32
    rounding, and lse matches the oracle."""
    D, V, bits, group = 64, 300, 4, 32
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=(V, D)).astype(np.uint64)
    words = np.zeros((V, D // 8), np.uint64)
    for j in range(8):
        words |= codes[:, j::8] << np.uint64(4 * j)
    s = WL.f32_to_bf16_bits(rng.uniform(0.01, 0.1, (V, D // group)).astype(np.float32))
    bb = WL.f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (V, D // group)).astype(np.float32))
    qh = WL.QuantHead(bits=bits, group_size=group, Wq=words.astype(np.uint32), scale_bits=s,
                      bias_bits=bb)
    Wo = oracle_head(qh)
    # M = D rows, row i one-hot at column i: logit (i, v) = W[v, i] exactly
    M = D
    hb = WL.f32_to_bf16_bits(np.eye(M, D, dtype=np.float32))
    yv = (np.arange(M) * 7 % V).astype(np.int32)
    head = B.Head(M, V, D, device, quantized=True)
    h = B.to_device_bits(hb, device)
    y = torch.from_numpy(yv).to(device)
    Wq, sd, bd = quant_upload(qh, device)
    logp, lse = head.forward_q(h, Wq, sd, bd, bits, group, y)
    torch.cuda.synchronize()
    assert head.read_status() == 0
    # the target logit is logp + lse; compare it with W[y_i, i] (fp32 sums of exact values)
    z = (logp.cpu().numpy().astype(np.float64) + lse.cpu().numpy())
    np.testing.assert_allclose(z, Wo[yv, np.arange(M)], rtol=0, atol=2e-6)
    lp_o, lse_o = O.forward(np.eye(M, D), Wo, yv)
    check_rows(lse.cpu().numpy(), lse_o, "lse")


def test_quant_gemma_head_sampled(device):
    """The 4-bit head (group 64) at the Gemma-4B head's M = 8192 and D = 2560,
    with V = 65536: every launch is per 16384-entry vocab chunk and the same as
    at V = 262144 (there are four chunks instead of sixteen), which keeps the
    host-side quantisation and the oracle's dequantisation within seconds.
    Sampled rows against the oracle."""
    wl = WL.make_workload("gemma4b_head", V=65536)
    say(f"[gpu] quant gemma4b_head M={wl.M} V={wl.V} D={wl.D}: quantising the head on the host")
    qh = WL.quantize_affine(WL.bf16_bits_to_f32(wl.W_bits), 4, 64)
    head = B.Head(wl.M, wl.V, wl.D, device, quantized=True)
    h = B.to_device_bits(wl.h_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    Wq, s, b = quant_upload(qh, device)
    head.clear_status()
    logp, lse = head.forward_q(h, Wq, s, b, 4, 64, y)
    coef = seeded_coef(wl, 78, 1e-4)
    dh = head.backward_q(h, Wq, s, b, 4, 64, y, lse, torch.from_numpy(coef).to(device))
    torch.cuda.synchronize()
    assert head.read_status() == 0
    rng = np.random.default_rng(np.random.SeedSequence([WL.BASE_SEED, 79]))
    rows = np.sort(rng.choice(wl.M, size=16, replace=False))
    Wo = oracle_head(qh)
    H64 = WL.bf16_bits_to_f32(wl.h_bits[rows]).astype(np.float64)
    lp_o, lse_o = O.forward(H64, Wo, wl.y[rows])
    ok = wl.y[rows] >= 0
    check_rows(logp.cpu().numpy()[rows][ok], lp_o[ok], "gemma quant logp")
    check_rows(lse.cpu().numpy()[rows], lse_o, "gemma quant lse")
    dh_o = O.backward_dh_rows(H64, Wo, wl.y[rows], lse_o, coef[rows].astype(np.float64),
                              np.arange(len(rows)))
    dh_g = dh.cpu().numpy()[rows]
    nz = coef[rows] != 0
    e = rel_l2(dh_g[nz], dh_o[nz])
    say(f"  sampled dh rel L2 {e:.3e}")
    assert e <= RTOL_GRAD


def test_quant_workspace_reuse(device):
    """The quantised forward dequantises into the backward's buffers: one head
    (one workspace) running forward and backward on one head and input, then
    on another, gives byte-identical results on the second to a fresh
    head's.  Two forward chunks and more than ten backward chunks."""
    D, V, bits, group = 64, 170001, 4, 32
    spans = [(7, 30, 20, 3)]

    def run(head, seed):
        wl = WL.make_custom(spans, D=D, V=V, seed=seed, w_std=0.05, targets="zipf")
        qh = WL.quantize_affine(WL.bf16_bits_to_f32(wl.W_bits), bits, group)
        h = B.to_device_bits(wl.h_bits, device)
        y = torch.from_numpy(wl.y).to(device)
        Wq, s, b = quant_upload(qh, device)
        head.clear_status()
        logp, lse = head.forward_q(h, Wq, s, b, bits, group, y)
        coef = torch.from_numpy(seeded_coef(wl, seed + 1)).to(device)
        dh = head.backward_q(h, Wq, s, b, bits, group, y, lse, coef)
        torch.cuda.synchronize()
        assert head.read_status() == 0
        return [t.cpu().numpy().tobytes() for t in (logp, lse, dh)]

    M = sum(sum(sp) for sp in spans)
    shared = B.Head(M, V, D, device, quantized=True)
    run(shared, 900)
    second = run(shared, 901)
    fresh = run(B.Head(M, V, D, device, quantized=True), 901)
    assert second == fresh
