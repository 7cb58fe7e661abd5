"""The head's calls under HIP graph capture.

The library allocates nothing, synchronises nothing and records no memset, so
a whole step (forward, epilogue, backward) can be captured into a HIP graph
(torch.cuda.CUDAGraph drives hipGraph on ROCm) and replayed.  Every replay,
with eager work and synchronisations in between, must reproduce the eager
step byte for byte (the kernels are deterministic).
"""
import sys

import numpy as np
import pytest
import torch

from linear_cross_entropy_forward_amd import binding as B
from linear_cross_entropy_forward_amd import workloads as WL

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _capture_and_replay(step_fn, replays=3):
    eager = {k: v.detach().cpu().numpy().copy() for k, v in step_fn().items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step_fn()
    torch.cuda.synchronize()
    for r in range(replays):
        # eager work between replays: poison every output the graph writes
        for v in out.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert v.detach().cpu().numpy().tobytes() == eager[k].tobytes(), (r, k)
    return eager


def test_bf16_step_in_graph(device):
    wl = WL.make_custom([(20, 150, 140, 10)], D=128, V=17000, seed=900, w_std=0.05,
                        targets="zipf")
    say(f"[gpu] graph capture, bf16 head: M={wl.M} V={wl.V} D={wl.D}")
    head = B.Head(wl.M, wl.V, wl.D, device)
    h = B.to_device_bits(wl.h_bits, device)
    W = B.to_device_bits(wl.W_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    seg = torch.from_numpy(wl.seg).to(device)
    bm = torch.empty(B.block_max_shape(wl.M, wl.V), device=device)

    def step():
        out = B.step(head, h, W, y, seg, wl.n_pairs, wl.lam, wl.scope, 1e-6, 1e-6,
                     block_max=bm)
        out["block_max"] = bm
        return out

    head.clear_status()
    _capture_and_replay(step)
    assert head.read_status() == 0


def test_quant_step_in_graph(device):
    wl = WL.make_custom([(10, 100, 90, 8)], D=128, V=17000, seed=901, w_std=0.05)
    qh = WL.quantize_affine(WL.bf16_bits_to_f32(wl.W_bits), 4, 32)
    say(f"[gpu] graph capture, 4-bit head: M={wl.M} V={wl.V} D={wl.D}")
    head = B.Head(wl.M, wl.V, wl.D, device, quantized=True)
    h = B.to_device_bits(wl.h_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    seg = torch.from_numpy(wl.seg).to(device)
    Wq = torch.from_numpy(qh.Wq.view(np.int32)).to(device)
    s = B.to_device_bits(qh.scale_bits, device)
    b = B.to_device_bits(qh.bias_bits, device)

    def step():
        logp, lse = head.forward_q(h, Wq, s, b, 4, 32, y)
        out5, pst, coef = head.epilogue(logp, y, seg, wl.n_pairs, wl.lam, wl.scope)
        dh = head.backward_q(h, Wq, s, b, 4, 32, y, lse, coef)
        return dict(logp=logp, lse=lse, out5=out5, pair_stats=pst, coef=coef, dh=dh)

    head.clear_status()
    _capture_and_replay(step)
    assert head.read_status() == 0


def test_bf16_step_in_graph_work_queues(device):
    """8192 rows over three vocab chunks, without the skip: two pipelined
    launches take their recompute tiles from the two alternating sets of
    work-queue counters, which the launches themselves clear (no memset node
    in the graph); every replay matches the eager step byte for byte."""
    wl = WL.make_custom([(1000, 3600, 3500, 92)], D=64, V=40000, seed=902, targets="zipf")
    say(f"[gpu] graph capture, work queues: M={wl.M} V={wl.V} D={wl.D}")
    head = B.Head(wl.M, wl.V, wl.D, device)
    h = B.to_device_bits(wl.h_bits, device)
    W = B.to_device_bits(wl.W_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    seg = torch.from_numpy(wl.seg).to(device)

    def step():
        return B.step(head, h, W, y, seg, wl.n_pairs, wl.lam, wl.scope)

    head.clear_status()
    _capture_and_replay(step)
    assert head.read_status() == 0
