"""GPU parity at the library's size limits and degenerate shapes.

M at its maximum (2^21 rows: 32-bit offset arithmetic in every kernel, 8192
row tiles, a 2 GB gradient chunk), a 2-million-entry ragged vocabulary (128
backward chunks and a ragged tail tile), D at its maximum (65536: 2048 K-slices,
32 MB operand tiles) and D = 1 (everything in the K tail).  Same gates as the
other parity tests; the oracle sees only the seeded inputs.
"""
import numpy as np
import pytest
import torch

from linear_cross_entropy_forward_amd import binding as B
from linear_cross_entropy_forward_amd import workloads as WL
from oracle import cce_oracle as O

from test_gpu_parity import check_full, run_gpu, say  # noqa: E402

pytestmark = pytest.mark.gpu

LIMITS = [
    # name, spans, D, V, targets, hidden_scale, w_std
    ("max_M", [(0, 1 << 20, 1 << 20)], 8, 300, "zipf", 2.0, 0.3),
    ("big_V", [(10, 100, 100)], 8, (1 << 21) + 77, "zipf", 2.0, 0.3),
    ("max_D", [(10, 100, 100)], 65536, 1000, "uniform", 1.0, 0.01),
    ("D_1", [(7, 150, 140, 3)], 1, 5000, "uniform", 3.0, 1.0),
]


@pytest.mark.parametrize("case", range(len(LIMITS)))
def test_limit_shapes(device, case):
    name, spans, D, V, tg, hs, ws = LIMITS[case]
    wl = WL.make_custom(spans, D=D, V=V, seed=900 + case, hidden_scale=hs, w_std=ws, targets=tg)
    assert wl.M <= 1 << 21 and D <= 65536
    say(f"[gpu] limit case {name}: M={wl.M} V={wl.V} D={wl.D}")
    g, st = run_gpu(wl, device)
    assert st == 0
    o = O.step(wl.h64(), wl.W64(), wl.y, wl.seg, wl.n_pairs, wl.lam, wl.scope)
    check_full(wl, g, o, wl.scope, tag=name)
