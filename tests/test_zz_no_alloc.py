"""The no-allocation forward (cce_forward_noalloc, scratch in the library's
fixed device array) against cce_forward (workspace from the caller): the same
kernels, so logp, lse, block_max and the status word must be byte-identical.
Two calls in a row on one stream, the second smaller than the first (the
array keeps the first call's contents), plus a call with the cap and the block
maximum, and a third call back at the first size."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_forward_amd import binding as B
from linear_cross_entropy_forward_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _compare(wl, device, softcap=0.0, with_bm=False):
    h = B.to_device_bits(wl.h_bits, device)
    W = B.to_device_bits(wl.W_bits, device)
    y = torch.from_numpy(wl.y).to(device)
    head = B.Head(wl.M, wl.V, wl.D, device)
    bm_a = torch.empty(B.block_max_shape(wl.M, wl.V), device=device) if with_bm else None
    bm_b = torch.empty_like(bm_a) if with_bm else None
    head.clear_status()
    lp_a, ls_a = head.forward(h, W, y, softcap=softcap, block_max=bm_a)
    st = torch.zeros(1, dtype=torch.int32, device=device)
    lp_b, ls_b = B.forward_noalloc(h, W, y, st, softcap=softcap, block_max=bm_b)
    torch.cuda.synchronize()
    assert head.read_status() == 0 and int(st.item()) == 0
    assert lp_a.cpu().numpy().tobytes() == lp_b.cpu().numpy().tobytes()
    assert ls_a.cpu().numpy().tobytes() == ls_b.cpu().numpy().tobytes()
    if with_bm:
        assert bm_a.cpu().numpy().tobytes() == bm_b.cpu().numpy().tobytes()
    # sanity: the outputs are log-probabilities
    valid = wl.y >= 0
    assert np.all(lp_b.cpu().numpy()[valid] <= 0.0)


def test_forward_noalloc_matches_forward(device):
    big = WL.make_custom([(100, 2000, 1900, 17)], D=256, V=20011, seed=990, targets="zipf")
    small = WL.make_custom([(3, 100, 90, 2)], D=128, V=7000, seed=991)
    _say(f"[gpu] no-allocation forward: M={big.M} V={big.V} D={big.D}, then M={small.M} V={small.V}")
    _compare(big, device)
    _compare(small, device)
    _compare(small, device, softcap=3.0, with_bm=True)
    _compare(big, device)


def test_forward_noalloc_rejects_beyond_its_scratch(device):
    lib = B.load()
    M = B.NOALLOC_MAX_M + 1
    st = lib.cce_forward_noalloc(1 << 20, 1 << 20, 1 << 20, M, 10, 8, 0.0, 1 << 20, 1 << 20, None,
                                 1 << 20, None)
    assert st == B.CCE_ESHAPE
