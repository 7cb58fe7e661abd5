"""Host-side checks of the C-ABI library (no kernel is launched here).

The library must load, export every function include/flashcce.h declares, size
its workspace independently of V, and reject bad arguments on the host before
touching a device.
"""
import ctypes
import os
import re

import pytest

from linear_cross_entropy_forward_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashcce.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libflashcce.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == {"cce_abi_version", "cce_status_string", "cce_workspace_bytes", "cce_forward",
                     "orpo_epilogue", "pref_epilogue", "cce_backward", "cce_workspace_bytes_q",
                     "cce_forward_q", "cce_backward_q", "cce_timing_begin", "cce_timing_end",
                     "cce_kernel_name", "cce_forward_noalloc"}
    assert names == set(B.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert B.load().cce_abi_version() == 6


def test_status_strings():
    for s in range(6):
        assert B.status_string(s).startswith("CCE_")
    assert "unknown" in B.status_string(99)


def test_workspace_is_independent_of_V():
    M, D = 8192, 2560
    sizes = [B.workspace_bytes(M, V, D) for V in (32768, 65536, 131072, 262144, 1 << 20)]
    assert len(set(sizes)) == 1 and sizes[0] > 0
    # and it does not grow with V below one chunk either beyond the chunk size
    assert B.workspace_bytes(M, 300, D) <= sizes[0]
    assert B.workspace_bytes(0, 10, 10) == 0
    assert B.workspace_bytes(10, 0, 10) == 0
    assert B.workspace_bytes(10, 10, 0) == 0
    assert B.workspace_bytes(1 << 22, 10, 10) == 0


def grad_buffers(D):
    """bf16 gradient chunk buffers: two when D % 32 == 0 (the pipelined backward
    alternates between them), else one."""
    return 2 if D % 32 == 0 else 1


def test_workspace_small_M_bounded():
    """Small M reserves split-K partials of dh, within half the gradient chunk."""
    for M, D in ((1279, 2048), (1024, 4096), (300, 64), (300, 65)):
        ws = B.workspace_bytes(M, 262144, D)
        Mpad = (M + 255) // 256 * 256
        g = 2 * Mpad * 16384
        nb = grad_buffers(D)
        assert nb * g <= ws <= nb * g + g // 2 + 4 * 1024 * 1024
        assert ws == B.workspace_bytes(M, 1 << 20, D)


def test_workspace_bound_at_gemma_and_stress():
    # the two bf16 gradient chunks dominate: 2 * (2 * Mpad * 16384) bytes; besides them about
    # 300 bytes a row (forward partials, the epilogue's pair table and run records, the onehot
    # part's per-row t and sort buffers) and D / 8 bytes a row (the onehot dW pass's window
    # partials, two fp32 rows of D per 64 sorted rows)
    for M, D in ((8192, 2560), (16384, 4096)):
        ws = B.workspace_bytes(M, 262144, D)
        assert 4 * M * 16384 <= ws < 4 * M * 16384 + 300 * M + M * D // 8 + 1_000_000


FAKE = 1 << 20   # a non-null pointer value; never dereferenced on these paths


def test_forward_argument_errors():
    lib = B.load()
    ws = B.workspace_bytes(300, 1000, 64)
    # h, W, y, M, V, D, softcap, logp, lse, block_max, dev_status, ws, ws_bytes, stream
    ok = (FAKE, FAKE, FAKE, 300, 1000, 64, 0.0, FAKE, FAKE, None, FAKE, FAKE * 256, ws, None)
    for i in (0, 1, 2, 7, 8, 10, 11):
        args = list(ok)
        args[i] = None
        assert lib.cce_forward(*args) == B.CCE_EINVAL
    for bad in (-1.0, float("nan"), float("inf")):
        args = list(ok)
        args[6] = bad
        assert lib.cce_forward(*args) == B.CCE_EINVAL
    for i in (3, 4, 5):
        args = list(ok)
        args[i] = 0
        assert lib.cce_forward(*args) == B.CCE_ESHAPE
    args = list(ok)
    args[12] = ws - 1
    assert lib.cce_forward(*args) == B.CCE_EWORKSPACE
    args = list(ok)
    args[11] = FAKE * 256 + 16          # misaligned workspace
    assert lib.cce_forward(*args) == B.CCE_EWORKSPACE


def test_epilogue_argument_errors():
    lib = B.load()
    ws = B.workspace_bytes(300, 1, 1)
    ok = [FAKE, FAKE, FAKE, 300, 2, 0.1, 0, FAKE, None, FAKE, FAKE, FAKE * 256, ws, None]
    a = list(ok); a[6] = 7
    assert lib.orpo_epilogue(*a) == B.CCE_EINVAL
    a = list(ok); a[5] = float("nan")
    assert lib.orpo_epilogue(*a) == B.CCE_EINVAL
    a = list(ok); a[4] = 0
    assert lib.orpo_epilogue(*a) == B.CCE_ESHAPE
    a = list(ok); a[4] = 301
    assert lib.orpo_epilogue(*a) == B.CCE_ESHAPE
    a = list(ok); a[0] = None
    assert lib.orpo_epilogue(*a) == B.CCE_EINVAL
    a = list(ok); a[12] = 10
    assert lib.orpo_epilogue(*a) == B.CCE_EWORKSPACE


def test_pref_epilogue_argument_errors():
    lib = B.load()
    ws = B.workspace_bytes(300, 1, 1)
    # logp, y, seg, M, n_pairs, objective, nll_weight, lambda, beta, gamma, scope, out5,
    # pair_stats, coef, dev_status, ws, ws_bytes, stream
    ok = [FAKE, FAKE, FAKE, 300, 2, 1, 1.0, 0.1, 2.0, 0.5, 0, FAKE, None, FAKE, FAKE, FAKE * 256, ws,
          None]
    for i, bad in ((5, -1), (5, 4), (10, 2), (6, float("nan")), (7, float("inf")), (8, float("nan")),
                   (9, float("-inf")), (0, None), (13, None)):
        a = list(ok); a[i] = bad
        assert lib.pref_epilogue(*a) == B.CCE_EINVAL, (i, bad)
    a = list(ok); a[4] = 301
    assert lib.pref_epilogue(*a) == B.CCE_ESHAPE
    a = list(ok); a[16] = 10
    assert lib.pref_epilogue(*a) == B.CCE_EWORKSPACE


def test_backward_argument_errors():
    lib = B.load()
    ws = B.workspace_bytes(300, 1000, 64)
    # h, W, y, lse, coef, block_max, M, V, D, softcap, filter_eps, block_eps, dh, dW, dev_status,
    # ws, ws_bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 300, 1000, 64, 0.0, 0.0, 0.0, FAKE, FAKE, FAKE,
          FAKE * 256, ws, None]
    for i, bad in ((9, -1.0), (9, float("nan")), (10, -1.0), (11, float("inf"))):
        a = list(ok); a[i] = bad
        assert lib.cce_backward(*a) == B.CCE_EINVAL
    a = list(ok); a[13] = None
    assert lib.cce_backward(*a) == B.CCE_EINVAL
    a = list(ok); a[8] = -3
    assert lib.cce_backward(*a) == B.CCE_ESHAPE
    a = list(ok); a[16] = 1
    assert lib.cce_backward(*a) == B.CCE_EWORKSPACE


def test_quant_workspace_adds_two_chunk_buffers():
    M, D = 8192, 2560
    sizes = [B.workspace_bytes_q(M, V, D) for V in (32768, 262144, 1 << 20)]
    assert len(set(sizes)) == 1
    # both backwards are pipelined over two gradient buffers; the quantised one
    # adds two bf16 chunk buffers of the dequantised head (16384 x D each), two
    # fp32 rows of Mpad, and its own split dh partials (at most 7 fp32 M x D
    # buffers) in place of the bf16 head's
    bf16 = B.workspace_bytes(M, 262144, D)
    extra = sizes[0] - bf16
    assert 2 * 2 * 16384 * D + 8 * M - 7 * M * D * 4 <= extra
    assert extra <= 2 * 2 * 16384 * D + 8 * M + 7 * M * D * 4 + 4 * 256
    # the partials stay within half the gradient chunk
    assert sizes[0] <= bf16 + 2 * 2 * 16384 * D + 8 * M + 8192 * 16384 + 4 * 256
    assert B.workspace_bytes_q(0, 10, 64) == 0


def test_forward_q_argument_errors():
    lib = B.load()
    ws = B.workspace_bytes_q(300, 1000, 128)
    # h, Wq, scales, biases, bits, group_size, y, M, V, D, softcap, logp, lse, block_max,
    # dev_status, ws, ws_bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, 4, 64, FAKE, 300, 1000, 128, 0.0, FAKE, FAKE, None, FAKE,
          FAKE * 256, ws, None]
    for i, bad in ((0, None), (1, None), (2, None), (3, None), (6, None), (11, None), (14, None),
                   (4, 2), (4, 16), (5, 16), (5, 256), (10, float("nan")), (10, -1.0)):
        a = list(ok); a[i] = bad
        assert lib.cce_forward_q(*a) == B.CCE_EINVAL, (i, bad)
    a = list(ok); a[9] = 96                       # D not a multiple of the group
    assert lib.cce_forward_q(*a) == B.CCE_EINVAL
    a = list(ok); a[7] = 0
    assert lib.cce_forward_q(*a) == B.CCE_ESHAPE
    a = list(ok); a[16] = ws - 1                   # one byte short
    assert lib.cce_forward_q(*a) == B.CCE_EWORKSPACE


def test_backward_q_argument_errors():
    lib = B.load()
    ws = B.workspace_bytes_q(300, 1000, 128)
    # h, Wq, scales, biases, bits, group_size, y, lse, coef, block_max, M, V, D, softcap,
    # filter_eps, block_eps, dh, dev_status, ws, ws_bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, 8, 32, FAKE, FAKE, FAKE, None, 300, 1000, 128, 0.0, 0.0, 0.0, FAKE,
          FAKE, FAKE * 256, ws, None]
    for i, bad in ((1, None), (8, None), (16, None), (4, 3), (5, 48), (14, -1.0), (15, float("inf"))):
        a = list(ok); a[i] = bad
        assert lib.cce_backward_q(*a) == B.CCE_EINVAL, (i, bad)
    a = list(ok); a[11] = -1
    assert lib.cce_backward_q(*a) == B.CCE_ESHAPE
    a = list(ok); a[19] = ws - 1
    assert lib.cce_backward_q(*a) == B.CCE_EWORKSPACE


def test_valid_call_without_gfx950_is_refused():
    """With valid arguments and no gfx950 device the library refuses (it never
    falls back to another path)."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible; covered by the gpu tests")
    except Exception:
        pass
    lib = B.load()
    ws = B.workspace_bytes(300, 1000, 64)
    st = lib.cce_forward(FAKE, FAKE, FAKE, 300, 1000, 64, 0.0, FAKE, FAKE, None, FAKE, FAKE * 256, ws,
                         None)
    assert st == B.CCE_EDEVICE
    wq = B.workspace_bytes_q(300, 1000, 64)
    st = lib.cce_forward_q(FAKE, FAKE, FAKE, FAKE, 4, 32, FAKE, 300, 1000, 64, 0.0, FAKE, FAKE, None,
                           FAKE, FAKE * 256, wq, None)
    assert st == B.CCE_EDEVICE


def test_timing_hook_host_side():
    """The timing window's argument checks, names of the kernel kinds, and
    end-without-begin (no GPU call is made)."""
    lib = B.load()
    assert lib.cce_timing_end() == -1
    kinds = (ctypes.c_int32 * 2)()
    ev = (ctypes.c_void_p * 4)(1, 2, 3, 0)
    assert lib.cce_timing_begin(None, kinds, None, 2) == B.CCE_EINVAL
    assert lib.cce_timing_begin(ev, None, None, 2) == B.CCE_EINVAL
    assert lib.cce_timing_begin(ev, kinds, None, 0) == B.CCE_EINVAL
    assert lib.cce_timing_begin(ev, kinds, None, 2) == B.CCE_EINVAL   # a NULL event
    assert lib.cce_timing_end() == -1
    names = {lib.cce_kernel_name(k).decode() for k in range(1, 21)}
    assert {"k_fwd", "k_bwd_fused", "k_grads", "k_recompute_tall", "k_epi_blocks", "k_target_dh",
            "k_sort", "k_target_dw"} <= names
    assert "unknown" not in names
    assert lib.cce_kernel_name(0).decode() == "unknown"


def test_forward_noalloc_argument_errors():
    """Host checks of the no-allocation forward, before any HIP call: NULLs, a bad
    cap, bad sizes, and M above the fixed scratch's limit."""
    lib = B.load()
    f = lib.cce_forward_noalloc
    args = [FAKE, FAKE, FAKE, 100, 200, 64, 0.0, FAKE, FAKE, None, FAKE, None]
    for i in (0, 1, 2, 7, 8, 10):
        a = list(args)
        a[i] = None
        assert f(*a) == B.CCE_EINVAL, i
    a = list(args)
    a[6] = -1.0
    assert f(*a) == B.CCE_EINVAL
    for M, V, D in ((0, 10, 10), (10, 0, 10), (10, 10, 0), (B.NOALLOC_MAX_M + 1, 10, 10)):
        a = list(args)
        a[3:6] = [M, V, D]
        assert f(*a) == B.CCE_ESHAPE, (M, V, D)
    # within the limit the call gets past the size checks and, with no GPU visible,
    # stops at the device check (never reached with a GPU: the pointers are fake)
    try:
        import torch
        if torch.cuda.is_available():
            return
    except Exception:
        pass
    a = list(args)
    a[3] = B.NOALLOC_MAX_M
    assert f(*a) == B.CCE_EDEVICE
