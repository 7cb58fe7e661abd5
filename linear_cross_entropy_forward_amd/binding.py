"""ctypes binding of libflashcce.so (C-ABI declared in include/flashcce.h).

Argument marshalling only: every step of the head runs in the HIP library.
Torch is used for device memory and the current stream.  If the library is
missing the first call raises; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflashcce.so")

CCE_OK, CCE_EINVAL, CCE_ESHAPE, CCE_EWORKSPACE, CCE_EDEVICE, CCE_ELAUNCH = range(6)
KIND_IGNORE, KIND_PROMPT, KIND_CHOSEN, KIND_REJECTED = 0, 1, 2, 3
SCOPE_FULL, SCOPE_RESPONSE = 0, 1
DERR_TARGET, DERR_PAIR, DERR_EMPTY_SPAN, DERR_NONFINITE = 1, 2, 4, 8
OBJ_ORPO, OBJ_SIGMOID, OBJ_IPO, OBJ_HINGE = 0, 1, 2, 3

# exported symbols and their C signatures (kept in step with include/flashcce.h)
_c_i64, _c_f, _c_p, _c_sz, _c_i = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "cce_abi_version": (ctypes.c_int, []),
    "cce_status_string": (ctypes.c_char_p, [_c_i]),
    "cce_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "cce_forward": (_c_i, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_f, _c_p, _c_p, _c_p, _c_p, _c_p,
                           _c_sz, _c_p]),
    "orpo_epilogue": (_c_i, [_c_p, _c_p, _c_p, _c_i64, ctypes.c_int32, _c_f, _c_i, _c_p, _c_p, _c_p,
                             _c_p, _c_p, _c_sz, _c_p]),
    "cce_backward": (_c_i, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_f, _c_f,
                            _c_f, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "pref_epilogue": (_c_i, [_c_p, _c_p, _c_p, _c_i64, ctypes.c_int32, _c_i, _c_f, _c_f, _c_f, _c_f,
                             _c_i, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "cce_workspace_bytes_q": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "cce_forward_q": (_c_i, [_c_p, _c_p, _c_p, _c_p, _c_i, _c_i, _c_p, _c_i64, _c_i64, _c_i64, _c_f,
                             _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "cce_backward_q": (_c_i, [_c_p, _c_p, _c_p, _c_p, _c_i, _c_i, _c_p, _c_p, _c_p, _c_p, _c_i64,
                              _c_i64, _c_i64, _c_f, _c_f, _c_f, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "cce_forward_noalloc": (_c_i, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_f, _c_p, _c_p, _c_p,
                                   _c_p, _c_p]),
    "cce_timing_begin": (_c_i, [_c_p, _c_p, _c_p, ctypes.c_int32]),
    "cce_timing_end": (ctypes.c_int32, []),
    "cce_kernel_name": (ctypes.c_char_p, [ctypes.c_int32]),
}

_lib = None
_lock = threading.Lock()


class CCEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m linear_cross_entropy_forward_amd.build`")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def kernel_source_hash() -> str:
    """sha256 over the HIP sources (identifies the kernels a measurement was taken on)."""
    import glob
    import hashlib
    hsh = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(p, "rb") as f:
            hsh.update(os.path.basename(p).encode() + b"\0" + f.read())
    return hsh.hexdigest()[:16]


def status_string(status: int) -> str:
    return load().cce_status_string(int(status)).decode()


def workspace_bytes(M: int, V: int, D: int) -> int:
    return int(load().cce_workspace_bytes(int(M), int(V), int(D)))


def workspace_bytes_q(M: int, V: int, D: int) -> int:
    return int(load().cce_workspace_bytes_q(int(M), int(V), int(D)))


def block_max_shape(M: int, V: int) -> Tuple[int, int]:
    """Shape of the forward's saved block maximum: [ceil(V / 256), M]."""
    return ((int(V) + 255) // 256, int(M))


def _opt(t, name: str, shape) -> int:
    """Pointer of an optional fp32 device tensor (None -> NULL)."""
    return 0 if t is None else _dev(t, name, torch.float32, shape)


def _check(fn: str, status: int):
    if status != CCE_OK:
        raise CCEError(fn, status)


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _bf16(t: torch.Tensor, name: str, shape):
    if t.dtype in (torch.int16, torch.uint16):
        t = t.view(torch.bfloat16)
    return _dev(t, name, torch.bfloat16, shape)


class Head:
    """One head configuration (M, V, D) with its workspace and status word.

    The workspace is allocated once by torch (the library allocates nothing)
    and reused by every call; calls enqueue on the given (or current) stream.
    """

    def __init__(self, M: int, V: int, D: int, device=None, quantized: bool = False):
        self.M, self.V, self.D = int(M), int(V), int(D)
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        nbytes = (workspace_bytes_q if quantized else workspace_bytes)(self.M, self.V, self.D)
        if nbytes == 0:
            raise ValueError(f"invalid sizes M={M} V={V} D={D}")
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.ws.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        self.ws_bytes = nbytes
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)

    # -- forward --------------------------------------------------------------
    def forward(self, h, W, y, logp=None, lse=None, stream=None, softcap: float = 0.0,
                block_max=None):
        """block_max: None, or an fp32 [ceil(V / 256), M] tensor that receives the
        per-(vocab block, row) maximum logit for the backward's block skip."""
        M, V, D = self.M, self.V, self.D
        if logp is None:
            logp = torch.empty(M, dtype=torch.float32, device=self.device)
        if lse is None:
            lse = torch.empty(M, dtype=torch.float32, device=self.device)
        st = load().cce_forward(_bf16(h, "h", (M, D)), _bf16(W, "W", (V, D)),
                                _dev(y, "y", torch.int32, (M,)), M, V, D, float(softcap),
                                _dev(logp, "logp", torch.float32, (M,)),
                                _dev(lse, "lse", torch.float32, (M,)),
                                _opt(block_max, "block_max", block_max_shape(M, V)),
                                self.status.data_ptr(), self.ws_ptr, self.ws_bytes, _stream_ptr(stream))
        _check("cce_forward", st)
        return logp, lse

    # -- ORPO epilogue ------------------------------------------------------
    def epilogue(self, logp, y, seg, n_pairs: int, lam: float, scope: int,
                 out5=None, pair_stats=None, coef=None, stream=None):
        M = self.M
        if out5 is None:
            out5 = torch.empty(5, dtype=torch.float32, device=self.device)
        if pair_stats is None:
            pair_stats = torch.empty((n_pairs, 8), dtype=torch.float32, device=self.device)
        if coef is None:
            coef = torch.empty(M, dtype=torch.float32, device=self.device)
        st = load().orpo_epilogue(_dev(logp, "logp", torch.float32, (M,)),
                                  _dev(y, "y", torch.int32, (M,)),
                                  _dev(seg, "seg", torch.int32, (M,)), M, int(n_pairs), float(lam),
                                  int(scope), _dev(out5, "out5", torch.float32, (5,)),
                                  _dev(pair_stats, "pair_stats", torch.float32, (n_pairs, 8)),
                                  _dev(coef, "coef", torch.float32, (M,)),
                                  self.status.data_ptr(), self.ws_ptr, self.ws_bytes, _stream_ptr(stream))
        _check("orpo_epilogue", st)
        return out5, pair_stats, coef

    # -- preference-objective epilogue ----------------------------------------
    def pref_epilogue(self, logp, y, seg, n_pairs: int, objective: int, nll_weight: float,
                      lam: float, beta: float, gamma: float, scope: int,
                      out5=None, pair_stats=None, coef=None, stream=None):
        M = self.M
        if out5 is None:
            out5 = torch.empty(5, dtype=torch.float32, device=self.device)
        if pair_stats is None:
            pair_stats = torch.empty((n_pairs, 8), dtype=torch.float32, device=self.device)
        if coef is None:
            coef = torch.empty(M, dtype=torch.float32, device=self.device)
        st = load().pref_epilogue(_dev(logp, "logp", torch.float32, (M,)),
                                  _dev(y, "y", torch.int32, (M,)),
                                  _dev(seg, "seg", torch.int32, (M,)), M, int(n_pairs),
                                  int(objective), float(nll_weight), float(lam), float(beta),
                                  float(gamma), int(scope),
                                  _dev(out5, "out5", torch.float32, (5,)),
                                  _dev(pair_stats, "pair_stats", torch.float32, (n_pairs, 8)),
                                  _dev(coef, "coef", torch.float32, (M,)),
                                  self.status.data_ptr(), self.ws_ptr, self.ws_bytes, _stream_ptr(stream))
        _check("pref_epilogue", st)
        return out5, pair_stats, coef

    # -- backward -------------------------------------------------------------
    def backward(self, h, W, y, lse, coef, filter_eps: float = 0.0, block_eps: float = 0.0,
                 dh=None, dW=None, stream=None, softcap: float = 0.0, block_max=None):
        M, V, D = self.M, self.V, self.D
        if dh is None:
            dh = torch.empty((M, D), dtype=torch.float32, device=self.device)
        if dW is None:
            dW = torch.empty((V, D), dtype=torch.float32, device=self.device)
        st = load().cce_backward(_bf16(h, "h", (M, D)), _bf16(W, "W", (V, D)),
                                 _dev(y, "y", torch.int32, (M,)),
                                 _dev(lse, "lse", torch.float32, (M,)),
                                 _dev(coef, "coef", torch.float32, (M,)),
                                 _opt(block_max, "block_max", block_max_shape(M, V)), M, V, D,
                                 float(softcap), float(filter_eps), float(block_eps),
                                 _dev(dh, "dh", torch.float32, (M, D)),
                                 _dev(dW, "dW", torch.float32, (V, D)),
                                 self.status.data_ptr(), self.ws_ptr, self.ws_bytes, _stream_ptr(stream))
        _check("cce_backward", st)
        return dh, dW

    # -- quantised (frozen) head ---------------------------------------------
    def _quant_args(self, Wq, scales, biases, bits: int, group_size: int):
        V, D = self.V, self.D
        if bits not in (4, 8) or group_size not in (32, 64, 128) or D % group_size:
            raise ValueError(f"unsupported quantisation bits={bits} group_size={group_size} D={D}")
        if Wq.dtype == torch.uint32:
            Wq = Wq.view(torch.int32)
        return (_dev(Wq, "Wq", torch.int32, (V, D * bits // 32)),
                _bf16(scales, "scales", (V, D // group_size)),
                _bf16(biases, "biases", (V, D // group_size)), int(bits), int(group_size))

    def forward_q(self, h, Wq, scales, biases, bits: int, group_size: int, y, logp=None, lse=None,
                  stream=None, softcap: float = 0.0, block_max=None):
        """Forward over an affine-quantised head (needs a Head built with quantized=True)."""
        M, V, D = self.M, self.V, self.D
        if logp is None:
            logp = torch.empty(M, dtype=torch.float32, device=self.device)
        if lse is None:
            lse = torch.empty(M, dtype=torch.float32, device=self.device)
        st = load().cce_forward_q(_bf16(h, "h", (M, D)), *self._quant_args(Wq, scales, biases, bits, group_size),
                                  _dev(y, "y", torch.int32, (M,)), M, V, D, float(softcap),
                                  _dev(logp, "logp", torch.float32, (M,)),
                                  _dev(lse, "lse", torch.float32, (M,)),
                                  _opt(block_max, "block_max", block_max_shape(M, V)),
                                  self.status.data_ptr(), self.ws_ptr, self.ws_bytes, _stream_ptr(stream))
        _check("cce_forward_q", st)
        return logp, lse

    def backward_q(self, h, Wq, scales, biases, bits: int, group_size: int, y, lse, coef,
                   filter_eps: float = 0.0, block_eps: float = 0.0, dh=None, stream=None,
                   softcap: float = 0.0, block_max=None):
        """dh of an affine-quantised (frozen) head."""
        M, V, D = self.M, self.V, self.D
        if dh is None:
            dh = torch.empty((M, D), dtype=torch.float32, device=self.device)
        st = load().cce_backward_q(_bf16(h, "h", (M, D)), *self._quant_args(Wq, scales, biases, bits, group_size),
                                   _dev(y, "y", torch.int32, (M,)),
                                   _dev(lse, "lse", torch.float32, (M,)),
                                   _dev(coef, "coef", torch.float32, (M,)),
                                   _opt(block_max, "block_max", block_max_shape(M, V)), M, V, D,
                                   float(softcap), float(filter_eps), float(block_eps),
                                   _dev(dh, "dh", torch.float32, (M, D)),
                                   self.status.data_ptr(), self.ws_ptr, self.ws_bytes, _stream_ptr(stream))
        _check("cce_backward_q", st)
        return dh

    def read_status(self) -> int:
        torch.cuda.synchronize(self.device)
        return int(self.status.item()) & 0xFFFFFFFF

    def clear_status(self):
        self.status.zero_()


NOALLOC_MAX_M = 786432


def forward_noalloc(h, W, y, status, logp=None, lse=None, stream=None, softcap: float = 0.0,
                    block_max=None):
    """cce_forward through its no-allocation variant (scratch in the library's
    fixed device array; M <= NOALLOC_MAX_M).  status: an int32 [1] device tensor
    (the device status word)."""
    M, D = int(h.shape[0]), int(h.shape[1])
    V = int(W.shape[0])
    if logp is None:
        logp = torch.empty(M, dtype=torch.float32, device=h.device)
    if lse is None:
        lse = torch.empty(M, dtype=torch.float32, device=h.device)
    st = load().cce_forward_noalloc(_bf16(h, "h", (M, D)), _bf16(W, "W", (V, D)),
                                    _dev(y, "y", torch.int32, (M,)), M, V, D, float(softcap),
                                    _dev(logp, "logp", torch.float32, (M,)),
                                    _dev(lse, "lse", torch.float32, (M,)),
                                    _opt(block_max, "block_max", block_max_shape(M, V)),
                                    _dev(status, "status", torch.int32, (1,)), _stream_ptr(stream))
    _check("cce_forward_noalloc", st)
    return logp, lse


class LaunchTimer:
    """Per-launch timing through the library's profiling hook: within
    ``with timer:`` every kernel the library enqueues from this thread is
    bracketed by two events (recorded on the call's stream).  After the stream
    has completed, ``launches()`` gives (kernel name, milliseconds, algorithmic
    FLOPs) per launch.
    Holds `capacity` launches; later ones are not bracketed."""

    def __init__(self, capacity: int = 256):
        self.capacity = int(capacity)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * self.capacity)]
        # torch creates an event's HIP handle on its first record
        st = torch.cuda.current_stream()
        for e in self.events:
            e.record(st)
        torch.cuda.synchronize()
        self._handles = (ctypes.c_void_p * (2 * self.capacity))(*[e.cuda_event for e in self.events])
        self._kinds = (ctypes.c_int32 * self.capacity)()
        self._flops = (ctypes.c_double * self.capacity)()
        self.n = 0

    def __enter__(self):
        _check("cce_timing_begin", load().cce_timing_begin(self._handles, self._kinds, self._flops,
                                                           self.capacity))
        return self

    def __exit__(self, *exc):
        n = int(load().cce_timing_end())
        if n < 0 and exc[0] is None:
            raise RuntimeError("cce_timing_end: the timing window failed to record its events")
        self.n = max(n, 0)
        return False

    def launches(self):
        """[(kernel name, milliseconds, algorithmic FLOPs)] per bracketed launch."""
        lib = load()
        return [(lib.cce_kernel_name(int(self._kinds[i])).decode(),
                 self.events[2 * i].elapsed_time(self.events[2 * i + 1]), float(self._flops[i]))
                for i in range(self.n)]


def to_device_bits(bits, device) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bf16 device tensor (same bits)."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def step(head: Head, h, W, y, seg, n_pairs, lam, scope, filter_eps=0.0, block_eps=0.0, stream=None,
         softcap=0.0, block_max=None):
    """One whole pass: forward, epilogue, backward (all enqueued on one stream).
    block_max: None, or a [ceil(V / 256), M] fp32 tensor the forward fills and
    the backward's block skip reads."""
    logp, lse = head.forward(h, W, y, stream=stream, softcap=softcap, block_max=block_max)
    out5, pstats, coef = head.epilogue(logp, y, seg, n_pairs, lam, scope, stream=stream)
    dh, dW = head.backward(h, W, y, lse, coef, filter_eps, block_eps, stream=stream, softcap=softcap,
                           block_max=block_max)
    return dict(logp=logp, lse=lse, out5=out5, pair_stats=pstats, coef=coef, dh=dh, dW=dW)
