"""MI355X-native error-feedback top-k gradient sparsifier.

Thin ctypes binding over ``libtgs.so`` (C ABI declared in ``include/tgs.h``).
This module only marshals arguments: every step of the three operations runs
in the library's HIP kernels.  PyTorch supplies device memory and streams.

Operations (cited by page title and section):

* ``topk_ef_step``      -- error-feedback top-k (arxivdaily listing for arXiv
  2004.05298, entries "Sparsified SGD with Memory" and "The Convergence of
  Sparsified Gradient Methods").
* ``threshold_ef_step`` -- hard-threshold sparsifier with error feedback (same
  listing, entry "Rethinking gradient sparsification as total error
  minimization").
* ``gtopk_merge``       -- the gTop-k tournament (nubint review "A Distributed
  Synchronous SGD Algorithm with Global Top-k Sparsification for Low Bandwidth
  Networks", ABSTRACT and Method).
* ``threshold_estimate`` / ``estimated_threshold_ef_step`` -- a threshold
  estimated from a sample, fed to the hard threshold on the device (arxivdaily
  listing, entry "Near-Optimal Sparse Allreduce for Distributed Deep
  Learning"; fugumt page for arXiv 2502.07634, related-paper entry "An
  Efficient Statistical-based Gradient Compression Technique for Distributed
  Training Systems").
* ``rtopk_ef_step``     -- k random entries of the top r (arxivdaily listing,
  entry "rTop-k: A Statistical Estimation Approach to Distributed SGD").

There is no fallback: if ``libtgs.so`` is missing or cannot be loaded, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtgs.so")

TGS_OK = 0
TGS_EINVAL = -1
TGS_EWORKSPACE = -2
TGS_EHIP = -3
TGS_EDEVICE = -4

OPT_TOPK_PATH = 1
OPT_MAIN_GRID = 2

_STATUS_EXC = {TGS_EINVAL: ValueError, TGS_EWORKSPACE: MemoryError}


class TgsError(RuntimeError):
    """Raised for TGS_EHIP and TGS_EDEVICE (a bounded wait timed out or
    counts were inconsistent: the outputs of the calls since the error word was
    last read are not to be used)."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None
_lib_lock = threading.Lock()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libtgs.so not found at %s; build it with "
                "`python -m top_gradient_sparsification_amd.build`" % LIB_PATH)
        # torch is imported first, so the library binds to torch's HIP runtime
        # (same soname) and torch streams are valid handles for it.
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        lib.tgs_topk_workspace_bytes.argtypes = [i64, i64]
        lib.tgs_topk_workspace_bytes.restype = sz
        lib.tgs_topk_ef_step.argtypes = [vp, vp, i64, i64, vp, vp, vp, sz, vp]
        lib.tgs_topk_ef_step.restype = i32
        lib.tgs_topk_segmented_workspace_bytes.argtypes = [i32, vp, vp]
        lib.tgs_topk_segmented_workspace_bytes.restype = sz
        lib.tgs_topk_ef_step_segmented.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        lib.tgs_topk_ef_step_segmented.restype = i32
        lib.tgs_threshold_workspace_bytes.argtypes = [i64]
        lib.tgs_threshold_workspace_bytes.restype = sz
        lib.tgs_threshold_ef_step.argtypes = [vp, vp, i64, ctypes.c_float, vp, vp, i64, vp, vp, sz, vp]
        lib.tgs_threshold_ef_step.restype = i32
        lib.tgs_gtopk_workspace_bytes.argtypes = [i32, i64, i64]
        lib.tgs_gtopk_workspace_bytes.restype = sz
        lib.tgs_gtopk_merge.argtypes = [vp, vp, i32, i64, i64, vp, vp, vp, vp, sz, vp]
        lib.tgs_gtopk_merge.restype = i32
        lib.tgs_check_device_error.argtypes = [vp, vp]
        lib.tgs_check_device_error.restype = i32
        lib.tgs_workspace_init.argtypes = [vp, sz, vp]
        lib.tgs_workspace_init.restype = i32
        lib.tgs_threshold_estimate_workspace_bytes.argtypes = [i64]
        lib.tgs_threshold_estimate_workspace_bytes.restype = sz
        lib.tgs_threshold_estimate.argtypes = [vp, vp, i64, vp, i64, i64, vp, vp, sz, vp]
        lib.tgs_threshold_estimate.restype = i32
        lib.tgs_threshold_ef_step_dev.argtypes = [vp, vp, i64, vp, vp, vp, i64, vp, vp, sz, vp]
        lib.tgs_threshold_ef_step_dev.restype = i32
        u64 = ctypes.c_uint64
        lib.tgs_rtopk_workspace_bytes.argtypes = [i64, i64, i64]
        lib.tgs_rtopk_workspace_bytes.restype = sz
        lib.tgs_rtopk_ef_step.argtypes = [vp, vp, i64, i64, i64, u64, u64, vp, vp, vp, sz, vp]
        lib.tgs_rtopk_ef_step.restype = i32
        lib.tgs_status_string.argtypes = [i32]
        lib.tgs_status_string.restype = ctypes.c_char_p
        lib.tgs_last_error.argtypes = []
        lib.tgs_last_error.restype = ctypes.c_char_p
        lib.tgs_set_option.argtypes = [i32, i64]
        lib.tgs_set_option.restype = i32
        lib.tgs_profile_next_call.argtypes = [vp, vp]
        lib.tgs_profile_next_call.restype = i32
        lib.tgs_profile_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
        lib.tgs_profile_elapsed_ms.restype = i32
        _lib = lib
    return _lib


def library():
    """The loaded ctypes library (raises if it is missing)."""
    return _load()


def _check(status: int, what: str):
    if status == TGS_OK:
        return
    lib = _load()
    msg = "%s: %s (%s)" % (what, lib.tgs_status_string(status).decode(), lib.tgs_last_error().decode())
    raise _STATUS_EXC.get(status, TgsError)(msg) if status in _STATUS_EXC else TgsError(status, msg)


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _full_device(device) -> torch.device:
    """``device`` with its index filled in ("cuda" -> the current device)."""
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    return dev


def _require(t, dtype, name, device=None, min_numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s holds %d entries, needs %d" % (name, t.numel(), min_numel))


# --------------------------------------------------------------- workspaces --
_ws_cache: dict = {}
_ws_lock = threading.Lock()


def workspace(kind: str, nbytes: int, device) -> torch.Tensor:
    """A zero-initialised (hence ready) uint8 device buffer of at least
    ``nbytes``, cached per (device, current stream, kind).  Calls that share it
    are ordered on that stream."""
    dev = torch.device(device)
    key = (dev.index, _stream_handle(dev), kind)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
            _ws_cache[key] = buf
        return buf


# --------------------------------------------------------------- operations --
def topk_workspace_bytes(n: int, k: int) -> int:
    return int(_load().tgs_topk_workspace_bytes(n, k))


def topk_ef_step(grad: torch.Tensor, residual: torch.Tensor, k: int, out_idx=None, out_val=None,
                 ws: torch.Tensor | None = None):
    """One error-feedback top-k step on the GPU.

    ``residual`` (float32, same length as ``grad``) is updated in place to
    ``acc`` with the selected entries zeroed, where ``acc = residual + grad``.
    Returns ``(idx int32[k], val float32[k])`` in (|acc| desc, index asc) order.
    """
    _require(grad, torch.float32, "grad")
    _require(residual, torch.float32, "residual")
    n = grad.numel()
    if residual.numel() != n or residual.device != grad.device:
        raise ValueError("grad and residual must have the same length and device")
    k = int(k)
    dev = grad.device
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty(k, dtype=torch.float32, device=dev)
    _require(out_idx, torch.int32, "out_idx")
    _require(out_val, torch.float32, "out_val")
    if out_idx.numel() < k or out_val.numel() < k:
        raise ValueError("outputs hold fewer than k entries")
    lib = _load()
    need = lib.tgs_topk_workspace_bytes(n, k)
    if need == 0:
        raise ValueError("invalid sizes n=%d k=%d" % (n, k))
    if ws is None:
        ws = workspace("topk", need, dev)
    st = lib.tgs_topk_ef_step(_ptr(grad), _ptr(residual), n, k, _ptr(out_idx), _ptr(out_val), ws.data_ptr(),
                              ws.numel(), _stream_handle(dev))
    _check(st, "tgs_topk_ef_step")
    return out_idx[:k], out_val[:k]


def workspace_init(ws: torch.Tensor, stream=None):
    """Makes ``ws`` ready for any operation (a kernel zero-fills its header on
    the current stream): for workspaces not allocated zero-filled, and after a
    TGS_EDEVICE report."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda:
        raise TypeError("ws must be a GPU tensor")
    st = stream.cuda_stream if stream is not None else _stream_handle(ws.device)
    _check(_load().tgs_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(), st), "tgs_workspace_init")


def error_word(ws: torch.Tensor) -> torch.Tensor:
    """The device error word of workspace ``ws`` as a one-element int32 device
    tensor (a view: no copy, no wait).  Nonzero means a kernel flagged a
    problem since the word was last cleared by ``check_device_error``."""
    return ws[:4].view(torch.int32)


class TopkStep:
    """A prepared top-k step for repeated calls on tensors of one shape.

    Holds the outputs, the workspace and the stream, so a call costs one C-ABI
    call plus a few attribute checks: for training loops that sparsify the same
    buffer every iteration.  The library still validates every call.  Calls
    are asynchronous: ``check()`` (or ``error`` for a device-side flag) reports
    whether a kernel flagged a problem."""

    def __init__(self, n: int, k: int, device="cuda", stream=None):
        lib = _load()
        self.n, self.k = int(n), int(k)
        self.device = _full_device(device)
        need = lib.tgs_topk_workspace_bytes(self.n, self.k)
        if need == 0:
            raise ValueError("invalid sizes n=%d k=%d" % (n, k))
        self.ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
        self.out_idx = torch.empty(self.k, dtype=torch.int32, device=self.device)
        self.out_val = torch.empty(self.k, dtype=torch.float32, device=self.device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self._fn = lib.tgs_topk_ef_step
        self._args = (self.out_idx.data_ptr() if self.k else None, self.out_val.data_ptr() if self.k else None,
                      self.ws.data_ptr(), self.ws.numel(), self.stream.cuda_stream)

    def __call__(self, grad: torch.Tensor, residual: torch.Tensor):
        for t, name in ((grad, "grad"), (residual, "residual")):
            if (t.dtype != torch.float32 or t.device != self.device or t.numel() != self.n
                    or not t.is_contiguous()):
                _require(t, torch.float32, name, self.device)
                raise ValueError("this step is prepared for n=%d, %s holds %d" % (self.n, name, t.numel()))
        oi, ov, wp, wn, st = self._args
        status = self._fn(grad.data_ptr(), residual.data_ptr(), self.n, self.k, oi, ov, wp, wn, st)
        if status:
            _check(status, "tgs_topk_ef_step")
        return self.out_idx, self.out_val

    @property
    def error(self) -> torch.Tensor:
        """The workspace's device error word (int32 device tensor, no wait)."""
        return error_word(self.ws)

    def check(self):
        """Waits for the stream and raises if a kernel flagged a problem."""
        _check(_load().tgs_check_device_error(self.ws.data_ptr(), self.stream.cuda_stream), "tgs_topk_ef_step")


def _segment_table(offsets, ks):
    """(nseg, int64 offsets[nseg+1], int64 ks[nseg]) as contiguous host arrays."""
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    kk = np.ascontiguousarray(np.asarray(ks, dtype=np.int64))
    if offs.ndim != 1 or kk.ndim != 1 or offs.size != kk.size + 1:
        raise ValueError("offsets must have one entry more than ks")
    return int(kk.size), offs, kk


def topk_segmented_workspace_bytes(offsets, ks) -> int:
    nseg, offs, kk = _segment_table(offsets, ks)
    return int(_load().tgs_topk_segmented_workspace_bytes(nseg, offs.ctypes.data, kk.ctypes.data))


def topk_ef_step_segmented(grad: torch.Tensor, residual: torch.Tensor, offsets, ks, out_idx=None, out_val=None,
                           ws: torch.Tensor | None = None):
    """Layer-wise error-feedback top-k: segment s = [offsets[s], offsets[s+1])
    of ``grad``/``residual`` gets the top-k step with k = ks[s], in one call.

    Returns ``(idx int32[sum ks], val float32[sum ks])``: segment s's pairs
    start at ``sum(ks[:s])``, with indices relative to the segment's start."""
    _require(grad, torch.float32, "grad")
    _require(residual, torch.float32, "residual")
    nseg, offs, kk = _segment_table(offsets, ks)
    n = grad.numel()
    if residual.numel() != n or residual.device != grad.device:
        raise ValueError("grad and residual must have the same length and device")
    if nseg and int(offs[-1]) != n:
        raise ValueError("offsets[-1] must equal the vector length")
    total = int(kk.sum()) if nseg else 0
    dev = grad.device
    if out_idx is None:
        out_idx = torch.empty(total, dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty(total, dtype=torch.float32, device=dev)
    _require(out_idx, torch.int32, "out_idx")
    _require(out_val, torch.float32, "out_val")
    if out_idx.numel() < total or out_val.numel() < total:
        raise ValueError("outputs hold fewer than sum(ks) entries")
    lib = _load()
    need = lib.tgs_topk_segmented_workspace_bytes(nseg, offs.ctypes.data, kk.ctypes.data)
    if need == 0:
        raise ValueError("invalid segment table")
    if ws is None:
        ws = workspace("topk", need, dev)
    st = lib.tgs_topk_ef_step_segmented(_ptr(grad), _ptr(residual), nseg, offs.ctypes.data, kk.ctypes.data,
                                        _ptr(out_idx), _ptr(out_val), ws.data_ptr(), ws.numel(), _stream_handle(dev))
    _check(st, "tgs_topk_ef_step_segmented")
    return out_idx[:total], out_val[:total]


class TopkSegments:
    """A prepared layer-wise top-k step (fixed segment table) for repeated
    calls: holds the host table, the outputs, the workspace and the stream."""

    def __init__(self, offsets, ks, device="cuda", stream=None):
        lib = _load()
        self.nseg, self.offsets, self.ks = _segment_table(offsets, ks)
        self.n = int(self.offsets[-1]) if self.nseg else 0
        self.total = int(self.ks.sum()) if self.nseg else 0
        self.device = _full_device(device)
        need = lib.tgs_topk_segmented_workspace_bytes(self.nseg, self.offsets.ctypes.data, self.ks.ctypes.data)
        if need == 0:
            raise ValueError("invalid segment table")
        self.ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
        self.out_idx = torch.empty(max(self.total, 1), dtype=torch.int32, device=self.device)
        self.out_val = torch.empty(max(self.total, 1), dtype=torch.float32, device=self.device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self._fn = lib.tgs_topk_ef_step_segmented
        self._args = (self.nseg, self.offsets.ctypes.data, self.ks.ctypes.data, self.out_idx.data_ptr(),
                      self.out_val.data_ptr(), self.ws.data_ptr(), self.ws.numel(), self.stream.cuda_stream)

    def __call__(self, grad: torch.Tensor, residual: torch.Tensor):
        for t, name in ((grad, "grad"), (residual, "residual")):
            if (t.dtype != torch.float32 or t.device != self.device or t.numel() != self.n
                    or not t.is_contiguous()):
                _require(t, torch.float32, name, self.device)
                raise ValueError("this call is prepared for n=%d, %s holds %d" % (self.n, name, t.numel()))
        ns, op, kp, oi, ov, wp, wn, st = self._args
        status = self._fn(grad.data_ptr(), residual.data_ptr(), ns, op, kp, oi, ov, wp, wn, st)
        if status:
            _check(status, "tgs_topk_ef_step_segmented")
        return self.out_idx[:self.total], self.out_val[:self.total]

    @property
    def error(self) -> torch.Tensor:
        """The workspace's device error word (int32 device tensor, no wait)."""
        return error_word(self.ws)

    def check(self):
        """Waits for the stream and raises if a kernel flagged a problem."""
        _check(_load().tgs_check_device_error(self.ws.data_ptr(), self.stream.cuda_stream),
               "tgs_topk_ef_step_segmented")


def threshold_workspace_bytes(n: int) -> int:
    return int(_load().tgs_threshold_workspace_bytes(n))


def threshold_ef_step(grad: torch.Tensor, residual: torch.Tensor, lam: float, capacity: int,
                      out_idx=None, out_val=None, count=None, ws: torch.Tensor | None = None):
    """One hard-threshold step on the GPU.

    Returns ``(idx int32[capacity], val float32[capacity], count int64[1])``:
    the first ``min(count, capacity)`` entries of idx/val are the qualifying
    entries in ascending index order; ``count`` (a device tensor) is the total
    number of qualifying entries.
    """
    _require(grad, torch.float32, "grad")
    _require(residual, torch.float32, "residual")
    n = grad.numel()
    if residual.numel() != n or residual.device != grad.device:
        raise ValueError("grad and residual must have the same length and device")
    dev = grad.device
    capacity = int(capacity)
    if capacity < 0:
        raise ValueError("capacity must be >= 0")
    if out_idx is None:
        out_idx = torch.empty(capacity, dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty(capacity, dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=dev)
    _require(out_idx, torch.int32, "out_idx", dev, capacity)
    _require(out_val, torch.float32, "out_val", dev, capacity)
    _require(count, torch.int64, "count", dev, 1)
    lib = _load()
    need = lib.tgs_threshold_workspace_bytes(n)
    if need == 0:
        raise ValueError("invalid size n=%d" % n)
    if ws is None:
        ws = workspace("threshold", need, dev)
    st = lib.tgs_threshold_ef_step(_ptr(grad), _ptr(residual), n, ctypes.c_float(lam), _ptr(out_idx),
                                   _ptr(out_val), capacity, count.data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream_handle(dev))
    _check(st, "tgs_threshold_ef_step")
    return out_idx, out_val, count


def threshold_estimate_workspace_bytes(m: int) -> int:
    return int(_load().tgs_threshold_estimate_workspace_bytes(m))


def threshold_estimate(grad: torch.Tensor, residual: torch.Tensor, sample_idx: torch.Tensor, q: int,
                       d_lambda: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """The q-th largest |residual + grad| over the positions ``sample_idx``
    (int32 device tensor), as a one-element float32 device tensor (no host
    round trip).  grad and residual are only read."""
    _require(grad, torch.float32, "grad")
    dev = grad.device
    _require(residual, torch.float32, "residual", dev, grad.numel())
    _require(sample_idx, torch.int32, "sample_idx", dev)
    n, m = grad.numel(), sample_idx.numel()
    if residual.numel() != n:
        raise ValueError("grad and residual must have the same length")
    if d_lambda is None:
        d_lambda = torch.empty(1, dtype=torch.float32, device=dev)
    _require(d_lambda, torch.float32, "d_lambda", dev, 1)
    lib = _load()
    need = lib.tgs_threshold_estimate_workspace_bytes(m)
    if need == 0:
        raise ValueError("invalid sample count m=%d" % m)
    if ws is None:
        ws = workspace("estimate", need, dev)
    st = lib.tgs_threshold_estimate(_ptr(grad), _ptr(residual), n, _ptr(sample_idx), m, int(q), d_lambda.data_ptr(),
                                    ws.data_ptr(), ws.numel(), _stream_handle(dev))
    _check(st, "tgs_threshold_estimate")
    return d_lambda


def threshold_ef_step_dev(grad: torch.Tensor, residual: torch.Tensor, d_lambda: torch.Tensor, capacity: int,
                          out_idx=None, out_val=None, count=None, ws: torch.Tensor | None = None):
    """``threshold_ef_step`` with the threshold in device memory (a
    one-element float32 tensor, read when the kernels run)."""
    _require(grad, torch.float32, "grad")
    dev = grad.device
    _require(residual, torch.float32, "residual", dev)
    _require(d_lambda, torch.float32, "d_lambda", dev, 1)
    n = grad.numel()
    if residual.numel() != n:
        raise ValueError("grad and residual must have the same length")
    capacity = int(capacity)
    if capacity < 0:
        raise ValueError("capacity must be >= 0")
    if out_idx is None:
        out_idx = torch.empty(capacity, dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty(capacity, dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=dev)
    _require(out_idx, torch.int32, "out_idx", dev, capacity)
    _require(out_val, torch.float32, "out_val", dev, capacity)
    _require(count, torch.int64, "count", dev, 1)
    lib = _load()
    need = lib.tgs_threshold_workspace_bytes(n)
    if need == 0:
        raise ValueError("invalid size n=%d" % n)
    if ws is None:
        ws = workspace("threshold", need, dev)
    st = lib.tgs_threshold_ef_step_dev(_ptr(grad), _ptr(residual), n, d_lambda.data_ptr(), _ptr(out_idx),
                                       _ptr(out_val), capacity, count.data_ptr(), ws.data_ptr(), ws.numel(),
                                       _stream_handle(dev))
    _check(st, "tgs_threshold_ef_step_dev")
    return out_idx, out_val, count


def estimated_threshold_ef_step(grad: torch.Tensor, residual: torch.Tensor, sample_idx: torch.Tensor, q: int,
                                capacity: int, out_idx=None, out_val=None, count=None, d_lambda=None,
                                ws: torch.Tensor | None = None):
    """The sampled estimate, then the hard-threshold step with it, both on
    the current stream with no host round trip.  Returns ``(idx, val, count,
    d_lambda)`` (device tensors).  ``ws``, if given, must be large enough for
    both calls."""
    n, m = grad.numel(), sample_idx.numel()
    if ws is None:
        need = max(threshold_estimate_workspace_bytes(m), threshold_workspace_bytes(n))
        ws = workspace("threshold", need, grad.device)
    d_lambda = threshold_estimate(grad, residual, sample_idx, q, d_lambda=d_lambda, ws=ws)
    idx, val, cnt = threshold_ef_step_dev(grad, residual, d_lambda, capacity, out_idx=out_idx, out_val=out_val,
                                          count=count, ws=ws)
    return idx, val, cnt, d_lambda


def rtopk_workspace_bytes(n: int, r: int, k: int) -> int:
    return int(_load().tgs_rtopk_workspace_bytes(n, r, k))


def rtopk_ef_step(grad: torch.Tensor, residual: torch.Tensor, r: int, k: int, seed: int, step: int,
                  out_idx=None, out_val=None, ws: torch.Tensor | None = None):
    """One rTop-k step: k entries drawn at random (Philox4x32-10 keyed by
    ``seed``, counter by entry index and ``step``) from the top r of
    |residual + grad|.  ``residual`` is updated in place.  Returns ``(idx
    int32[k], val float32[k])`` in (|acc| desc, index asc) order."""
    _require(grad, torch.float32, "grad")
    dev = grad.device
    _require(residual, torch.float32, "residual", dev)
    n = grad.numel()
    if residual.numel() != n:
        raise ValueError("grad and residual must have the same length")
    r, k = int(r), int(k)
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty(k, dtype=torch.float32, device=dev)
    _require(out_idx, torch.int32, "out_idx", dev, k)
    _require(out_val, torch.float32, "out_val", dev, k)
    lib = _load()
    need = lib.tgs_rtopk_workspace_bytes(n, r, k)
    if need == 0:
        raise ValueError("invalid sizes n=%d r=%d k=%d" % (n, r, k))
    if ws is None:
        ws = workspace("rtopk", need, dev)
    st = lib.tgs_rtopk_ef_step(_ptr(grad), _ptr(residual), n, r, k, int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
                               _ptr(out_idx), _ptr(out_val), ws.data_ptr(), ws.numel(), _stream_handle(dev))
    _check(st, "tgs_rtopk_ef_step")
    return out_idx[:k], out_val[:k]


def gtopk_workspace_bytes(P: int, k: int, n: int) -> int:
    return int(_load().tgs_gtopk_workspace_bytes(P, k, n))


def gtopk_merge(idx: torch.Tensor, val: torch.Tensor, n: int, ws: torch.Tensor | None = None,
                check: bool = False):
    """gTop-k tournament of the P rows of ``idx``/``val`` (shape [P, k]).

    Returns ``(gidx int32[k], gval float32[k], mask uint8[P, k])``,
    asynchronously.  With ``check`` the call also waits for the device and
    raises ValueError if a row broke the index precondition (distinct indices
    inside [0, n)); otherwise ``check_device_error(ws)`` reports it later."""
    _require(idx, torch.int32, "idx")
    _require(val, torch.float32, "val")
    if idx.dim() != 2 or idx.shape != val.shape:
        raise ValueError("idx and val must both have shape [P, k]")
    P, k = idx.shape
    dev = idx.device
    out_idx = torch.empty(k, dtype=torch.int32, device=dev)
    out_val = torch.empty(k, dtype=torch.float32, device=dev)
    mask = torch.empty((P, k), dtype=torch.uint8, device=dev)
    lib = _load()
    need = lib.tgs_gtopk_workspace_bytes(P, k, n)
    if need == 0:
        raise ValueError("invalid sizes P=%d k=%d n=%d" % (P, k, n))
    if ws is None:
        ws = workspace("gtopk", need, dev)
    st = lib.tgs_gtopk_merge(_ptr(idx), _ptr(val), P, k, n, _ptr(out_idx), _ptr(out_val), _ptr(mask),
                             ws.data_ptr(), ws.numel(), _stream_handle(dev))
    _check(st, "tgs_gtopk_merge")
    if check:
        _check(lib.tgs_check_device_error(ws.data_ptr(), _stream_handle(dev)), "tgs_gtopk_merge (device)")
    return out_idx, out_val, mask


def check_device_error(ws: torch.Tensor):
    """Waits for the current stream, then reads and clears the workspace's
    device error word: raises ValueError for bad merge input, TgsError for a
    wait timeout or inconsistent counts."""
    lib = _load()
    _check(lib.tgs_check_device_error(ws.data_ptr(), _stream_handle(ws.device)), "tgs_check_device_error")


def set_option(option: int, value: int):
    _check(_load().tgs_set_option(option, value), "tgs_set_option")


def profile_next_call(start_event, stop_event):
    """The next topk/threshold call records these torch.cuda.Events around its
    streaming pass (on its stream)."""
    lib = _load()
    for ev in (start_event, stop_event):
        if ev is not None and not ev.cuda_event:
            ev.record()  # torch creates the HIP event lazily, on its first record
    s = start_event.cuda_event if start_event is not None else None
    e = stop_event.cuda_event if stop_event is not None else None
    _check(lib.tgs_profile_next_call(s, e), "tgs_profile_next_call")


def profile_elapsed_ms(start_event, stop_event) -> float:
    """Milliseconds between two events recorded by the library."""
    ms = ctypes.c_float()
    _check(_load().tgs_profile_elapsed_ms(start_event.cuda_event, stop_event.cuda_event, ctypes.byref(ms)),
           "tgs_profile_elapsed_ms")
    return ms.value


__all__ = [
    "TopkStep", "TopkSegments", "topk_ef_step", "topk_ef_step_segmented", "threshold_ef_step", "gtopk_merge",
    "topk_workspace_bytes", "topk_segmented_workspace_bytes", "threshold_workspace_bytes",
    "gtopk_workspace_bytes", "check_device_error", "error_word", "workspace_init", "set_option",
    "threshold_estimate", "threshold_estimate_workspace_bytes", "threshold_ef_step_dev",
    "estimated_threshold_ef_step", "rtopk_ef_step", "rtopk_workspace_bytes",
    "profile_next_call", "profile_elapsed_ms", "library", "workspace",
    "TgsError", "OPT_TOPK_PATH", "OPT_MAIN_GRID", "LIB_PATH",
]
