"""CPU oracle for the error-feedback top-k sparsifier -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it never imports them: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, sequential, full sorts); this
module only compiles it with gcc and marshals numpy arrays through ctypes.
Every routine follows a definition from the pages, cited in ``oracle.c``:

* ``topk_ef_step``      -- error feedback plus top-k by magnitude
  (arxivdaily listing for arXiv 2004.05298, entries "Sparsified SGD with
  Memory" and "The Convergence of Sparsified Gradient Methods").
* ``threshold_ef_step`` -- hard-threshold sparsifier with error feedback
  (same listing, entry "Rethinking gradient sparsification as total error
  minimization").
* ``gtopk_merge``       -- the O(log P) tournament of the nubint review "A
  Distributed Synchronous SGD Algorithm with Global Top-k Sparsification for
  Low Bandwidth Networks" (ABSTRACT, Method).
* ``threshold_estimate`` / ``estimated_threshold_ef_step`` -- a threshold
  estimated from a sample in place of the sort (arxivdaily listing, entry
  "Near-Optimal Sparse Allreduce for Distributed Deep Learning"; fugumt page
  for arXiv 2502.07634, related-paper entry "An Efficient Statistical-based
  Gradient Compression Technique for Distributed Training Systems"), feeding
  the hard threshold.
* ``rtopk_ef_step``     -- random k of the top r (arxivdaily listing, entry
  "rTop-k: A Statistical Estimation Approach to Distributed SGD"), with the
  Philox4x32-10 generator (``philox4x32_10``; Salmon et al., SC'11).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -O2 without fast-math; -ffp-contract=off keeps every add a plain binary32 add.
GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-msse2", "-mfpmath=sse"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.oracle_topk_ef_step.argtypes = [vp, vp, i64, i64, vp, vp]
        lib.oracle_topk_ef_step.restype = ctypes.c_int
        lib.oracle_threshold_ef_step.argtypes = [vp, vp, i64, ctypes.c_float, vp, vp, i64]
        lib.oracle_threshold_ef_step.restype = i64
        lib.oracle_gtopk_merge.argtypes = [vp, vp, i32, i64, i64, vp, vp, vp, vp]
        lib.oracle_gtopk_merge.restype = ctypes.c_int
        lib.oracle_fp_mode_inside_call.argtypes = []
        lib.oracle_fp_mode_inside_call.restype = ctypes.c_uint
        u32, u64 = ctypes.c_uint32, ctypes.c_uint64
        lib.oracle_threshold_ef_step_key.argtypes = [vp, vp, i64, u32, vp, vp, i64]
        lib.oracle_threshold_ef_step_key.restype = i64
        lib.oracle_threshold_estimate.argtypes = [vp, vp, i64, vp, i64, i64, ctypes.POINTER(u32)]
        lib.oracle_threshold_estimate.restype = ctypes.c_int
        lib.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_rtopk_ef_step.argtypes = [vp, vp, i64, i64, i64, u64, u64, vp, vp]
        lib.oracle_rtopk_ef_step.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("expected float32, got %s" % a.dtype)
    return a


def topk_ef_step(grad: np.ndarray, residual: np.ndarray, k: int):
    """One error-feedback top-k step.  ``residual`` is updated in place.

    Returns ``(idx int32[k], val float32[k])`` in (|acc| desc, index asc) order.
    """
    grad = _f32(grad)
    if not (residual.dtype == np.float32 and residual.flags.c_contiguous):
        raise TypeError("residual must be a contiguous float32 array (updated in place)")
    n = grad.size
    if residual.size != n:
        raise ValueError("grad and residual differ in length")
    out_idx = np.empty(k, dtype=np.int32)
    out_val = np.empty(k, dtype=np.float32)
    rc = _load().oracle_topk_ef_step(_ptr(grad), _ptr(residual), n, k, _ptr(out_idx), _ptr(out_val))
    if rc != 0:
        raise ValueError("oracle_topk_ef_step failed (%d)" % rc)
    return out_idx, out_val


def threshold_ef_step(grad: np.ndarray, residual: np.ndarray, lam: float, capacity: int):
    """One hard-threshold step.  Returns ``(idx, val, count)``; idx/val hold the
    first ``min(count, capacity)`` qualifying entries in ascending index order."""
    grad = _f32(grad)
    if not (residual.dtype == np.float32 and residual.flags.c_contiguous):
        raise TypeError("residual must be a contiguous float32 array (updated in place)")
    n = grad.size
    if residual.size != n:
        raise ValueError("grad and residual differ in length")
    out_idx = np.empty(max(capacity, 0), dtype=np.int32)
    out_val = np.empty(max(capacity, 0), dtype=np.float32)
    count = _load().oracle_threshold_ef_step(_ptr(grad), _ptr(residual), n, ctypes.c_float(lam),
                                             _ptr(out_idx), _ptr(out_val), capacity)
    if count < 0:
        raise ValueError("oracle_threshold_ef_step rejected its input")
    m = min(count, capacity)
    return out_idx[:m].copy(), out_val[:m].copy(), int(count)


def gtopk_merge(idx: np.ndarray, val: np.ndarray, n: int, return_rounds: bool = False):
    """Tournament merge of P sparse sets (rows of ``idx``/``val``, shape [P, k]).

    Returns ``(gidx int32[k], gval float32[k], mask uint8[P, k])`` and, if asked,
    the number of pairwise rounds played."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    val = _f32(val)
    if idx.ndim != 2 or idx.shape != val.shape:
        raise ValueError("idx and val must both have shape [P, k]")
    P, k = idx.shape
    out_idx = np.empty(k, dtype=np.int32)
    out_val = np.empty(k, dtype=np.float32)
    mask = np.empty((P, k), dtype=np.uint8)
    rounds = ctypes.c_int32(-1)
    rc = _load().oracle_gtopk_merge(_ptr(idx), _ptr(val), P, k, n, _ptr(out_idx), _ptr(out_val),
                                    _ptr(mask), ctypes.byref(rounds))
    if rc != 0:
        raise ValueError("oracle_gtopk_merge rejected its input (%d)" % rc)
    if return_rounds:
        return out_idx, out_val, mask, rounds.value
    return out_idx, out_val, mask


def threshold_ef_step_key(grad: np.ndarray, residual: np.ndarray, key: int, capacity: int):
    """``threshold_ef_step`` with the threshold given as its magnitude key
    (an integer in [0, 0x7FFFFFFF])."""
    grad = _f32(grad)
    if not (residual.dtype == np.float32 and residual.flags.c_contiguous):
        raise TypeError("residual must be a contiguous float32 array (updated in place)")
    n = grad.size
    if residual.size != n:
        raise ValueError("grad and residual differ in length")
    out_idx = np.empty(max(capacity, 0), dtype=np.int32)
    out_val = np.empty(max(capacity, 0), dtype=np.float32)
    count = _load().oracle_threshold_ef_step_key(_ptr(grad), _ptr(residual), n, int(key), _ptr(out_idx),
                                                 _ptr(out_val), capacity)
    if count < 0:
        raise ValueError("oracle_threshold_ef_step_key rejected its input")
    m = min(count, capacity)
    return out_idx[:m].copy(), out_val[:m].copy(), int(count)


def threshold_estimate(grad: np.ndarray, residual: np.ndarray, sample_idx: np.ndarray, q: int) -> int:
    """The q-th largest magnitude key of acc = residual + grad over the
    positions ``sample_idx`` (int32, repeats allowed).  Reads only."""
    grad = _f32(grad)
    residual = _f32(residual)
    sample_idx = np.ascontiguousarray(sample_idx, dtype=np.int32)
    key = ctypes.c_uint32()
    rc = _load().oracle_threshold_estimate(_ptr(grad), _ptr(residual), grad.size, _ptr(sample_idx),
                                           sample_idx.size, q, ctypes.byref(key))
    if rc != 0:
        raise ValueError("oracle_threshold_estimate rejected its input (%d)" % rc)
    return int(key.value)


def estimated_threshold_ef_step(grad: np.ndarray, residual: np.ndarray, sample_idx: np.ndarray, q: int,
                                capacity: int):
    """The estimate, then the hard-threshold step with it.  Returns
    ``(idx, val, count, key)``; ``residual`` is updated in place."""
    key = threshold_estimate(grad, residual, sample_idx, q)
    idx, val, count = threshold_ef_step_key(grad, residual, key, capacity)
    return idx, val, count, key


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of the 4-word counter under the 2-word key (uint32[4])."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    if c.size != 4 or k.size != 2:
        raise ValueError("counter has 4 words, key 2")
    out = np.empty(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def rtopk_ef_step(grad: np.ndarray, residual: np.ndarray, r: int, k: int, seed: int, step: int):
    """One rTop-k step with error feedback: k random entries of the top r.
    ``residual`` is updated in place.  Returns ``(idx int32[k], val
    float32[k])`` in (|acc| desc, index asc) order."""
    grad = _f32(grad)
    if not (residual.dtype == np.float32 and residual.flags.c_contiguous):
        raise TypeError("residual must be a contiguous float32 array (updated in place)")
    n = grad.size
    if residual.size != n:
        raise ValueError("grad and residual differ in length")
    out_idx = np.empty(k, dtype=np.int32)
    out_val = np.empty(k, dtype=np.float32)
    rc = _load().oracle_rtopk_ef_step(_ptr(grad), _ptr(residual), n, r, k, seed & (2**64 - 1), step & (2**64 - 1),
                                      _ptr(out_idx), _ptr(out_val))
    if rc != 0:
        raise ValueError("oracle_rtopk_ef_step rejected its input (%d)" % rc)
    return out_idx, out_val


def fp_mode_inside_call() -> int:
    """MXCSR FTZ|DAZ|rounding bits as seen inside an oracle call (expected 0)."""
    return int(_load().oracle_fp_mode_inside_call())
