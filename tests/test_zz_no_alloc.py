"""The allocation-free top-k entry point, through the C ABI: its results equal
tgs_topk_ef_step's bit for bit (indices, values, residual) on calls in a row,
the later ones on smaller inputs, and once the device's first call has looked
up the library's device array (the runtime maps it then), no call takes
device memory."""
import ctypes

import numpy as np
import pytest
import torch

from _helpers import bits, gpu, host
from top_gradient_sparsification_amd import workloads

pytestmark = pytest.mark.gpu


def _noalloc(tgs):
    lib = tgs.library()
    fn = lib.tgs_topk_ef_step_noalloc
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    return fn


def _both(tgs, fn, grad, res, k, check_memory=True):
    """(regular, allocation-free) results on identical device copies."""
    n = grad.size
    stream = torch.cuda.current_stream().cuda_stream
    # the regular entry point, on its own workspace
    g1, r1 = gpu(grad), gpu(res)
    ws = torch.zeros(tgs.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    i1 = torch.empty(k, dtype=torch.int32, device="cuda")
    v1 = torch.empty(k, dtype=torch.float32, device="cuda")
    st = tgs.library().tgs_topk_ef_step(g1.data_ptr(), r1.data_ptr(), n, k, i1.data_ptr(), v1.data_ptr(),
                                        ws.data_ptr(), ws.numel(), stream)
    assert st == 0
    tgs.check_device_error(ws)
    # the allocation-free one: inputs and outputs allocated before the call
    g2, r2 = gpu(grad), gpu(res)
    i2 = torch.empty(k, dtype=torch.int32, device="cuda")
    v2 = torch.empty(k, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    st = fn(g2.data_ptr(), r2.data_ptr(), n, k, i2.data_ptr(), v2.data_ptr(), stream)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert st == 0, tgs.library().tgs_last_error()
    if check_memory:
        assert free0 - free1 < (1 << 20), "the call took device memory"
    return (host(i1), host(v1), host(r1)), (host(i2), host(v2), host(r2))


def _same(a, b, what):
    assert np.array_equal(a[0], b[0]), what + ": indices"
    assert np.array_equal(bits(a[1]), bits(b[1])), what + ": values"
    assert np.array_equal(bits(a[2]), bits(b[2])), what + ": residual"


def test_noalloc_matches_the_workspace_entry_point(tgs_gpu):
    fn = _noalloc(tgs_gpu)
    # call 1: the ResNet-50-sized mixture at 0.1% (the single-launch step)
    n = 25_600_000
    k = workloads.k_for_density(n, 0.001)
    grad = workloads.grad_resnet50(1, variant=41)
    res = workloads.grad_resnet50(2, variant=41)
    reg, na = _both(tgs_gpu, fn, grad, res, k, check_memory=False)  # this device's first call may be its set-up
    _same(reg, na, "n=25.6M")
    # call 2, right after on the same array: a smaller vector (k_small route)
    rng = np.random.default_rng(41)
    n2, k2 = 100_000, 100
    grad2 = rng.standard_normal(n2).astype(np.float32)
    res2 = rng.standard_normal(n2).astype(np.float32)
    reg, na = _both(tgs_gpu, fn, grad2, res2, k2)
    _same(reg, na, "n=100,000")
    # call 3: 1,048,576 entries (single-launch step again, smaller grid share)
    grad3 = workloads.grad_small(1)
    reg, na = _both(tgs_gpu, fn, grad3, np.zeros(grad3.size, np.float32), 1048)
    _same(reg, na, "n=1,048,576")


def test_noalloc_rejects_sizes_beyond_its_array(tgs_gpu):
    fn = _noalloc(tgs_gpu)
    lib = tgs_gpu.library()
    n, k = 200_000_000, 2_000_000  # workspace far above 64 MiB
    assert tgs_gpu.topk_workspace_bytes(n, k) > (64 << 20)
    dummy = ctypes.c_void_p(0x100000)
    st = fn(dummy, ctypes.c_void_p(0x100000 + 4 * n), n, k, ctypes.c_void_p(0x100000 + 8 * n),
            ctypes.c_void_p(0x100000 + 12 * n), None)
    assert st == -1 and b"device array" in lib.tgs_last_error()
    st = fn(None, None, 10, 1, None, None, None)  # null pointers: rejected before any launch
    assert st == -1
