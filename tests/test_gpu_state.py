"""GPU tests of what a top-k call leaves behind in its workspace.

The library keeps no state on the host: a workspace made ready once
(tgs_workspace_init, or zero-filled) stays ready across any sequence of calls,
including calls captured in a HIP graph and replayed.  Each case is compared
bit for bit with the oracle, with the device error word read after every step.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import assert_topk_equal, gpu, host
from top_gradient_sparsification_amd import workloads

pytestmark = pytest.mark.gpu

N_C2 = 25_600_000


def _words(ws):
    """(verdict, fallbacks, parity) of a top-k workspace's control block."""
    w = host(ws[:36].view(torch.int32))
    return int(w[2]), int(w[3]), int(w[8])


def test_garbage_workspace_after_init_three_chained_steps(tgs_gpu):
    """ResNet-50-sized mixture, 0.1%: a workspace filled with 0xA5 bytes, made
    ready by tgs_workspace_init, then three chained EF steps on it."""
    n, k = N_C2, workloads.k_for_density(N_C2, 0.001)
    ws = torch.full((tgs_gpu.topk_workspace_bytes(n, k),), 0xA5, dtype=torch.uint8, device="cuda")
    tgs_gpu.workspace_init(ws)
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    parities = []
    for step in (1, 2, 3):
        g = workloads.grad_resnet50(step, variant=11)
        idx, val = tgs_gpu.topk_ef_step(gpu(g), r_gpu, k, ws=ws)
        tgs_gpu.check_device_error(ws)
        ei, ev = oracle.topk_ef_step(g, r_cpu, k)
        assert_topk_equal((host(idx), host(val), host(r_gpu)), (ei, ev, r_cpu), "step %d" % step)
        verdict, fallbacks, parity = _words(ws)
        assert verdict == 1 and fallbacks == 0, "the single-launch plan held"
        parities.append(parity)
    assert parities == [1, 0, 1], "each launch flips the counter-set parity on the device"


def test_graph_captured_step_replayed_on_fresh_gradients(tgs_gpu):
    """One tgs_topk_ef_step captured with torch.cuda.graph, replayed three
    times with a fresh gradient copied in before each replay (eager work and
    synchronisation between replays); every replay against the oracle's chain."""
    n, k = N_C2, workloads.k_for_density(N_C2, 0.001)
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    g_static = torch.empty(n, dtype=torch.float32, device="cuda")
    r_static = torch.zeros(n, dtype=torch.float32, device="cuda")
    oi = torch.empty(k, dtype=torch.int32, device="cuda")
    ov = torch.empty(k, dtype=torch.float32, device="cuda")
    # an eager call first (device properties are read once, outside capture)
    scratch_g = torch.ones(n, dtype=torch.float32, device="cuda")
    scratch_r = torch.zeros(n, dtype=torch.float32, device="cuda")
    tgs_gpu.topk_ef_step(scratch_g, scratch_r, k, out_idx=oi, out_val=ov, ws=ws)
    tgs_gpu.check_device_error(ws)
    del scratch_g, scratch_r
    torch.cuda.synchronize()
    fb0 = _words(ws)[1]  # (all-equal values: that call's plan could not hold)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tgs_gpu.topk_ef_step(g_static, r_static, k, out_idx=oi, out_val=ov, ws=ws)
    torch.cuda.synchronize()
    r_cpu = np.zeros(n, np.float32)
    for step in (1, 2, 3):
        g = workloads.grad_resnet50(step, variant=12)
        g_static.copy_(torch.from_numpy(g))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        tgs_gpu.check_device_error(ws)
        ei, ev = oracle.topk_ef_step(g, r_cpu, k)
        assert_topk_equal((host(oi), host(ov), host(r_static)), (ei, ev, r_cpu), "replay %d" % step)
        verdict, fallbacks, _ = _words(ws)
        assert verdict == 1 and fallbacks == fb0, "every replay took the single-launch plan"
    del graph


def test_error_word_is_sticky_until_read(tgs_gpu):
    """A flag set by one call survives the calls after it on the same
    workspace (the top-k launches only set bits) until check_device_error
    reads and clears it."""
    n, k = 1 << 20, 1048
    need = max(tgs_gpu.topk_workspace_bytes(n, k), tgs_gpu.gtopk_workspace_bytes(2, 3, 10))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    bad_idx = gpu(np.array([[1, 1, 2], [3, 4, 5]], np.int32))
    tgs_gpu.gtopk_merge(bad_idx, gpu(np.ones((2, 3), np.float32)), 10, ws=ws)
    g = workloads.grad_small(1)
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    tgs_gpu.topk_ef_step(gpu(g), r, k, ws=ws)          # k_step
    tgs_gpu.topk_ef_step(gpu(g[:5000]), r[:5000], 7, ws=ws)  # k_small
    assert int(host(tgs_gpu.error_word(ws))[0]) == 1
    with pytest.raises(ValueError):
        tgs_gpu.check_device_error(ws)
    assert int(host(tgs_gpu.error_word(ws))[0]) == 0
    tgs_gpu.topk_ef_step(gpu(g), r, k, ws=ws)
    tgs_gpu.check_device_error(ws)


def test_prepared_calls_validate_their_tensors(tgs_gpu):
    n, k = 1 << 20, 1048
    step = tgs_gpu.TopkStep(n, k)
    g = torch.zeros(n, dtype=torch.float32, device="cuda")
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        step(g.half().repeat(2)[:n], r)          # right length, wrong dtype
    with pytest.raises(ValueError):
        step(torch.zeros(2 * n, device="cuda")[::2], r)  # right length, not contiguous
    with pytest.raises(ValueError):
        step(g[: n - 1], r[: n - 1])
    with pytest.raises(TypeError):
        step(g.cpu(), r)
    step(g, r)
    step.check()
    seg = tgs_gpu.TopkSegments([0, 1000, n], [1, 1000])
    with pytest.raises(ValueError):
        seg(torch.zeros(2 * n, device="cuda")[::2], r)
    with pytest.raises(ValueError):
        tgs_gpu.threshold_ef_step(g, r, 0.5, 16, out_idx=torch.empty(8, dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        tgs_gpu.threshold_ef_step(g, r, 0.5, 16, count=torch.empty(1, dtype=torch.int32, device="cuda"))
