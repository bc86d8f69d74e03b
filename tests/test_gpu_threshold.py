"""GPU parity of tgs_threshold_ef_step against the CPU oracle (bit for bit)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from _helpers import bits, gpu, host, keys
from top_gradient_sparsification_amd import workloads

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_thr(tgs, grad, res, lam, cap):
    g, r = gpu(grad), gpu(res)
    idx, val, cnt = tgs.threshold_ef_step(g, r, lam, cap)
    c = int(host(cnt)[0])
    m = min(c, cap)
    return host(idx)[:m], host(val)[:m], c, host(r)


def oracle_thr(grad, res, lam, cap):
    r = res.copy()
    i, v, c = oracle.threshold_ef_step(grad, r, lam, cap)
    return i, v, c, r


def assert_thr_equal(got, exp, what):
    gi, gv, gc, gr = got
    ei, ev, ec, er = exp
    assert gc == ec, "%s: count %d vs %d" % (what, gc, ec)
    assert np.array_equal(gi, ei), what + ": indices differ"
    assert np.array_equal(bits(gv), bits(ev)), what + ": values differ"
    bad = np.nonzero(bits(gr) != bits(er))[0]
    assert bad.size == 0, "%s: %d residual mismatches, first at %d" % (what, bad.size, bad[0])


def test_golden(tgs_gpu):
    g = json.load(open(os.path.join(GOLDEN, "threshold_ties.json")))
    for case in g["cases"]:
        got = gpu_thr(tgs_gpu, np.float32(g["grad"]), np.float32(g["residual"]), case["lambda"], case["capacity"])
        assert got[2] == case["count"]
        assert got[0].tolist() == case["idx"]
        assert np.array_equal(bits(got[1]), bits(case["val"]))
        assert np.array_equal(bits(got[3]), bits(case["residual_after"]))


@pytest.mark.parametrize("n", [1, 3, 64, 1000, 4097, 65536, 1_000_003])
def test_random_parity(tgs_gpu, n):
    rng = np.random.default_rng(n)
    grad = rng.standard_normal(n).astype(np.float32)
    res = (rng.integers(-4, 5, n) * 0.25).astype(np.float32)
    for lam in (0.0, 0.5, 1.0, 2.5, 1e30):
        for cap in (0, 1, n // 10, n):
            assert_thr_equal(gpu_thr(tgs_gpu, grad, res, lam, cap), oracle_thr(grad, res, lam, cap),
                             "n=%d lam=%g cap=%d" % (n, lam, cap))


def test_ties_at_lambda_and_special_values(tgs_gpu):
    rng = np.random.default_rng(2)
    n = 200_001
    grad = (rng.integers(-8, 9, n) * 0.25).astype(np.float32)
    res = np.zeros(n, np.float32)
    grad[::997] = np.nan
    grad[5::1001] = np.inf
    grad[7::1003] = -0.0
    grad[9::1009] = 1e-45
    for lam in (0.5, 1.0, 1.75, 1e-45, np.inf):
        for cap in (n, 1000):
            assert_thr_equal(gpu_thr(tgs_gpu, grad, res, lam, cap), oracle_thr(grad, res, lam, cap), "lam=%g" % lam)


def test_stash_overflow_rescan(tgs_gpu):
    """lambda = 0: every entry qualifies, so every wave's stash overflows and
    the emit pass rescans acc in index order."""
    rng = np.random.default_rng(3)
    n = 2_000_000
    grad = rng.standard_normal(n).astype(np.float32)
    res = rng.standard_normal(n).astype(np.float32)
    for cap in (n, n // 3, 12345):
        assert_thr_equal(gpu_thr(tgs_gpu, grad, res, 0.0, cap), oracle_thr(grad, res, 0.0, cap), "cap=%d" % cap)


@pytest.mark.parametrize("layout", ["dense", "clustered", "round_edge"])
def test_stash_overflow_positive_lambda(tgs_gpu, layout):
    """lambda > 0 with more qualifying entries than a stash holds: every wave
    (dense: 38% of N(0,1) has |x| >= 0.5) or only the waves whose rows fall in
    one index range (clustered; round_edge: a range across the boundary of the
    first two rounds of 4096 rows of 256 entries) overflow.  The pass has
    already set the stashed entries' residual to +0, so the rescan must skip
    them and number the rest from the stash's end, and stashed entries past
    the capacity must get acc back."""
    rng = np.random.default_rng(4)
    n = 2_000_003
    grad = rng.standard_normal(n).astype(np.float32)
    res = rng.standard_normal(n).astype(np.float32)
    lam = 0.5 if layout == "dense" else 4.0
    if layout == "clustered":
        grad[700_000:760_000] = rng.uniform(5.0, 6.0, 60_000).astype(np.float32)
    if layout == "round_edge":
        grad[1_000_000:1_100_000] = rng.uniform(5.0, 6.0, 100_000).astype(np.float32)
    exp_all = oracle_thr(grad, res, lam, n)
    c = exp_all[2]
    for cap in (n, c, c - 1, c // 3, 7, 0):
        assert_thr_equal(gpu_thr(tgs_gpu, grad, res, lam, cap), oracle_thr(grad, res, lam, cap),
                         "%s cap=%d" % (layout, cap))


@pytest.mark.parametrize("off_g,off_r", [(1, 1), (3, 3), (0, 2), (63, 63)])
def test_misaligned(tgs_gpu, off_g, off_r):
    """Offsets of 1 and 3 entries: a scalar head, slots off the 256-byte
    grid (stored with the streaming hint alone); 0 and 2: grad and residual
    unequally aligned (scalar slots); 63: a one-entry head after which the
    slots start on a 256-byte boundary (written through at device scope)."""
    rng = np.random.default_rng(10 + off_g + off_r)
    n = 500_001
    grad = rng.standard_normal(n).astype(np.float32)
    res = rng.standard_normal(n).astype(np.float32)
    gb = torch.zeros(n + 64, dtype=torch.float32, device="cuda")
    rb = torch.zeros(n + 64, dtype=torch.float32, device="cuda")
    gb[off_g:off_g + n] = gpu(grad)
    rb[off_r:off_r + n] = gpu(res)
    r = rb[off_r:off_r + n]
    idx, val, cnt = tgs_gpu.threshold_ef_step(gb[off_g:off_g + n], r, 2.0, n)
    c = int(host(cnt)[0])
    exp = oracle_thr(grad, res, 2.0, n)
    assert_thr_equal((host(idx)[:c], host(val)[:c], c, host(r)), exp, "offsets")


def test_large_config_reduced_n_exact(tgs_gpu):
    """The n = 1.5e9 workload's distribution at n = 50M, lambda = fl32(4e-3),
    capacity 2% of n, two chained steps against the oracle."""
    n = 50_000_000
    cap = n // 50
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    for step in (1, 2):
        g = workloads.mixture(n, 1e-3, 0.005, 0.05, (5, 7, step))
        idx, val, cnt = tgs_gpu.threshold_ef_step(gpu(g), r_gpu, 4e-3, cap)
        c = int(host(cnt)[0])
        ei, ev, ec = oracle.threshold_ef_step(g, r_cpu, 4e-3, cap)
        m = min(c, cap)
        assert_thr_equal((host(idx)[:m], host(val)[:m], c, host(r_gpu)), (ei, ev, ec, r_cpu), "step %d" % step)


def test_large_config_full_n(tgs_gpu):
    """n = 1.5e9 with capacity 2% of n, residual from 0 over two chained steps
    with fresh gradients (drawn on the GPU, copied to the host): each step
    against the oracle's, count, emitted pairs and residual bit for bit."""
    n = 1_500_000_000
    cap = n // 50
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    for step in (1, 2):
        g = workloads.mixture_gpu(n, 1e-3, 0.005, 0.05, (5, 0, step))
        grad_h = host(g)
        idx, val, cnt = tgs_gpu.threshold_ef_step(g, r, 4e-3, cap)
        c = int(host(cnt)[0])
        m = min(c, cap)
        idx_h, val_h = host(idx)[:m], host(val)[:m]
        del g, idx, val
        torch.cuda.empty_cache()
        ei, ev, ec = oracle.threshold_ef_step(grad_h, r_cpu, 4e-3, cap)
        del grad_h
        assert c == ec, "step %d count" % step
        assert np.array_equal(idx_h, ei) and np.array_equal(bits(val_h), bits(ev)), "step %d pairs" % step
        bad = np.nonzero(bits(host(r)) != bits(r_cpu))[0]
        assert bad.size == 0, "step %d: %d residual mismatches" % (step, bad.size)
