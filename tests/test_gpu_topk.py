"""GPU parity of tgs_topk_ef_step against the CPU oracle (bit for bit).

Covers every path of the library: the general exact path (small n, large k,
forced), the sampled fast path, its on-device fallback (forced with a plan
that cannot hold), vector and scalar streaming (aligned, misaligned, unequal
alignment), the three configurations' shapes and the edge cases.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from _helpers import assert_topk_equal, bits, check_topk_invariants, gpu, gpu_topk, host, keys, topk_dev
from top_gradient_sparsification_amd import workloads

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def oracle_topk(grad, res, k):
    r = res.copy()
    i, v = oracle.topk_ef_step(grad, r, k)
    return i, v, r


@pytest.fixture(autouse=True)
def reset_options(tgs_gpu):
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, 0)
    tgs_gpu.set_option(tgs_gpu.OPT_MAIN_GRID, 0)
    yield
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, 0)
    tgs_gpu.set_option(tgs_gpu.OPT_MAIN_GRID, 0)


def make(dist, n, rng):
    if dist == "normal":
        return rng.standard_normal(n).astype(np.float32), rng.standard_normal(n).astype(np.float32)
    if dist == "ties":
        return (rng.integers(-4, 5, n) * 0.5).astype(np.float32), (rng.integers(-2, 3, n) * 0.25).astype(np.float32)
    if dist == "special":
        g = rng.standard_normal(n).astype(np.float32)
        r = np.zeros(n, np.float32)
        pick = rng.integers(0, n, max(1, n // 50))
        g[pick] = rng.choice(np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45, 3e-39], np.float32),
                             pick.size)
        return g, r
    if dist == "mixture":
        g = workloads.mixture(n, 1e-3, 0.01, 0.1, (77, n, 1))
        r = workloads.mixture(n, 1e-3, 0.01, 0.1, (77, n, 2))
        return g, r
    raise ValueError(dist)


def test_golden_fixtures(tgs_gpu):
    g = json.load(open(os.path.join(GOLDEN, "topk_ef_ties.json")))
    for case in g["cases"]:
        got = gpu_topk(tgs_gpu, np.float32(g["grad"]), np.float32(g["residual"]), case["k"])
        assert got[0].tolist() == case["idx"]
        assert np.array_equal(bits(got[1]), bits(case["val"]))
        assert np.array_equal(bits(got[2]), bits(case["residual_after"]))
    g = json.load(open(os.path.join(GOLDEN, "topk_ef_two_steps.json")))
    r = gpu(np.float32(g["residual0"]))
    for st in g["steps"]:
        idx, val = tgs_gpu.topk_ef_step(gpu(np.float32(st["grad"])), r, g["k"])
        assert host(idx).tolist() == st["idx"]
        assert np.array_equal(bits(host(val)), bits(st["val"]))
        assert np.array_equal(bits(host(r)), bits(st["residual_after"]))
    g = json.load(open(os.path.join(GOLDEN, "acc_rounding.json")))
    res = np.array([int(h, 16) for h in g["residual_bits"]], np.uint32).view(np.float32)
    grad = np.array([int(h, 16) for h in g["grad_bits"]], np.uint32).view(np.float32)
    got = gpu_topk(tgs_gpu, grad, res, g["k"])
    assert got[0].tolist() == g["idx"]
    assert [int(b) for b in bits(got[1])] == [int(h, 16) for h in g["val_bits"]]


@pytest.mark.parametrize("dist", ["normal", "ties", "special"])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 63, 64, 65, 257, 1000, 4099, 65537, 70001])
def test_small_sizes_all_k(tgs_gpu, n, dist):
    rng = np.random.default_rng(n * 7 + len(dist))
    grad, res = make(dist, n, rng)
    for k in sorted({0, 1, n // 7, n // 2, n - 1, n}):
        if k < 0:
            continue
        assert_topk_equal(gpu_topk(tgs_gpu, grad, res, k), oracle_topk(grad, res, k), "n=%d k=%d %s" % (n, k, dist))


@pytest.mark.parametrize("dist", ["normal", "mixture", "ties"])
@pytest.mark.parametrize("n,ks", [(65536, [1, 64, 8192]), (100_003, [17, 1000, 12_500]),
                                  (524_365, [2, 524, 5000]), (1 << 20, [1, 1048, 49_152, 131_072]),
                                  (3_000_001, [3, 3000, 30_000])])
def test_fast_path_sizes(tgs_gpu, n, ks, dist):
    rng = np.random.default_rng(n + 3 * len(dist))
    grad, res = make(dist, n, rng)
    for k in ks:
        assert_topk_equal(gpu_topk(tgs_gpu, grad, res, k), oracle_topk(grad, res, k), "n=%d k=%d %s" % (n, k, dist))


@pytest.mark.parametrize("path", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("dist", ["normal", "ties", "special"])
def test_forced_general_and_fallback(tgs_gpu, path, dist):
    """path 1: the exact general path only; 2: fast path whose plan cannot
    hold, so the on-device fallback produces the result; 3 and 4: fast path
    whose streaming workgroups must re-read their rows (no local list, or an
    overflowing one); 5: fast path whose workgroups cannot publish their
    candidates (fallback); 6: fast path with one slot per bucket and
    workgroup (candidates go through the overflow area)."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, path)
    rng = np.random.default_rng(31 + path)
    n = 1_000_003
    grad, res = make(dist, n, rng)
    for k in (1, 1048, 40_000):
        assert_topk_equal(gpu_topk(tgs_gpu, grad, res, k), oracle_topk(grad, res, k), "path=%d k=%d" % (path, k))


@pytest.mark.parametrize("layout", ["spread", "clustered", "crowded"])
def test_general_path_candidate_layouts(tgs_gpu, layout):
    """The standalone general path copies the entries of the threshold's
    first-level bin and above into one region per wave and selects among
    the copies.  Large entries bunched in one index range overflow the
    regions of the waves that hold them, and a value shared by half the
    vector is too many to copy at all: both must give the oracle's result
    through the route over the whole vector."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, 1)
    rng = np.random.default_rng({"spread": 5, "clustered": 6, "crowded": 7}[layout])
    n = 1_000_003
    grad = rng.normal(0.0, 1e-3, n).astype(np.float32)
    res = rng.normal(0.0, 1e-3, n).astype(np.float32)
    if layout == "clustered":
        grad[200_000:260_000] = rng.uniform(1.0, 2.0, 60_000).astype(np.float32)
    if layout == "crowded":
        grad[rng.random(n) < 0.5] = np.float32(0.5)
        res[:] = 0.0
    for k in (1, 1000, 40_000, 70_000):
        assert_topk_equal(gpu_topk(tgs_gpu, grad, res, k), oracle_topk(grad, res, k), "%s k=%d" % (layout, k))


def test_small_config_three_chained_steps(tgs_gpu):
    """n = 1,048,576, N(0,1) gradients, residual from 0, k = 1,048 (0.1%)."""
    n = 1_048_576
    k = workloads.k_for_density(n, 0.001)
    assert k == 1048
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    for step in (1, 2, 3):
        g = workloads.grad_small(step)
        got = topk_dev(tgs_gpu, gpu(g), r_gpu, k)
        ei, ev = oracle.topk_ef_step(g, r_cpu, k)
        assert_topk_equal(got, (ei, ev, r_cpu), "step %d" % step)


@pytest.mark.parametrize("off_g,off_r", [(1, 1), (2, 2), (3, 3), (0, 1), (1, 2), (3, 0)])
def test_misaligned_slices(tgs_gpu, off_g, off_r):
    """Slices starting at arbitrary 4-byte offsets (equal offsets keep the
    vector path with a scalar head; unequal ones take the scalar path)."""
    rng = np.random.default_rng(off_g * 4 + off_r)
    n = 300_007
    grad, res = make("normal", n, rng)
    for k in (0, 5, 300, 30_000):
        gb = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
        rb = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
        gb[off_g:off_g + n] = gpu(grad)
        rb[off_r:off_r + n] = gpu(res)
        g, r = gb[off_g:off_g + n], rb[off_r:off_r + n]
        got = topk_dev(tgs_gpu, g, r, k)
        exp = oracle_topk(grad, res, k)
        assert_topk_equal(got, exp, "offsets %d/%d k=%d" % (off_g, off_r, k))
        # nothing outside the slice was touched
        assert np.all(host(rb[:off_r]) == 0) and np.all(host(rb[off_r + n:]) == 0)


@pytest.mark.parametrize("grid", [1, 7, 64, 65, 100, 256, 2048])
def test_results_do_not_depend_on_grid(tgs_gpu, grid):
    rng = np.random.default_rng(5)
    n = 2_000_000
    grad, res = make("mixture", n, rng)
    exp = oracle_topk(grad, res, 2000)
    tgs_gpu.set_option(tgs_gpu.OPT_MAIN_GRID, grid)
    assert_topk_equal(gpu_topk(tgs_gpu, grad, res, 2000), exp, "grid=%d" % grid)
    assert_topk_equal(gpu_topk(tgs_gpu, grad, res, 2000), exp, "grid=%d repeat" % grid)


def test_edge_cases(tgs_gpu):
    # n = 0
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    idx, val = tgs_gpu.topk_ef_step(e, e.clone(), 0)
    assert idx.numel() == 0
    # k = n on a mid-size input (full sort by magnitude) and all-equal values
    rng = np.random.default_rng(8)
    for grad in (rng.standard_normal(70_001).astype(np.float32), np.full(70_001, -1.5, np.float32)):
        res = np.zeros_like(grad)
        assert_topk_equal(gpu_topk(tgs_gpu, grad, res, grad.size), oracle_topk(grad, res, grad.size), "k=n")
    # all-equal values on the fast-path shape: every bucket is one key
    grad = np.full(1 << 20, 0.25, np.float32)
    res = np.zeros_like(grad)
    assert_topk_equal(gpu_topk(tgs_gpu, grad, res, 1000), oracle_topk(grad, res, 1000), "all equal")


def test_invalid_arguments_raise(tgs_gpu):
    g = torch.zeros(10, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        tgs_gpu.topk_ef_step(g, g.clone(), 11)
    with pytest.raises(ValueError):
        tgs_gpu.topk_ef_step(g, g, 1)  # grad and residual overlap
    with pytest.raises(TypeError):
        tgs_gpu.topk_ef_step(g.double(), g.clone(), 1)


def _resnet_state(density, prior_steps=5):
    n = 25_600_000
    k = workloads.k_for_density(n, density)
    res = np.zeros(n, np.float32)
    for step in range(1, prior_steps + 1):
        oracle.topk_ef_step(workloads.grad_resnet50(step, variant=int(density * 1e5)), res, k)
    return n, k, res, workloads.grad_resnet50(prior_steps + 1, variant=int(density * 1e5))


@pytest.mark.parametrize("density", [0.001, 0.0002, 0.02])
def test_resnet50_sized_after_five_ef_steps(tgs_gpu, density):
    """n = 25.6M, 99% N(0,1e-3) + 1% Laplace(0,0.1), residual from 5 prior
    oracle EF steps at the same density; step 6 on the GPU vs the oracle."""
    n, k, res, grad = _resnet_state(density)
    exp = oracle_topk(grad, res, k)
    got = gpu_topk(tgs_gpu, grad, res, k)
    assert_topk_equal(got, exp, "density %g" % density)


def _vgg16_segments_oracle(grad, res, starts, sizes):
    """One oracle EF step per segment (residual updated in place); the pairs."""
    outs = []
    for s0, sz in zip(starts, sizes):
        r = res[s0:s0 + sz].copy()
        outs.append(oracle.topk_ef_step(grad[s0:s0 + sz], r, workloads.k_for_density(int(sz), 0.001)))
        res[s0:s0 + sz] = r
    return outs


def test_vgg16_sized_segments(tgs_gpu):
    """n = 138M in 32 log-uniform segments (1e3..1e8), per-segment 0.1% top-k.
    The residual starts at 0; step 1 is the oracle's, step 2 runs on the GPU
    (one call per contiguous slice, and all 32 in one layer-wise call) and is
    compared with the oracle's step 2, segment by segment."""
    n = 138_000_000
    sizes = workloads.segments_log_uniform(n)
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    res1 = np.zeros(n, np.float32)
    _vgg16_segments_oracle(workloads.grad_vgg16(1), res1, starts, sizes)
    grad = workloads.grad_vgg16(2)
    g_d, r_d = gpu(grad), gpu(res1)
    outs = []
    for s0, sz in zip(starts, sizes):
        k = workloads.k_for_density(int(sz), 0.001)
        i, v, _ = topk_dev(tgs_gpu, g_d[s0:s0 + sz], r_d[s0:s0 + sz], k)
        outs.append((i, v))
    r_after = host(r_d)
    del g_d, r_d
    # the same 32 segments in one layer-wise call, on fresh copies
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ks_all = [workloads.k_for_density(int(sz), 0.001) for sz in sizes]
    g2, r2 = gpu(grad), gpu(res1)
    ws2 = torch.zeros(tgs_gpu.topk_segmented_workspace_bytes(offsets, ks_all), dtype=torch.uint8, device="cuda")
    si, sv = tgs_gpu.topk_ef_step_segmented(g2, r2, offsets, ks_all, ws=ws2)
    tgs_gpu.check_device_error(ws2)
    si, sv, sr = host(si), host(sv), host(r2)
    del g2, r2, ws2
    assert np.array_equal(bits(sr), bits(r_after)), "segmented residual"
    koffs = np.concatenate([[0], np.cumsum(ks_all)])
    for j, (gi, gv) in enumerate(outs):
        assert np.array_equal(si[koffs[j]:koffs[j + 1]], gi) and np.array_equal(bits(sv[koffs[j]:koffs[j + 1]]), bits(gv))
    res2 = res1
    exp = _vgg16_segments_oracle(grad, res2, starts, sizes)
    for (s0, sz), (gi, gv), (ei, ev) in zip(zip(starts, sizes), outs, exp):
        assert_topk_equal((gi, gv, r_after[s0:s0 + sz]), (ei, ev, res2[s0:s0 + sz]), "segment at %d size %d" % (s0, sz))


def test_vgg16_sized_whole_vector(tgs_gpu):
    """n = 138M as one vector, k = 138,000: the residual is the oracle's step 1
    from 0; step 2 on the GPU, certified by the invariants that pin the unique
    top-k (exact count, values, residual, order, tie rule)."""
    n = 138_000_000
    k = workloads.k_for_density(n, 0.001)
    res1 = np.zeros(n, np.float32)
    oracle.topk_ef_step(workloads.grad_vgg16(1, variant=1), res1, k)
    grad = workloads.grad_vgg16(2, variant=1)
    got = gpu_topk(tgs_gpu, grad, res1, k)
    check_topk_invariants(res1 + grad, got[2], got[0], got[1], k)


def test_large_transformer_sized_two_chained_steps(tgs_gpu):
    """n = 1.5e9, N(0,1e-3) + 0.5% Laplace(0,0.05), k = 1.5M (0.1%), residual
    from 0 over two chained steps with fresh gradients drawn on the GPU.  Each
    step is certified on the host by the invariants that pin the unique top-k
    (exact count, values, residual, order, tie rule), so the residual step 2
    starts from is the one the definition gives."""
    n = 1_500_000_000
    k = workloads.k_for_density(n, 0.001)
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    res_h = np.zeros(n, np.float32)
    for step in (1, 2):
        g = workloads.mixture_gpu(n, 1e-3, 0.005, 0.05, (5, 0, step))
        grad_h = host(g)
        idx_h, val_h, r_after = topk_dev(tgs_gpu, g, r, k)
        del g
        torch.cuda.empty_cache()
        acc = res_h + grad_h
        del grad_h
        check_topk_invariants(acc, r_after, idx_h, val_h, k)
        del acc
        res_h = r_after


def _ctl(ws):
    """(verdict, fallbacks, why, rescans) words at the start of a top-k workspace."""
    w = host(ws[:24].view(torch.int32))
    return int(w[2]), int(w[3]), int(w[4]), int(w[5])


@pytest.mark.parametrize("path,route", [(0, "fast"), (6, "fast"), (3, "reread"), (4, "reread"), (2, "fallback"),
                                        (5, "fallback")])
def test_fast_path_routes(tgs_gpu, path, route):
    """Each route through the single-launch step: the plan holds (with the
    usual slots, or with one slot so that candidates overflow); workgroups
    re-read their rows (no list / overflowing list); the plan fails and the
    exact path runs on the same launch.  Results always match the oracle."""
    rng = np.random.default_rng(17)
    n, k = 4_000_000, 4000  # shares of ~15.7K entries: more than a local list holds when T_loc = 0
    grad, res = make("mixture", n, rng)
    exp = oracle_topk(grad, res, k)
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, path)
    g, r = gpu(grad), gpu(res)
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    idx, val = tgs_gpu.topk_ef_step(g, r, k, ws=ws)
    tgs_gpu.check_device_error(ws)
    assert_topk_equal((host(idx), host(val), host(r)), exp, "path=%d" % path)
    verdict, fallbacks, why, rescans = _ctl(ws)
    if route == "fast":
        assert verdict == 1 and fallbacks == 0 and rescans == 0
    elif route == "reread":
        assert verdict == 1 and fallbacks == 0 and rescans > 0
    else:
        assert verdict == 0 and fallbacks == 1 and why != 0


def test_workspace_shared_by_all_operations(tgs_gpu):
    """One zero-filled buffer serves top-k, threshold and gTop-k calls in turn
    (each operation leaves the top-k counters clean), with grids that change
    from one top-k call to the next."""
    rng = np.random.default_rng(23)
    n, k = 1_500_000, 1500
    need = max(tgs_gpu.topk_workspace_bytes(n, k), tgs_gpu.threshold_workspace_bytes(n),
               tgs_gpu.gtopk_workspace_bytes(4, 512, n))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    for step, grid in enumerate([0, 100, 0, 256, 80, 0]):
        tgs_gpu.set_option(tgs_gpu.OPT_MAIN_GRID, grid)
        grad = rng.standard_normal(n).astype(np.float32)
        idx, val = tgs_gpu.topk_ef_step(gpu(grad), r_gpu, k, ws=ws)
        tgs_gpu.check_device_error(ws)
        ei, ev = oracle.topk_ef_step(grad, r_cpu, k)
        assert_topk_equal((host(idx), host(val), host(r_gpu)), (ei, ev, r_cpu), "step %d grid %d" % (step, grid))
        if step % 2 == 0:  # another operation on the same buffer in between
            g2 = rng.standard_normal(n).astype(np.float32)
            r2 = torch.zeros(n, dtype=torch.float32, device="cuda")
            tgs_gpu.threshold_ef_step(gpu(g2), r2, 2.5, 4096, ws=ws)
            tgs_gpu.check_device_error(ws)
            gi, gv = workloads.gtopk_sets(P=4, k=512, n=n, hot=1024)
            tgs_gpu.gtopk_merge(gpu(gi), gpu(gv), n, ws=ws)
            tgs_gpu.check_device_error(ws)


def _guided(ws):
    """(guided_used, guided_missed) words of a top-k workspace."""
    w = host(ws[:32].view(torch.int32))
    return int(w[6]), int(w[7])


def _guided_step(tgs_gpu, g, r, k):
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(g.numel(), k), dtype=torch.uint8, device=g.device)
    idx, val = tgs_gpu.topk_ef_step(g, r, k, ws=ws)
    tgs_gpu.check_device_error(ws)
    return (host(idx), host(val), host(r)), _guided(ws)


@pytest.mark.parametrize("dist", ["normal", "mixture", "ties", "special"])
def test_guided_general_path(tgs_gpu, dist):
    """Path 9: the accumulate pass copies out the entries of a sampled
    first-level bin and above while it streams, and the general path selects
    among the copies (no second read of acc).  n spans 256 chunks of whole
    rows plus a ragged last chunk and tail."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, 9)
    rng = np.random.default_rng(41)
    n = 4_200_007
    grad, res = make(dist, n, rng)
    for k in (1, 4200, 100_000):
        got, (used, missed) = _guided_step(tgs_gpu, gpu(grad), gpu(res), k)
        assert_topk_equal(got, oracle_topk(grad, res, k), "%s k=%d" % (dist, k))
        assert used + missed == 1
        if dist in ("normal", "mixture"):
            assert used == 1, "%s k=%d: the sampled guess should hold" % (dist, k)


@pytest.mark.parametrize("path", [7, 8, 9])
def test_guided_general_path_misses(tgs_gpu, path):
    """Path 7: the guessed bin is the highest one sampled, above the k-th
    key's bin; path 8: every candidate region overflows; path 9 with 3000
    entries of one value among the largest: one ranking bucket holds more
    than it may.  Each time the general path reads acc again and must still
    match the oracle."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, path)
    rng = np.random.default_rng(43 + path)
    n = 4_194_304 + 4097
    grad, res = make("mixture", n, rng)
    if path == 9:
        grad[rng.choice(n, 3000, replace=False)] = np.float32(0.75)
        res[:] = 0.0
    for k in (5000, 60_000):
        got, (used, missed) = _guided_step(tgs_gpu, gpu(grad), gpu(res), k)
        assert_topk_equal(got, oracle_topk(grad, res, k), "path=%d k=%d" % (path, k))
        assert (used, missed) == (0, 1)


@pytest.mark.parametrize("off", [1, 2, 3])
def test_guided_general_path_misaligned(tgs_gpu, off):
    """Equal 4-byte offsets: a scalar head in workgroup 0's chunk, whose
    candidates must come before those of the first row."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, 9)
    rng = np.random.default_rng(47 + off)
    n = 4_194_304 + 3 * off
    grad, res = make("normal", n, rng)
    # the largest entries sit in the head and the tail
    grad[:off] = np.float32(100.0)
    grad[-3:] = np.float32(-100.0)
    gb = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
    rb = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
    gb[off:off + n] = gpu(grad)
    rb[off:off + n] = gpu(res)
    k = 20_000
    got, (used, _) = _guided_step(tgs_gpu, gb[off:off + n], rb[off:off + n], k)
    assert_topk_equal(got, oracle_topk(grad, res, k), "offset %d" % off)
    assert used == 1
    assert np.all(host(rb[:off]) == 0) and np.all(host(rb[off + n:]) == 0)


def _bucketed(ws):
    """(used, missed) counters of the bucketed ranking in a top-k workspace."""
    w = host(ws[:64].view(torch.int32))
    return int(w[13]), int(w[14])


def test_bucketed_is_the_default_for_large_k(tgs_gpu):
    """k above what the one-launch step buckets: the bucketed ranking (the
    accumulate pass files the candidates into sampled key buckets, one
    workgroup orders each bucket) runs by default, over 3 chained EF steps
    sharing one workspace."""
    rng = np.random.default_rng(53)
    n, k = 6_000_000, 120_000
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    for step in range(3):
        grad = workloads.mixture(n, 1e-3, 0.01, 0.1, (91, step, 1))
        idx, val = tgs_gpu.topk_ef_step(gpu(grad), r_gpu, k, ws=ws)
        tgs_gpu.check_device_error(ws)
        ei, ev = oracle.topk_ef_step(grad, r_cpu, k)
        assert_topk_equal((host(idx), host(val), host(r_gpu)), (ei, ev, r_cpu), "step %d" % step)
    assert _bucketed(ws) == (3, 0) and _guided(ws) == (0, 0)


def test_bucketed_ranking_over_chained_steps(tgs_gpu):
    """Twenty chained EF steps at 2% on one residual with fresh gradients:
    every step bit for bit against the oracle.  As the residual piles up
    just below the last threshold the buckets near the k-th key grow; the
    ranking's list still holds them, so nearly every call keeps to the
    bucketed route rather than the general path."""
    n, k = 4_000_000, 80_000
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    for step in range(20):
        grad = workloads.mixture(n, 1e-3, 0.01, 0.1, (97, step, 1))
        idx, val = tgs_gpu.topk_ef_step(gpu(grad), r_gpu, k, ws=ws)
        tgs_gpu.check_device_error(ws)
        ei, ev = oracle.topk_ef_step(grad, r_cpu, k)
        assert_topk_equal((host(idx), host(val), host(r_gpu)), (ei, ev, r_cpu), "step %d" % step)
    used, missed = _bucketed(ws)
    assert used + missed == 20 and used >= 18, (used, missed)


@pytest.mark.parametrize("dist", ["normal", "mixture", "ties", "special"])
def test_bucketed_ranking(tgs_gpu, dist):
    """The bucketed ranking at several sizes and k (k >= 32768): it holds on
    the smooth distributions; on the tie-heavy grid and the special values
    (NaN, +-inf, +-0, subnormals) a bucket may exceed what one workgroup
    orders, and the general path then selects from acc.  Either way the
    oracle's result."""
    rng = np.random.default_rng(83 + len(dist))
    for n, k in ((300_001, 40_000), (4_200_007, 60_000), (6_000_000, 300_000)):
        grad, res = make(dist, n, rng)
        ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
        r = gpu(res)
        idx, val = tgs_gpu.topk_ef_step(gpu(grad), r, k, ws=ws)
        tgs_gpu.check_device_error(ws)
        assert_topk_equal((host(idx), host(val), host(r)), oracle_topk(grad, res, k), "%s n=%d k=%d" % (dist, n, k))
        used, missed = _bucketed(ws)
        assert used + missed == 1
        if dist in ("normal", "mixture"):
            assert used == 1, "%s n=%d k=%d: the bucketed ranking should hold" % (dist, n, k)


@pytest.mark.parametrize("path", [12, 13])
def test_bucketed_ranking_off_and_overflow(tgs_gpu, path):
    """Path 12: the accumulate workgroups may stage one candidate each, so
    they overflow and the general path selects from acc; path 13: the
    bucketed ranking off (the guided general path ranks the copied
    candidates)."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, path)
    rng = np.random.default_rng(89 + path)
    n, k = 4_200_007, 100_000
    grad, res = make("mixture", n, rng)
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    r = gpu(res)
    idx, val = tgs_gpu.topk_ef_step(gpu(grad), r, k, ws=ws)
    tgs_gpu.check_device_error(ws)
    assert_topk_equal((host(idx), host(val), host(r)), oracle_topk(grad, res, k), "path %d" % path)
    assert _bucketed(ws) == ({12: (0, 1), 13: (0, 0)}[path])
    assert _guided(ws) == ({12: (0, 0), 13: (1, 0)}[path])


@pytest.mark.parametrize("dist", ["normal", "ties", "special", "mixture"])
def test_small_vector_kernel(tgs_gpu, dist):
    """n <= 2^18 and k <= 256 run in one launch: each workgroup of 8192
    entries selects its own top k, the last to finish selects among those
    lists.  Sizes at the workgroup boundaries, k at both ends, ties across
    workgroups (the lower index wins) and unaligned slices."""
    rng = np.random.default_rng(59 + len(dist))
    for n in (1, 2, 8191, 8192, 8193, 100_003, 262_144):
        grad, res = make(dist, n, rng)
        for k in (1, 7, 255, 256):
            if k > n:
                continue
            assert_topk_equal(gpu_topk(tgs_gpu, grad, res, k), oracle_topk(grad, res, k), "n=%d k=%d %s" % (n, k, dist))
    # every entry equal: the k lowest indices, all from workgroup 0
    grad = np.full(50_000, 0.75, np.float32)
    res = np.zeros_like(grad)
    assert_topk_equal(gpu_topk(tgs_gpu, grad, res, 256), oracle_topk(grad, res, 256), "all equal")
    # unaligned slice
    n, off = 30_001, 3
    grad, res = make(dist, n, rng)
    gb = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
    rb = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
    gb[1:1 + n] = gpu(grad)
    rb[off:off + n] = gpu(res)
    got = topk_dev(tgs_gpu, gb[1:1 + n], rb[off:off + n], 100)
    assert_topk_equal(got, oracle_topk(grad, res, 100), "unaligned")
    assert np.all(host(rb[:off]) == 0) and np.all(host(rb[off + n:]) == 0)


def _oracle_segments(grad, res, offsets, ks):
    """Per-slice oracle steps: (concatenated idx, concatenated val, residual)."""
    r = res.copy()
    ii, vv = [], []
    for s in range(len(ks)):
        a, b = int(offsets[s]), int(offsets[s + 1])
        rs = r[a:b].copy()
        i, v = oracle.topk_ef_step(grad[a:b], rs, int(ks[s]))
        r[a:b] = rs
        ii.append(i)
        vv.append(v)
    return np.concatenate(ii).astype(np.int32), np.concatenate(vv).astype(np.float32), r


def _segmented_dev(tgs_gpu, grad, res, offsets, ks):
    g, r = gpu(grad), gpu(res)
    ws = torch.zeros(tgs_gpu.topk_segmented_workspace_bytes(offsets, ks), dtype=torch.uint8, device="cuda")
    idx, val = tgs_gpu.topk_ef_step_segmented(g, r, offsets, ks, ws=ws)
    tgs_gpu.check_device_error(ws)
    return host(idx), host(val), host(r)


@pytest.mark.parametrize("dist", ["mixture", "ties", "special"])
def test_segmented_step(tgs_gpu, dist):
    """One layer-wise call: small segments (batched in one kernel launch,
    k = 0 and k = length among them), segments just above the small limit,
    fast-path and large-k segments, an empty segment; every segment's pairs
    and residual as the oracle's step on that slice."""
    rng = np.random.default_rng(61 + len(dist))
    sizes = [1, 5, 1000, 8192, 8193, 0, 77, 100_003, 262_144, 262_145, 300_000, 600_000, 4_300_001, 3]
    ks = [1, 0, 1, 256, 8, 0, 77, 100, 256, 262, 300, 600, 60_000, 3]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    grad, res = make(dist, int(offsets[-1]), rng)
    got = _segmented_dev(tgs_gpu, grad, res, offsets, ks)
    assert_topk_equal(got, _oracle_segments(grad, res, offsets, ks), dist)


def test_segmented_many_small_segments(tgs_gpu):
    """More small segments than one launch takes (64): several launches of
    the batched kernel, chained EF steps on one workspace."""
    rng = np.random.default_rng(67)
    sizes = rng.integers(1, 20_000, 150)
    ks = np.minimum(sizes, rng.integers(0, 257, 150))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(offsets[-1])
    r_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_cpu = np.zeros(n, np.float32)
    ws = torch.zeros(tgs_gpu.topk_segmented_workspace_bytes(offsets, ks), dtype=torch.uint8, device="cuda")
    for step in range(2):
        grad = rng.standard_normal(n).astype(np.float32)
        idx, val = tgs_gpu.topk_ef_step_segmented(gpu(grad), r_gpu, offsets, ks, ws=ws)
        tgs_gpu.check_device_error(ws)
        ei, ev, r_cpu = _oracle_segments(grad, r_cpu, offsets, ks)
        assert_topk_equal((host(idx), host(val), host(r_gpu)), (ei, ev, r_cpu), "step %d" % step)


def _mid_exact(ws):
    """Segments of the batched layer-wise path that selected exactly from acc."""
    return int(host(ws[36:40].view(torch.int32))[0])


@pytest.mark.parametrize("path", [0, 10, 11])
def test_segmented_batched_routes(tgs_gpu, path):
    """Segments of at most 2^23 entries with k <= 4096 take the batched path
    (a sampled guess per segment, one streaming pass over all of them, one
    selecting workgroup per segment).  By default the guesses hold on the
    mixture, and only the dense segment (k = 4096 of 16,385) and the all-zero
    one (every key ties) select exactly from acc; path 10 forces every
    segment to, path 11 turns the batched path off.  Sizes cover a whole
    segment read into LDS (<= 8192 entries), the sampled guess, k = 0, k
    above the batched limit and odd offsets; every segment's pairs and
    residual as the oracle's step on that slice."""
    tgs_gpu.set_option(tgs_gpu.OPT_TOPK_PATH, path)
    rng = np.random.default_rng(71)
    sizes = [16_384, 16_385, 20_000, 3, 100_000, 50_000, 583_306, 9_000, 1_112_885, 300_000, 2_701_282, 4_200_001]
    ks = [16, 4096, 1, 2, 100, 10, 583, 0, 1112, 5000, 2701, 2000]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    grad, res = make("mixture", int(offsets[-1]), rng)
    z0, z1 = int(offsets[5]), int(offsets[6])
    grad[z0:z1] = 0.0
    res[z0:z1] = 0.0
    g, r = gpu(grad), gpu(res)
    ws = torch.zeros(tgs_gpu.topk_segmented_workspace_bytes(offsets, ks), dtype=torch.uint8, device="cuda")
    idx, val = tgs_gpu.topk_ef_step_segmented(g, r, offsets, ks, ws=ws)
    tgs_gpu.check_device_error(ws)
    got = (host(idx), host(val), host(r))
    assert_topk_equal(got, _oracle_segments(grad, res, offsets, ks), "path %d" % path)
    batched = sum(1 for n_, k_ in zip(sizes, ks) if n_ <= 1 << 23 and 0 < k_ <= 4096)
    assert _mid_exact(ws) == {0: 2, 10: batched, 11: 0}[path]


@pytest.mark.parametrize("n,k", [(300_001, 300), (583_306, 583), (600_000, 60_000), (1_000_003, 100_000)])
def test_guided_mid_sizes(tgs_gpu, n, k):
    """Vectors between 2^18 and a few million entries, where the one-launch
    step does not apply, take the guided route with fewer accumulate
    workgroups than general-path workgroups."""
    rng = np.random.default_rng(n % 1000 + k)
    grad, res = make("mixture", n, rng)
    ws = torch.zeros(tgs_gpu.topk_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    r = gpu(res)
    idx, val = tgs_gpu.topk_ef_step(gpu(grad), r, k, ws=ws)
    tgs_gpu.check_device_error(ws)
    assert_topk_equal((host(idx), host(val), host(r)), oracle_topk(grad, res, k), "n=%d k=%d" % (n, k))
    # k from 32768 on: the bucketed ranking; below it the guided ranking
    assert (_bucketed(ws) if k >= 32768 else _guided(ws)) == (1, 0)
