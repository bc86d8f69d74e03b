"""GPU parity of tgs_gtopk_merge against the CPU oracle (bit for bit)."""
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


def run_both(tgs, idx, val, n):
    gi, gv, gm = tgs.gtopk_merge(gpu(idx), gpu(val), n, check=True)
    ei, ev, em = oracle.gtopk_merge(idx, val, n)
    return (host(gi), host(gv), host(gm)), (ei, ev, em)


def assert_merge_equal(got, exp, what):
    assert np.array_equal(got[0], exp[0]), what + ": indices differ"
    assert np.array_equal(bits(got[1]), bits(exp[1])), what + ": values differ"
    assert np.array_equal(got[2], exp[2]), what + ": masks differ"


def test_golden(tgs_gpu):
    g = json.load(open(os.path.join(GOLDEN, "gtopk_tournament.json")))
    for case in g["cases"]:
        gi, gv, gm = tgs_gpu.gtopk_merge(gpu(np.array(case["idx"], np.int32)), gpu(np.float32(case["val"])), case["n"],
                                         check=True)
        assert host(gi).tolist() == case["gidx"], case["name"]
        assert np.array_equal(bits(host(gv)), bits(case["gval"])), case["name"]
        assert host(gm).tolist() == case["mask"], case["name"]


def random_sets(rng, P, k, n, hot):
    H = rng.choice(n, hot, replace=False)
    idx = np.empty((P, k), np.int32)
    for p in range(P):
        a = rng.choice(H, min(k // 2, hot), replace=False)
        rest = np.setdiff1d(rng.choice(n, 3 * k, replace=False), a)[: k - a.size]
        idx[p] = rng.permutation(np.concatenate([a, rest]))
    val = rng.laplace(0, 1, (P, k)).astype(np.float32)
    return idx, val


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 13, 32])
@pytest.mark.parametrize("k", [1, 7, 100, 2048, 2049, 5000])
def test_random_parity(tgs_gpu, P, k):
    rng = np.random.default_rng(P * 1000 + k)
    n = max(4 * k, 64)
    idx, val = random_sets(rng, P, k, n, min(n, 2 * k))
    got, exp = run_both(tgs_gpu, idx, val, n)
    assert_merge_equal(got, exp, "P=%d k=%d" % (P, k))


def test_ties_and_cancellation(tgs_gpu):
    """Values on a coarse grid: many equal magnitudes and exact cancellations."""
    rng = np.random.default_rng(4)
    P, k, n = 16, 3000, 20000
    idx, _ = random_sets(rng, P, k, n, 4000)
    val = (rng.integers(-3, 4, (P, k)) * 0.5).astype(np.float32)
    val[val == 0] = 0.5
    got, exp = run_both(tgs_gpu, idx, val, n)
    assert_merge_equal(got, exp, "ties")


@pytest.mark.parametrize("k", [10000, 20000, 40000])
def test_mid_k_three_workers(tgs_gpu, k):
    """P = 3: round 0 merges rows 0 and 1, row 2 waits a round; k spans the
    select's one-LDS-list and streaming sizes."""
    rng = np.random.default_rng(k + 3)
    n = 4 * k
    idx, val = random_sets(rng, 3, k, n, 2 * k)
    got, exp = run_both(tgs_gpu, idx, val, n)
    assert_merge_equal(got, exp, "P=3 k=%d" % k)


def test_ties_large_k(tgs_gpu):
    """k = 40,000 on a coarse value grid: the k-th key is held by thousands of
    entries, so the lowest indices decide."""
    rng = np.random.default_rng(40)
    P, k, n = 4, 40000, 200000
    idx, _ = random_sets(rng, P, k, n, 60000)
    val = (rng.integers(-3, 4, (P, k)) * 0.5).astype(np.float32)
    val[val == 0] = 0.5
    got, exp = run_both(tgs_gpu, idx, val, n)
    assert_merge_equal(got, exp, "ties k=40000")


@pytest.mark.parametrize("P,k", [(2, 300_001), (3, 1 << 20)])
def test_large_k(tgs_gpu, P, k):
    """k far past one sorted run of the final set: 74 runs and seven merge
    passes with a ragged last run (k = 300,001), and the largest k the call
    takes (2^20: 256 runs, eight passes), with the hash parts at their most."""
    rng = np.random.default_rng(7 + P)
    n = 4 * k
    idx, val = random_sets(rng, P, k, n, 2 * k)
    got, exp = run_both(tgs_gpu, idx, val, n)
    assert_merge_equal(got, exp, "P=%d k=%d" % (P, k))


def test_nan_and_inf_values(tgs_gpu):
    """NaN (bit patterns 0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00000, 0xFFC00001) and
    +-inf on indices no other row holds (so they are never added): NaN keys
    rank above inf, inf above every finite key."""
    rng = np.random.default_rng(77)
    P, k, n = 5, 3000, 50000
    idx, val = random_sets(rng, P, k, n, 4000)
    specials = np.array([0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00000, 0xFFC00001, 0x7F800000, 0xFF800000],
                        np.uint32).view(np.float32)
    counts = np.bincount(idx.ravel(), minlength=n)
    for p in range(P):
        own = np.nonzero(counts[idx[p]] == 1)[0]
        pos = rng.choice(own, 3 * specials.size, replace=False)
        val[p, pos] = np.tile(specials, 3)
    got, exp = run_both(tgs_gpu, idx, val, n)
    assert_merge_equal(got, exp, "nan/inf")


def test_full_config(tgs_gpu):
    """P = 32 workers, k = 25,600 pairs over [0, 25.6M), half of each row from
    a shared hot set of 51,200: 5 rounds."""
    idx, val = workloads.gtopk_sets()
    got, exp = run_both(tgs_gpu, idx, val, 25_600_000)
    assert_merge_equal(got, exp, "P=32 k=25600")
    # rows handed over in the order a top-k step emits them (key desc, index asc)
    kk = keys(val).astype(np.int64)
    order = np.stack([np.lexsort((idx[p], -kk[p])) for p in range(idx.shape[0])])
    idx2 = np.take_along_axis(idx, order, 1)
    val2 = np.take_along_axis(val, order, 1)
    got2, exp2 = run_both(tgs_gpu, idx2, val2, 25_600_000)
    assert_merge_equal(got2, exp2, "rows in rank order")
    assert np.array_equal(got2[0], got[0])


def test_identical_supports(tgs_gpu):
    P, k = 32, 1000
    idx = np.tile(np.arange(0, 3 * k, 3, dtype=np.int32), (P, 1))
    val = np.full((P, k), 0.375, np.float32)
    gi, gv, gm = tgs_gpu.gtopk_merge(gpu(idx), gpu(val), 3 * k, check=True)
    assert np.all(host(gv) == np.float32(12.0)) and np.all(host(gm) == 1)


def test_bad_rows_raise(tgs_gpu):
    idx = np.array([[1, 1, 2], [3, 4, 5]], np.int32)
    val = np.ones((2, 3), np.float32)
    with pytest.raises(ValueError):
        tgs_gpu.gtopk_merge(gpu(idx), gpu(val), 10, check=True)
    idx = np.array([[1, 2, 12], [3, 4, 5]], np.int32)
    with pytest.raises(ValueError):
        tgs_gpu.gtopk_merge(gpu(idx), gpu(val), 10, check=True)
    # the check cleared the error word: a good call afterwards reports nothing
    idx = np.array([[1, 2, 7], [3, 4, 5]], np.int32)
    tgs_gpu.gtopk_merge(gpu(idx), gpu(val), 10, check=True)
