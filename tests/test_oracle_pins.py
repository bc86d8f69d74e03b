"""Pins the CPU oracle to facts that do not come from the oracle itself.

* hand-worked examples from the pages' definitions (tests/golden/*.json),
* IEEE binary32 addition as numpy performs it (a library routine),
* an O(n^2) rank definition and an exhaustive subset search for tiny n,
* closed forms (k = 0, k = n, all-equal values, permutations of 1..n),
* invariants that certify a top-k answer at any size,
* for the threshold: a direct count and the top-count set,
* for the merge: P = 1 and P = 2 against the exact top-k of the sparse sum,
  disjoint supports against the top-k of the concatenation, identical supports
  against P * v, input-order invariance and the log2 P round count.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def from_bits(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def keys(a):
    return bits(a) & np.uint32(0x7FFFFFFF)


def rank_order(acc):
    """Brute force O(n^2): rank_i = #{j : key_j > key_i or (key_j == key_i and j < i)}."""
    kk = [int(x) for x in keys(acc)]
    n = len(kk)
    ranks = [sum(1 for j in range(n) if kk[j] > kk[i] or (kk[j] == kk[i] and j < i)) for i in range(n)]
    order = [None] * n
    for i, r in enumerate(ranks):
        order[r] = i
    return order


def check_topk_invariants(acc, res_after, idx, val, k):
    """Invariants that pin the unique top-k answer at any size."""
    n = acc.size
    assert idx.size == k and val.size == k
    if k:
        assert idx.min() >= 0 and idx.max() < n
        assert np.unique(idx).size == k
        assert np.array_equal(bits(val), bits(acc[idx]))
    sel = np.zeros(n, dtype=bool)
    sel[idx] = True
    assert np.all(bits(res_after[sel]) == 0)
    assert np.array_equal(bits(res_after[~sel]), bits(acc[~sel]))
    ka = keys(acc).astype(np.int64)
    if 0 < k < n:
        # every selected (key, -index) beats every unselected one
        sel_keys, uns_keys = ka[sel], ka[~sel]
        kmin = sel_keys.min()
        assert kmin >= uns_keys.max()
        tie_sel = np.nonzero(sel & (ka == kmin))[0]
        tie_uns = np.nonzero(~sel & (ka == kmin))[0]
        if tie_uns.size:
            assert tie_sel.max() < tie_uns.min()
    # output order: key desc, index asc
    ko = ka[idx]
    ok = (ko[:-1] > ko[1:]) | ((ko[:-1] == ko[1:]) & (idx[:-1] < idx[1:]))
    assert np.all(ok)


# ----------------------------------------------------------------- golden ----
def test_golden_topk_ties(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "topk_ef_ties.json")))
    for case in g["cases"]:
        res = f32(g["residual"]).copy()
        idx, val = oracle_lib.topk_ef_step(f32(g["grad"]), res, case["k"])
        assert idx.tolist() == case["idx"]
        assert np.array_equal(bits(val), bits(case["val"]))
        assert np.array_equal(bits(res), bits(case["residual_after"]))


def test_golden_two_steps(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "topk_ef_two_steps.json")))
    res = f32(g["residual0"]).copy()
    for st in g["steps"]:
        idx, val = oracle_lib.topk_ef_step(f32(st["grad"]), res, g["k"])
        assert idx.tolist() == st["idx"]
        assert np.array_equal(bits(val), bits(st["val"]))
        assert np.array_equal(bits(res), bits(st["residual_after"]))


def test_golden_acc_rounding(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "acc_rounding.json")))
    res = from_bits(g["residual_bits"]).copy()
    grad = from_bits(g["grad_bits"])
    idx, val = oracle_lib.topk_ef_step(grad, res, g["k"])
    assert idx.tolist() == g["idx"]
    assert [int(b) for b in bits(val)] == [int(h, 16) for h in g["val_bits"]]
    assert np.all(bits(res) == 0)


def test_golden_threshold(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "threshold_ties.json")))
    for case in g["cases"]:
        res = f32(g["residual"]).copy()
        idx, val, count = oracle_lib.threshold_ef_step(f32(g["grad"]), res, case["lambda"], case["capacity"])
        assert count == case["count"]
        assert idx.tolist() == case["idx"]
        assert np.array_equal(bits(val), bits(case["val"]))
        assert np.array_equal(bits(res), bits(case["residual_after"]))
    assert int(bits(np.float32(4e-3))) == int(g["lambda_4e-3_bits"], 16)


def test_golden_gtopk(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "gtopk_tournament.json")))
    for case in g["cases"]:
        gi, gv, mask, rounds = oracle_lib.gtopk_merge(np.array(case["idx"], np.int32), f32(case["val"]),
                                                      case["n"], return_rounds=True)
        assert gi.tolist() == case["gidx"], case["name"]
        assert np.array_equal(bits(gv), bits(case["gval"])), case["name"]
        assert mask.tolist() == case["mask"], case["name"]
        assert rounds == case["rounds"], case["name"]


# --------------------------------------------------------- binary32 adds ----
def test_acc_matches_numpy_binary32_add(oracle_lib):
    rng = np.random.default_rng(7)
    n = 20000
    # wide exponent range, subnormals, signed zeros, infinities
    r = (rng.standard_normal(n) * 10.0 ** rng.integers(-45, 39, n)).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.integers(-45, 39, n)).astype(np.float32)
    r[:50] = np.float32(1e-45) * rng.integers(1, 5, 50).astype(np.float32)
    g[:50] = -np.float32(1e-45) * rng.integers(0, 5, 50).astype(np.float32)
    r[50:60] = -0.0
    g[50:55] = 0.0
    g[55:60] = -0.0
    r[60:70] = np.inf
    g[60:65] = -1.0
    expect = r + g  # numpy float32 add: IEEE binary32, round to nearest even
    res = r.copy()
    oracle_lib.topk_ef_step(g, res, 0)
    assert np.array_equal(bits(res), bits(expect))


def test_fp_mode_inside_oracle(oracle_lib):
    assert oracle_lib.fp_mode_inside_call() == 0


# ------------------------------------------------------------ brute force ----
def tie_heavy(rng, n):
    return (rng.integers(-6, 7, n) * 0.5).astype(np.float32)


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_bruteforce_rank(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    if seed % 3 == 0:
        grad, res0 = tie_heavy(rng, n), tie_heavy(rng, n)
    elif seed % 3 == 1:
        grad, res0 = rng.standard_normal(n).astype(np.float32), np.zeros(n, np.float32)
    else:
        grad, res0 = rng.standard_normal(n).astype(np.float32), rng.standard_normal(n).astype(np.float32)
    acc = res0 + grad
    order = rank_order(acc)
    for k in sorted({0, 1, n // 3, n // 2, n - 1, n} - {-1}):
        if k < 0:
            continue
        res = res0.copy()
        idx, val = oracle_lib.topk_ef_step(grad, res, k)
        assert idx.tolist() == order[:k]
        check_topk_invariants(acc, res, idx, val, k)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_exhaustive_subset_search(oracle_lib, seed):
    """For n <= 9 the selected set maximises the sum of keys and is the
    lexicographically first index tuple among maximisers."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 10))
    grad = tie_heavy(rng, n) if seed % 2 else rng.standard_normal(n).astype(np.float32)
    res0 = np.zeros(n, np.float32)
    kk = [int(x) for x in keys(res0 + grad)]
    for k in range(n + 1):
        best = None
        for comb in itertools.combinations(range(n), k):
            s = sum(kk[i] for i in comb)
            if best is None or s > best[0]:
                best = (s, comb)
        res = res0.copy()
        idx, _ = oracle_lib.topk_ef_step(grad, res, k)
        assert tuple(sorted(idx.tolist())) == best[1]


# ----------------------------------------------------------- closed forms ----
def test_topk_closed_forms(oracle_lib):
    n = 257
    rng = np.random.default_rng(3)
    perm = rng.permutation(n)
    grad = (perm + 1).astype(np.float32)  # a permutation of 1..n
    for k in (1, 17, n):
        res = np.zeros(n, np.float32)
        idx, val = oracle_lib.topk_ef_step(grad, res, k)
        assert val.tolist() == [float(n - j) for j in range(k)]
        assert np.array_equal(idx, np.argsort(-grad, kind="stable")[:k].astype(np.int32))
    # all equal: the first k indices
    grad = np.full(n, -0.75, np.float32)
    res = np.zeros(n, np.float32)
    idx, val = oracle_lib.topk_ef_step(grad, res, 40)
    assert idx.tolist() == list(range(40))
    # k = n: residual all zero; k = 0: residual = acc
    g2 = rng.standard_normal(n).astype(np.float32)
    r2 = rng.standard_normal(n).astype(np.float32)
    res = r2.copy()
    oracle_lib.topk_ef_step(g2, res, n)
    assert np.all(bits(res) == 0)
    res = r2.copy()
    idx, val = oracle_lib.topk_ef_step(g2, res, 0)
    assert idx.size == 0 and np.array_equal(bits(res), bits(r2 + g2))


def test_topk_special_values(oracle_lib):
    nan = np.float32(np.nan)
    grad = np.array([1.0, -np.inf, nan, -0.0, 0.0, 1e-45, -3.0, np.inf], np.float32)
    res = np.zeros(8, np.float32)
    idx, val = oracle_lib.topk_ef_step(grad, res, 5)
    # NaN key (0x7FC00000) ranks above +-inf (0x7F800000); -inf before +inf by index
    assert idx.tolist() == [2, 1, 7, 6, 0]
    assert np.isnan(val[0]) and val[1] == -np.inf and val[2] == np.inf
    # -0 and +0 tie (index order); the subnormal ranks above both
    res = np.zeros(8, np.float32)
    idx, _ = oracle_lib.topk_ef_step(grad, res, 8)
    assert idx.tolist()[5:] == [5, 3, 4]


def test_topk_invariants_medium(oracle_lib):
    rng = np.random.default_rng(11)
    n = 200_000
    grad = rng.standard_normal(n).astype(np.float32)
    res0 = (rng.laplace(0, 1, n) * (rng.random(n) < 0.01)).astype(np.float32)
    for k in (1, 200, 4000, n):
        res = res0.copy()
        idx, val = oracle_lib.topk_ef_step(grad, res, k)
        check_topk_invariants(res0 + grad, res, idx, val, k)


def test_invariant_checker_catches_planted_mistakes(oracle_lib):
    """The invariant check above must reject plausible wrong answers."""
    rng = np.random.default_rng(5)
    n, k = 1000, 50
    grad = tie_heavy(rng, n)
    res0 = np.zeros(n, np.float32)
    res = res0.copy()
    idx, val = oracle_lib.topk_ef_step(grad, res, k)
    acc = res0 + grad
    bad = []
    i2 = idx.copy(); i2[[0, 1]] = i2[[1, 0]]; bad.append((res, i2, acc[i2]))          # order
    ka = keys(acc)
    kmin = ka[idx].min()
    loser = np.nonzero((ka == kmin) & ~np.isin(np.arange(n), idx))[0][0]
    winner = idx[np.nonzero(ka[idx] == kmin)[0][-1]]
    i3 = idx.copy(); i3[i3 == winner] = loser                                          # tie rule
    r3 = acc.copy(); r3[i3] = 0
    bad.append((r3, i3, acc[i3]))
    r4 = res.copy(); r4[idx[0]] = acc[idx[0]]; bad.append((r4, idx, val))              # residual
    v5 = val.copy(); v5[0] = -v5[0]; bad.append((res, idx, v5))                        # sign
    for r_, i_, v_ in bad:
        with pytest.raises(AssertionError):
            check_topk_invariants(acc, r_, i_, v_, k)


# --------------------------------------------------------------- threshold ----
@pytest.mark.parametrize("seed", range(4))
def test_threshold_count_and_set(oracle_lib, seed):
    rng = np.random.default_rng(200 + seed)
    n = 50_000
    grad = (rng.integers(-8, 9, n) * 0.25).astype(np.float32) if seed % 2 else rng.standard_normal(n).astype(np.float32)
    res0 = rng.standard_normal(n).astype(np.float32) * np.float32(0.1)
    acc = res0 + grad
    for lam in (0.0, 0.5, 1.0, 2.25, 1e9):
        res = res0.copy()
        idx, val, count = oracle_lib.threshold_ef_step(grad, res, lam, n)
        direct = int(np.count_nonzero(keys(acc) >= keys(np.float32(lam))))
        assert count == direct
        assert np.all(np.diff(idx) > 0)
        # the emitted set is exactly the top-`count` set
        r2 = res0.copy()
        tidx, _ = oracle_lib.topk_ef_step(grad, r2, count)
        assert set(idx.tolist()) == set(tidx.tolist())
        assert np.array_equal(bits(res), bits(r2))
        assert np.array_equal(bits(val), bits(acc[idx]))
    # capacity truncation keeps the index-order prefix and leaves the rest in the residual
    res = res0.copy()
    idx, val, count = oracle_lib.threshold_ef_step(grad, res, 1.0, 100)
    full = np.nonzero(keys(acc) >= keys(np.float32(1.0)))[0]
    assert count == full.size and idx.tolist() == full[:100].tolist()
    assert np.array_equal(bits(res[full[100:]]), bits(acc[full[100:]]))


def test_threshold_expected_density_large_mixture(oracle_lib):
    """lambda = 4e-3 on N(0,1e-3) + 0.5% Laplace(0, 0.05): density
    0.995 * 2Q(4) + 0.005 * exp(-0.08) = 4.68e-3 (closed form), within 5 sigma."""
    from top_gradient_sparsification_amd import workloads
    n = 4_000_000
    grad = workloads.mixture(n, 1e-3, 0.005, 0.05, (99, 0, 1))
    res = np.zeros(n, np.float32)
    _, _, count = oracle_lib.threshold_ef_step(grad, res, 4e-3, 0)
    q4 = 0.5 * math.erfc(4 / math.sqrt(2))
    p = 0.995 * 2 * q4 + 0.005 * math.exp(-4e-3 / 0.05)
    assert abs(count - p * n) < 5 * math.sqrt(p * n)


# ------------------------------------------------------------------ merge ----
def exact_topk_of_sum(idx, val, k):
    """Top-k (key desc, index asc) of the sum of sparse vectors, by dict."""
    acc = {}
    for row_i, row_v in zip(idx.tolist(), val.tolist()):
        for i, v in zip(row_i, row_v):
            acc[i] = np.float32(acc[i] + np.float32(v)) if i in acc else np.float32(v)
    items = sorted(acc.items(), key=lambda t: (-int(keys(np.float32(t[1]))), t[0]))[:k]
    return [i for i, _ in items], f32([v for _, v in items])


def random_sets(rng, P, k, n, shared):
    idx = np.empty((P, k), np.int32)
    for p in range(P):
        pool = rng.choice(shared, size=min(k // 2, shared.size), replace=False) if shared.size else np.zeros(0, int)
        rest = rng.choice(np.setdiff1d(np.arange(n), pool), size=k - pool.size, replace=False)
        idx[p] = rng.permutation(np.concatenate([pool, rest]))
    val = rng.laplace(0, 1, (P, k)).astype(np.float32)
    return idx, val


@pytest.mark.parametrize("seed", range(6))
def test_merge_two_workers_is_exact_topk_of_sum(oracle_lib, seed):
    rng = np.random.default_rng(300 + seed)
    n, k = 200, int(rng.integers(1, 40))
    idx, val = random_sets(rng, 2, k, n, rng.choice(n, 30, replace=False))
    gi, gv, mask = oracle_lib.gtopk_merge(idx, val, n)
    ei, ev = exact_topk_of_sum(idx, val, k)
    assert gi.tolist() == ei and np.array_equal(bits(gv), bits(ev))
    assert np.array_equal(mask, np.isin(idx, gi).astype(np.uint8))


def test_merge_single_worker_is_sorted_identity(oracle_lib):
    rng = np.random.default_rng(9)
    idx, val = random_sets(rng, 1, 50, 1000, np.zeros(0, int))
    gi, gv, mask, rounds = oracle_lib.gtopk_merge(idx, val, 1000, return_rounds=True)
    order = np.lexsort((idx[0], -keys(val[0]).astype(np.int64)))
    assert gi.tolist() == idx[0][order].tolist() and rounds == 0
    assert np.all(mask == 1)


@pytest.mark.parametrize("P", [3, 4, 7, 8, 32])
def test_merge_disjoint_supports_is_topk_of_concatenation(oracle_lib, P):
    rng = np.random.default_rng(400 + P)
    k, n = 16, 5000
    flat = rng.choice(n, P * k, replace=False).astype(np.int32)
    idx = flat.reshape(P, k)
    val = rng.laplace(0, 1, (P, k)).astype(np.float32)
    gi, gv, mask, rounds = oracle_lib.gtopk_merge(idx, val, n, return_rounds=True)
    ei, ev = exact_topk_of_sum(idx, val, k)
    assert gi.tolist() == ei and np.array_equal(bits(gv), bits(ev))
    assert rounds == math.ceil(math.log2(P))


def test_merge_identical_supports_sum_exactly(oracle_lib):
    P, k, n = 32, 8, 100
    idx = np.tile(np.arange(0, 2 * k, 2, dtype=np.int32), (P, 1))
    v = np.float32(0.375)
    val = np.full((P, k), v, np.float32)
    gi, gv, mask, rounds = oracle_lib.gtopk_merge(idx, val, n, return_rounds=True)
    assert np.all(gv == np.float32(P) * v) and gi.tolist() == idx[0].tolist()
    assert rounds == 5 and np.all(mask == 1)


def test_merge_invariant_under_row_permutation(oracle_lib):
    rng = np.random.default_rng(17)
    P, k, n = 8, 30, 500
    idx, val = random_sets(rng, P, k, n, rng.choice(n, 60, replace=False))
    gi, gv, mask = oracle_lib.gtopk_merge(idx, val, n)
    perm = np.array([rng.permutation(k) for _ in range(P)])
    idx2 = np.take_along_axis(idx, perm, 1)
    val2 = np.take_along_axis(val, perm, 1)
    gi2, gv2, mask2 = oracle_lib.gtopk_merge(idx2, val2, n)
    assert gi.tolist() == gi2.tolist() and np.array_equal(bits(gv), bits(gv2))
    assert np.array_equal(np.take_along_axis(mask, perm, 1), mask2)


def test_merge_rejects_bad_rows(oracle_lib):
    idx = np.array([[1, 1], [2, 3]], np.int32)
    val = np.ones((2, 2), np.float32)
    with pytest.raises(ValueError):
        oracle_lib.gtopk_merge(idx, val, 10)
    with pytest.raises(ValueError):
        oracle_lib.gtopk_merge(np.array([[0, 10]], np.int32), np.ones((1, 2), np.float32), 10)


# ------------------------------------------------------ threshold estimate --
def test_golden_threshold_estimate(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "threshold_estimate.json")))
    grad, res = f32(g["grad"]), f32(g["residual"])
    sample = np.array(g["sample"], np.int32)
    for case in g["cases"]:
        r = res.copy()
        assert oracle_lib.threshold_estimate(grad, r, sample, case["q"]) == int(case["key"], 16)
        idx, val, count, key = oracle_lib.estimated_threshold_ef_step(grad, r, sample, case["q"], 8)
        assert key == int(case["key"], 16) and count == case["count"]


@pytest.mark.parametrize("seed", range(40))
def test_threshold_estimate_count_characterisation(oracle_lib, seed):
    """Brute force on tiny inputs: the estimate is a sampled key v with
    #{j : key_j > v} < q <= #{j : key_j >= v} (the q-th largest, counted with
    repeats), computed with numpy's binary32 add and no sort."""
    rng = np.random.default_rng(900 + seed)
    n = int(rng.integers(1, 40))
    grad = tie_heavy(rng, n) if seed % 2 else rng.standard_normal(n).astype(np.float32)
    res = tie_heavy(rng, n)
    m = int(rng.integers(1, 50))
    sample = rng.integers(0, n, m).astype(np.int32)
    sk = [int(x) for x in keys((res + grad)[sample])]
    for q in range(1, m + 1):
        v = oracle_lib.threshold_estimate(grad, res, sample, q)
        assert v in sk
        assert sum(1 for x in sk if x > v) < q <= sum(1 for x in sk if x >= v)


def test_threshold_estimate_closed_forms(oracle_lib):
    n = 1000
    # all-equal magnitudes: the estimate is that magnitude for every q
    grad = np.where(np.arange(n) % 3 == 0, -0.375, 0.375).astype(np.float32)
    sample = np.arange(0, n, 7, dtype=np.int32)
    for q in (1, 5, sample.size):
        assert oracle_lib.threshold_estimate(grad, np.zeros(n, np.float32), sample, q) == int(keys(f32(0.375)))
    # the sampled accs are a permutation of 1..m: the q-th largest is m - q + 1
    m = 200
    rng = np.random.default_rng(5)
    perm = rng.permutation(m) + 1
    sample = rng.choice(n, m, replace=False).astype(np.int32)
    grad = rng.standard_normal(n).astype(np.float32)
    grad[sample] = perm.astype(np.float32)
    for q in (1, 2, 50, 200):
        assert oracle_lib.threshold_estimate(grad, np.zeros(n, np.float32), sample, q) == int(keys(f32(m - q + 1)))


@pytest.mark.parametrize("seed", range(5))
def test_full_sample_estimate_is_the_topk_threshold(oracle_lib, seed):
    """Sampling every position with q = k: the hard threshold then keeps
    exactly the top-k set of the (separately pinned) top-k oracle, plus any
    ties at the k-th key."""
    rng = np.random.default_rng(70 + seed)
    n, k = 5000, 37 + 40 * seed
    grad = rng.standard_normal(n).astype(np.float32) if seed < 3 else tie_heavy(rng, n)
    res = rng.standard_normal(n).astype(np.float32)
    r1, r2 = res.copy(), res.copy()
    idx, val, count, key = oracle_lib.estimated_threshold_ef_step(grad, r1, np.arange(n, dtype=np.int32), k, n)
    ti, tv = oracle_lib.topk_ef_step(grad, r2, k)
    acc = res + grad
    assert key == int(keys(acc)[ti[-1]])
    assert count == int(np.sum(keys(acc) >= key)) >= k
    assert set(ti.tolist()) <= set(idx.tolist())
    if count == k:
        assert np.array_equal(np.sort(ti), idx) and np.array_equal(bits(r1), bits(r2))


def test_threshold_estimate_special_values_and_rejects(oracle_lib):
    grad = f32([np.nan, 1.0, -np.inf, 0.5, -0.0])
    res = np.zeros(5, np.float32)
    s = np.arange(5, dtype=np.int32)
    assert oracle_lib.threshold_estimate(grad, res, s, 1) == int(keys(f32(np.nan)))  # NaN above inf
    assert oracle_lib.threshold_estimate(grad, res, s, 2) == 0x7F800000
    assert oracle_lib.threshold_estimate(grad, res, s, 5) == 0  # -0 has key 0
    # a NaN-payload threshold keeps only the NaN
    idx, val, count, key = oracle_lib.estimated_threshold_ef_step(grad, res.copy(), s, 1, 5)
    assert count == 1 and idx.tolist() == [0]
    for q in (0, 6):
        with pytest.raises(ValueError):
            oracle_lib.threshold_estimate(grad, res, s, q)
    with pytest.raises(ValueError):
        oracle_lib.threshold_estimate(grad, res, np.array([0, 5], np.int32), 1)


# ----------------------------------------------------------------- rTop-k --
def test_golden_philox_known_answers(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "philox_kat.json")))
    for case in g["cases"]:
        out = oracle_lib.philox4x32_10([int(x, 16) for x in case["ctr"]], [int(x, 16) for x in case["key"]])
        assert [int(x) for x in out] == [int(x, 16) for x in case["out"]]


@pytest.mark.parametrize("seed", range(6))
def test_rtopk_with_r_equal_k_is_topk(oracle_lib, seed):
    rng = np.random.default_rng(300 + seed)
    n = 3000
    grad = rng.standard_normal(n).astype(np.float32) if seed % 2 else tie_heavy(rng, n)
    res = rng.standard_normal(n).astype(np.float32)
    for k in (0, 1, 17, 400, n):
        r1, r2 = res.copy(), res.copy()
        ri, rv = oracle_lib.rtopk_ef_step(grad, r1, k, k, 1234 + seed, seed)
        ti, tv = oracle_lib.topk_ef_step(grad, r2, k)
        assert np.array_equal(ri, ti) and np.array_equal(bits(rv), bits(tv)) and np.array_equal(bits(r1), bits(r2))


@pytest.mark.parametrize("seed", range(8))
def test_rtopk_picks_the_smallest_draws_of_the_top_r(oracle_lib, seed):
    """The k emitted entries are the members of the top r (from the pinned
    top-k oracle) with the smallest (draw, index), the draw being Philox word
    0 at counter (index, step low, step high, 0) under key (seed low, seed
    high); in (key desc, index asc) order; residual +0 there, acc elsewhere."""
    rng = np.random.default_rng(500 + seed)
    n = 4000
    grad = rng.standard_normal(n).astype(np.float32) if seed % 2 else tie_heavy(rng, n)
    res = rng.standard_normal(n).astype(np.float32)
    r, k = 64 + 50 * seed, 10 + 7 * seed
    s64, t64 = int(rng.integers(0, 2**63)) * 2 + 1, int(rng.integers(0, 2**40))
    rr = res.copy()
    idx, val = oracle_lib.rtopk_ef_step(grad, rr, r, k, s64, t64)
    top_i, _ = oracle_lib.topk_ef_step(grad, res.copy(), r)
    key2 = [s64 & 0xFFFFFFFF, s64 >> 32]

    def draw(i):
        return int(oracle_lib.philox4x32_10([i, t64 & 0xFFFFFFFF, t64 >> 32, 0], key2)[0])

    want = sorted(top_i.tolist(), key=lambda i: (draw(i), i))[:k]
    assert sorted(idx.tolist()) == sorted(want)
    pos = {int(i): p for p, i in enumerate(top_i)}
    assert [pos[int(i)] for i in idx] == sorted(pos[int(i)] for i in idx)  # the top-r list's order
    acc = res + grad
    assert np.array_equal(bits(val), bits(acc[idx]))
    sel = np.zeros(n, bool)
    sel[idx] = True
    assert np.all(bits(rr)[sel] == 0) and np.array_equal(bits(rr)[~sel], bits(acc)[~sel])


def test_rtopk_subset_is_uniform(oracle_lib):
    """Over 2000 steps each of the top r = 16 is picked (k = 4) with frequency
    k / r = 0.25 within 5 standard deviations: the draws select a uniform
    random subset, not a fixed or index-biased one."""
    n, r, k, T = 64, 16, 4, 2000
    grad = (np.arange(n, dtype=np.float32) + 1.0)[::-1].copy()  # top 16 are indices 0..15
    counts = np.zeros(r)
    for t in range(T):
        idx, _ = oracle_lib.rtopk_ef_step(grad, np.zeros(n, np.float32), r, k, 0xC0FFEE, t)
        assert idx.max() < r
        counts[idx] += 1
    p = k / r
    sd = math.sqrt(p * (1 - p) / T)
    assert np.all(np.abs(counts / T - p) < 5 * sd), counts / T


def test_rtopk_rejects_bad_sizes(oracle_lib):
    g = np.ones(10, np.float32)
    for r, k in ((11, 1), (3, 4), (-1, 0), (5, -1)):
        with pytest.raises(ValueError):
            oracle_lib.rtopk_ef_step(g, np.zeros(10, np.float32), r, k, 1, 1)
