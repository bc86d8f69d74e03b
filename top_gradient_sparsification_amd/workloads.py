"""Seeded synthetic gradients and sparse sets shaped like the pages' workloads.

The pages measure on DNN training (ResNet-20/50, VGG-16, RNNs on CIFAR-10,
ImageNet, Penn Treebank).  None of that is available or needed here: these
generators stand in with flat float32 gradients of the same sizes and a
heavy-tailed value mix.  They hold none of the sparsifier's arithmetic.

Every array is drawn on the host with numpy's PCG64 from a SeedSequence built
from (config, variant, step), in chunks of 2^24 elements whose generators are
spawned from that sequence, so any prefix or chunk is reproducible without
drawing the whole array.  Values are drawn in float64 and rounded to float32
(round to nearest even).
"""
from __future__ import annotations

import math

import numpy as np

CHUNK = 1 << 24

# configuration ids used in seeds
CFG_SMALL = 1      # n = 1,048,576, N(0, 1), residual starts at 0
CFG_RESNET50 = 2   # n = 25,600,000, 99% N(0, 1e-3) + 1% Laplace(0, 0.1)
CFG_VGG16 = 3      # n = 138,000,000 in 32 log-uniform segments, same mixture
CFG_GTOPK = 4      # P = 32 sets of k = 25,600 pairs over [0, 25.6M)
CFG_LARGE = 5      # n = 1.5e9, N(0, 1e-3) + 0.5% Laplace(0, 0.05)


def k_for_density(n: int, density: float) -> int:
    """k = floor(density * n); 0.1% of 1,048,576 is 1,048."""
    return int(math.floor(density * n + 1e-9))


def _chunks(n: int, seed: tuple):
    ss = np.random.SeedSequence(list(seed))
    nchunks = max(1, (n + CHUNK - 1) // CHUNK)
    for c, child in enumerate(ss.spawn(nchunks)):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        if lo >= hi:
            break
        yield lo, hi, np.random.Generator(np.random.PCG64(child))


def normal(n: int, sigma: float, seed: tuple, out: np.ndarray | None = None) -> np.ndarray:
    """float32[n] with N(0, sigma) entries."""
    out = np.empty(n, dtype=np.float32) if out is None else out
    for lo, hi, g in _chunks(n, seed):
        out[lo:hi] = g.normal(0.0, sigma, hi - lo)
    return out


def mixture(n: int, sigma: float, p_out: float, b_out: float, seed: tuple,
            out: np.ndarray | None = None) -> np.ndarray:
    """float32[n]: each entry is Laplace(0, b_out) with probability p_out
    (independent positions), else N(0, sigma)."""
    out = np.empty(n, dtype=np.float32) if out is None else out
    for lo, hi, g in _chunks(n, seed):
        m = hi - lo
        x = g.normal(0.0, sigma, m)
        hit = g.random(m) < p_out
        x[hit] = g.laplace(0.0, b_out, int(hit.sum()))
        out[lo:hi] = x
    return out


def grad_small(step: int, n: int = 1_048_576) -> np.ndarray:
    """Small case: N(0, 1) gradients, a fresh one per step."""
    return normal(n, 1.0, (CFG_SMALL, 0, step))


def grad_resnet50(step: int, n: int = 25_600_000, variant: int = 0) -> np.ndarray:
    """ResNet-50-sized flat gradient: 99% N(0, 1e-3) + 1% Laplace(0, 0.1)."""
    return mixture(n, 1e-3, 0.01, 0.1, (CFG_RESNET50, variant, step))


def grad_vgg16(step: int, n: int = 138_000_000, variant: int = 0) -> np.ndarray:
    """VGG-16-sized flat gradient with the same mixture as grad_resnet50."""
    return mixture(n, 1e-3, 0.01, 0.1, (CFG_VGG16, variant, step))


def grad_large(step: int, n: int = 1_500_000_000, variant: int = 0,
               out: np.ndarray | None = None) -> np.ndarray:
    """Transformer-sized flat gradient: N(0, 1e-3) + 0.5% Laplace(0, 0.05)."""
    return mixture(n, 1e-3, 0.005, 0.05, (CFG_LARGE, variant, step), out=out)


def segments_log_uniform(n: int = 138_000_000, nseg: int = 32, lo: float = 1e3, hi: float = 1e8,
                         seed: int = 0) -> np.ndarray:
    """Segment sizes (int64[nseg]) summing to n.

    Exponents e ~ U(log10 lo, log10 hi), sizes 10^e scaled by n / sum and
    floored, the remainder added to the largest segment.  A draw with any
    size outside [lo, hi] is rejected and the next seed is tried."""
    s = seed
    while True:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([CFG_VGG16, 1000 + s])))
        e = g.uniform(math.log10(lo), math.log10(hi), nseg)
        raw = 10.0 ** e
        sizes = np.floor(raw * (n / raw.sum())).astype(np.int64)
        sizes[int(np.argmax(sizes))] += n - int(sizes.sum())
        if sizes.min() >= lo and sizes.max() <= hi and int(sizes.sum()) == n:
            return sizes
        s += 1


def gtopk_sets(P: int = 32, k: int = 25_600, n: int = 25_600_000, hot: int = 51_200,
               hot_fraction: float = 0.5, seed: int = 0):
    """P workers' sparse sets: idx int32[P, k] (distinct per row, in [0, n)),
    val float32[P, k] (Laplace(0, 0.1), never 0).

    A hot set H of `hot` distinct indices is drawn uniformly from [0, n);
    worker p takes round(hot_fraction * k) indices from H without replacement
    and the rest from outside H, distinct.  Rows are shuffled: the result must
    not depend on input order."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([CFG_GTOPK, seed])))
    H = g.choice(n, size=hot, replace=False).astype(np.int64)
    hot_sorted = np.sort(H)
    n_hot = int(round(hot_fraction * k))
    n_cold = k - n_hot
    idx = np.empty((P, k), dtype=np.int32)
    val = np.empty((P, k), dtype=np.float32)
    for p in range(P):
        from_hot = g.choice(H, size=n_hot, replace=False)
        cold = np.zeros(0, dtype=np.int64)
        while cold.size < n_cold:
            cand = g.integers(0, n, size=2 * (n_cold - cold.size) + 16)
            pos = np.searchsorted(hot_sorted, cand)
            pos = np.minimum(pos, hot_sorted.size - 1)
            cand = cand[hot_sorted[pos] != cand]
            cold = np.unique(np.concatenate([cold, cand]))
        cold = g.permutation(cold)[:n_cold]
        row = np.concatenate([from_hot, cold])
        v = g.laplace(0.0, 0.1, k)
        while True:
            v32 = v.astype(np.float32)
            zero = v32 == 0
            if not zero.any():
                break
            v[zero] = g.laplace(0.0, 0.1, int(zero.sum()))
        perm = g.permutation(k)
        row, v32 = row[perm], v32[perm]
        idx[p] = row.astype(np.int32)
        val[p] = v32
    return idx, val


def mixture_gpu(n: int, sigma: float, p_out: float, b_out: float, seed: tuple, device="cuda",
                out=None, chunk: int = 1 << 26):
    """Same mixture as `mixture`, drawn on the GPU with torch's seeded Philox
    generator (float64 draws rounded to float32), for sizes where host
    generation would take minutes.  Laplace(0, b) is drawn by inverting its
    CDF from a uniform in (0, 1).  Returns a float32 torch tensor on `device`."""
    import torch
    s = 0
    for part in seed:
        s = (s * 1_000_003 + int(part) + 1) % (2 ** 61 - 1)
    gen = torch.Generator(device=device)
    gen.manual_seed(s)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    for lo in range(0, n, chunk):
        m = min(chunk, n - lo)
        x = torch.randn(m, dtype=torch.float64, device=device, generator=gen) * sigma
        hit = torch.rand(m, dtype=torch.float64, device=device, generator=gen) < p_out
        u = torch.rand(m, dtype=torch.float64, device=device, generator=gen) - 0.5
        lap = -b_out * torch.sign(u) * torch.log1p(-2.0 * u.abs())
        out[lo:lo + m] = torch.where(hit, lap, x).to(torch.float32)
        del x, hit, u, lap
    return out
