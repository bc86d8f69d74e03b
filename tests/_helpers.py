"""Helpers shared by the GPU parity tests (no sparsifier arithmetic here)."""
import numpy as np
import torch


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def keys(a):
    return bits(a) & np.uint32(0x7FFFFFFF)


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_topk(tgs, grad, res, k):
    """Runs the HIP path on copies of host arrays; returns host results after
    checking the device error word."""
    g, r = gpu(grad), gpu(res)
    return topk_dev(tgs, g, r, k)


def topk_dev(tgs, g, r, k):
    """Top-k step on device tensors (residual `r` updated in place) with its own
    workspace; raises if a kernel flagged an error."""
    ws = tgs.workspace("topk", tgs.topk_workspace_bytes(g.numel(), k), g.device)
    idx, val = tgs.topk_ef_step(g, r, k, ws=ws)
    tgs.check_device_error(ws)
    return host(idx), host(val), host(r)


def assert_topk_equal(got, exp, what=""):
    gi, gv, gr = got
    ei, ev, er = exp
    assert gi.shape == ei.shape, what
    mism = np.nonzero(gi != ei)[0]
    assert mism.size == 0, "%s: %d index mismatches, first at %d (%d vs %d)" % (
        what, mism.size, mism[0], gi[mism[0]], ei[mism[0]])
    assert np.array_equal(bits(gv), bits(ev)), what + ": values differ"
    bad = np.nonzero(bits(gr) != bits(er))[0]
    assert bad.size == 0, "%s: %d residual mismatches, first at %d" % (what, bad.size, bad[0])


def check_topk_invariants(acc, res_after, idx, val, k):
    """Certifies the unique top-k answer at any size (O(n) numpy)."""
    n = acc.size
    assert idx.size == k and val.size == k
    ka = keys(acc)
    if k:
        assert idx.min() >= 0 and idx.max() < n
        sel = np.zeros(n, dtype=bool)
        sel[idx] = True
        assert int(sel.sum()) == k, "repeated index"
        assert np.array_equal(bits(val), bits(acc[idx]))
        ko = ka[idx].astype(np.int64)
        assert np.all((ko[:-1] > ko[1:]) | ((ko[:-1] == ko[1:]) & (idx[:-1] < idx[1:]))), "output order"
        kmin = ka[idx[-1]]
        assert np.all(bits(res_after[idx]) == 0)
        uns = ~sel
        del sel
        if k < n:
            kmax_uns = ka[uns].max()
            assert kmin >= kmax_uns
            if kmin == kmax_uns:
                tie_uns = np.nonzero(uns & (ka == kmin))[0]
                tie_sel = idx[ka[idx] == kmin]
                assert tie_sel.max() < tie_uns.min(), "tie rule"
        assert np.array_equal(bits(res_after)[uns], bits(acc)[uns])
    else:
        assert np.array_equal(bits(res_after), bits(acc))
