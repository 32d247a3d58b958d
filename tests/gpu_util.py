"""Helpers shared by the GPU tests: device copies of synthetic inputs and
bitwise comparison."""
import numpy as np
import torch


def lib():
    import affine_q4_matvec_amd as q4
    return q4


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a.view(np.uint32)


def assert_bits_equal(got, want, what=""):
    """Bitwise equality; NaNs compare by NaN-ness only (their payloads are
    not part of the method)."""
    got = np.array(got, dtype=np.float32, copy=True)
    want = np.array(want, dtype=np.float32, copy=True)
    gn, wn = np.isnan(got), np.isnan(want)
    if gn.shape == wn.shape and np.array_equal(gn, wn):
        got[gn] = 0.0
        want[wn] = 0.0
    g, w = bits(got), bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError("%s: %d of %d values differ; first at %d: got %r want %r"
                             % (what, bad.size, g.size, i, float(np.asarray(got).ravel()[i]),
                                float(np.asarray(want).ravel()[i])))

