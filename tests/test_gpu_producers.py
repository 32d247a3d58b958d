"""GPU parity of rmsq, swq, argmax and embed against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [64, 128, 192, 2048, 6144, 8192])
def test_rmsq_bit_exact(n):
    q4 = lib()
    h = synth.normal_f32(1, "rh%d" % n, (n,), 0.0, 1.0)
    w = synth.normal_f32(1, "rw%d" % n, (n,), 1.0, 0.1)
    u, us = oracle.rmsq(h, w, 1e-6)
    ud, usd = q4.rmsq(dev(h), dev(w), 1e-6)
    torch.cuda.synchronize()
    assert_bits_equal(host(ud), u, "rmsq u n=%d" % n)
    assert_bits_equal(host(usd), us, "rmsq usum n=%d" % n)


def test_rmsq_edge_inputs():
    q4 = lib()
    n = 2048
    w = synth.normal_f32(2, "rw", (n,), 1.0, 0.1)
    for name, h in [("zero", np.zeros(n, np.float32)),
                    ("tiny", np.full(n, 1e-20, np.float32)),
                    ("const", np.full(n, -3.0, np.float32)),
                    ("large", synth.normal_f32(2, "big", (n,), 0.0, 1e15))]:
        u, us = oracle.rmsq(h, w, 1e-6)
        ud, usd = q4.rmsq(dev(h), dev(w), 1e-6)
        torch.cuda.synchronize()
        assert_bits_equal(host(ud), u, "rmsq " + name)
        assert_bits_equal(host(usd), us, "rmsq sums " + name)


def test_rmsq_2048_both_kernels():
    """n = 2048 runs a one-wave kernel when h, w and u are 16-byte aligned
    and the workgroup kernel otherwise: both give the oracle's bits."""
    q4 = lib()
    n = 2048
    h = synth.normal_f32(5, "ah", (n,), 0.0, 1.0)
    w = synth.normal_f32(5, "aw", (n,), 1.0, 0.1)
    u, us = oracle.rmsq(h, w, 1e-6)
    for off in (0, 1):
        hb = torch.zeros(n + 4, device="cuda")
        wb = torch.zeros(n + 4, device="cuda")
        ub = torch.zeros(n + 4, device="cuda")
        hb[off:off + n] = dev(h)
        wb[off:off + n] = dev(w)
        usd = torch.zeros(n // 64, device="cuda")
        q4.rmsq(hb[off:off + n], wb[off:off + n], 1e-6, ub[off:off + n], usd)
        torch.cuda.synchronize()
        assert_bits_equal(host(ub[off:off + n]), u, "rmsq u offset %d" % off)
        assert_bits_equal(host(usd), us, "rmsq usum offset %d" % off)


@pytest.mark.parametrize("n", [64, 6144])
def test_swq_fixed_bit_exact(n):
    q4 = lib()
    a = synth.normal_f32(3, "sa%d" % n, (2 * n,), 0.0, 3.0)
    o, os_ = oracle.swq(a, n)
    od, osd = q4.swq(dev(a), n)
    torch.cuda.synchronize()
    assert_bits_equal(host(od), o, "swq o")
    assert_bits_equal(host(osd), os_, "swq osum")


def test_swq_fixed_wide_range():
    """Gates over the whole range where exp's reduction, overflow and the
    binary64-to-binary32 rounding (including subnormal results) matter."""
    q4 = lib()
    n = 64 * 256
    g = np.concatenate([np.linspace(-800, 800, n // 2), synth.normal_f64(4, "sg", n // 2) * 20])
    up = synth.normal_f32(4, "su", (n,), 0.0, 2.0)
    a = np.concatenate([g.astype(np.float32), up])
    o, os_ = oracle.swq(a, n)
    od, osd = q4.swq(dev(a), n)
    torch.cuda.synchronize()
    assert_bits_equal(host(od), o, "swq wide o")
    assert_bits_equal(host(osd), os_, "swq wide osum")


def test_swq_fast_within_tolerance():
    q4 = lib()
    n = 6144
    a = synth.normal_f32(5, "sf", (2 * n,), 0.0, 3.0)
    o, _ = oracle.swq(a, n)
    od, _ = q4.swq(dev(a), n, mode=q4.FAST)
    torch.cuda.synchronize()
    o64 = o.astype(np.float64)
    rms = np.sqrt(np.mean(o64**2))
    assert np.all(np.abs(host(od) - o64) <= 1e-5 * np.abs(o64) + 1e-5 * rms)


def test_swq_rejects_n32():
    q4 = lib()
    with pytest.raises(q4.Q4Error):
        q4.swq(torch.zeros(64, device="cuda"), 32)


@pytest.mark.parametrize("n", [1, 100, 2048, 248320, 1 << 22])
def test_argmax(n):
    q4 = lib()
    v = synth.normal_f32(6, "am%d" % n, (n,), 0.0, 1.0)
    idx = q4.q4_argmax(dev(v))
    torch.cuda.synchronize()
    assert int(host(idx)[0]) == oracle.argmax(v)


def test_argmax_ties_nan_and_zero_signs():
    q4 = lib()
    n = 248320
    v = synth.normal_f32(7, "amt", (n,), 0.0, 1.0)
    v[200000] = 9.0
    v[123] = 9.0
    v[5000] = 9.0
    assert int(host(q4.q4_argmax(dev(v)))[0]) == oracle.argmax(v) == 123
    z = np.full(1000, -1.0, np.float32)
    z[10] = -0.0
    z[3] = 0.0
    z[700] = -0.0
    assert int(host(q4.q4_argmax(dev(z)))[0]) == oracle.argmax(z) == 3
    z[3] = -1.0
    assert int(host(q4.q4_argmax(dev(z)))[0]) == oracle.argmax(z) == 10
    v[100000] = np.nan
    assert int(host(q4.q4_argmax(dev(v)))[0]) == oracle.argmax(v) == -1
    w = np.full(777, -np.inf, np.float32)
    assert int(host(q4.q4_argmax(dev(w)))[0]) == oracle.argmax(w) == 0


def test_embed():
    q4 = lib()
    m = synth.q4_matrix(8, "emb", 1000, 2048)
    W = q4.Q4Matrix.from_host(m)
    for t in (0, 1, 517, 999):
        tok = torch.tensor([t], dtype=torch.int32, device="cuda")
        e = q4.q4_embed(W, tok)
        torch.cuda.synchronize()
        assert_bits_equal(host(e), oracle.embed(m, t), "embed %d" % t)
    for t in (-1, 1000):
        e = q4.q4_embed(W, torch.tensor([t], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert np.all(np.isnan(host(e))) and np.all(np.isnan(oracle.embed(m, t)))
