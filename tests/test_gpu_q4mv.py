"""GPU parity of q4mv (fixed and fast modes) and q4mv_add against the CPU
oracle, on the same seeded inputs.  Fixed mode must match bit for bit."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


def run_q4mv(m, x, xs, mode=0, resid=None):
    q4 = lib()
    W = q4.Q4Matrix.from_host(m)
    xd, xsd = dev(x), dev(xs)
    if resid is None:
        y = q4.q4mv(W, xd, xsd, mode=mode)
    else:
        y = q4.q4mv_add(W, xd, xsd, dev(resid), mode=mode)
    torch.cuda.synchronize()
    return host(y)


# Shapes: every segment width (G = 1, 2, 3, 5, 8, 16, 32), the split path
# (G = 33, 48, 96, 512), and ragged row counts that leave partial slots,
# partial waves and partial workgroups.
SHAPES = [(13, 128), (1, 64), (7, 64), (5, 192), (33, 320), (100, 512), (257, 1024),
          (1000, 2048), (1, 2048), (17, 2112), (9, 3072), (31, 6144), (3, 32768)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_q4mv_fixed_bit_exact(rows, cols):
    print("q4mv fixed %dx%d" % (rows, cols), flush=True)
    m = synth.small_product(seed=101, rows=rows, cols=cols, name="g%d_%d" % (rows, cols))
    xs = oracle.group_sums(m["x"])
    want = oracle.q4mv(m, m["x"], xs, NTHREADS)
    got = run_q4mv(m, m["x"], xs)
    assert_bits_equal(got, want, "q4mv %dx%d" % (rows, cols))


def test_q4mv_config0_13x128():
    m = synth.small_product(seed=synth.DEFAULT_SEED, rows=13, cols=128, name="c0")
    xs = oracle.group_sums(m["x"])
    assert_bits_equal(run_q4mv(m, m["x"], xs), oracle.q4mv(m, m["x"], xs), "13x128")


def test_q4mv_identity_and_one_hot():
    from test_oracle_pins import mat_from, unpack_codes
    rows, cols = 9, 192
    codes = np.zeros((rows, cols), np.int64)
    m = mat_from(codes, np.full((rows, 3), 0.01), np.ones((rows, 3)))
    x = synth.normal_f32(1, "idx", (cols,), 0.0, 1.0)
    xs = oracle.group_sums(x)
    y = run_q4mv(m, x, xs)
    assert_bits_equal(y, np.full(rows, oracle.tree(xs), np.float32), "identity")
    m = synth.q4_matrix(2, "onehot", rows, cols)
    codes = unpack_codes(m["q"], cols)
    for j in (0, 1, 7, 8, 63, 64, 100, 191):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        xs = np.zeros(3, np.float32)
        xs[j // 64] = 1.0
        got = run_q4mv(m, x, xs)
        g = j // 64
        want = (m["s"][:, g] * codes[:, j].astype(np.float32)).astype(np.float32) + m["b"][:, g]
        assert_bits_equal(got, want.astype(np.float32), "one-hot column %d" % j)


def test_q4mv_tree_order_adversarial():
    """Sums whose rounding reveals the tree shape at every level."""
    from test_oracle_pins import mat_from
    cols = 6144
    codes = np.ones((4, cols), np.int64)
    m = mat_from(codes, np.ones((4, 96)), np.zeros((4, 96)))
    cases = [
        {0: 2.0**24, 2048: 1.0, 4096: 1.0},  # pass level: (P0+P1)+P2
        {0: 2.0**24, 64: 1.0, 128: 1.0},     # group level inside a pass
        {0: 2.0**24, 128: 1.0, 192: 1.0},
        {0: 2.0**24, 2: 1.0, 3: 1.0},        # code level inside a group
        {0: 2.0**24, 32: 1.0, 33: 1.0},      # the two half-group chunks
        {0: 2.0**24, 8: 1.0, 16: 1.0},       # word level
    ]
    for case in cases:
        x = np.zeros(cols, np.float32)
        for k, v in case.items():
            x[k] = v
        xs = oracle.group_sums(x)
        assert_bits_equal(run_q4mv(m, x, xs), oracle.q4mv(m, x, xs), str(case))
    for c2048 in (2048, 128):
        m2 = mat_from(np.ones((3, c2048), np.int64), np.ones((3, c2048 // 64)),
                      np.zeros((3, c2048 // 64)))
        for case in ({0: 2.0**24, 64: 1.0, 128 % c2048: 1.0}, {0: 2.0**24, 33: 1.0, 34: 1.0}):
            x = np.zeros(c2048, np.float32)
            for k, v in case.items():
                x[k] = v
            xs = oracle.group_sums(x)
            assert_bits_equal(run_q4mv(m2, x, xs), oracle.q4mv(m2, x, xs), "%d %s" % (c2048, case))


@pytest.mark.parametrize("cols", [128, 2048, 6144])
def test_q4mv_special_values(cols):
    """Zeros of both signs, subnormal activations, and activations of 2^117
    and more (products up to 15 times those, near binary32 overflow)."""
    rows = 16
    m = synth.small_product(seed=3, rows=rows, cols=cols, name="spec%d" % cols)
    x = m["x"].copy()
    x[:32] = 0.0
    x[32:64] = -0.0
    x[64:96] = np.float32(1e-40)   # binary32 subnormals
    x[96:128] = np.float32(-3e-39)
    xs = oracle.group_sums(x)
    assert_bits_equal(run_q4mv(m, x, xs), oracle.q4mv(m, x, xs), "small values %d" % cols)
    for big in (np.float32(2.0**118), np.float32(1e37), np.float32(-3.4e38)):
        xb = x.copy()
        xb[cols - 5] = big
        xs = oracle.group_sums(xb)
        assert_bits_equal(run_q4mv(m, xb, xs), oracle.q4mv(m, xb, xs), "large %r %d" % (big, cols))
    xb = x.copy()
    xb[cols // 2] = np.float32(2.0**117)
    xs = oracle.group_sums(xb)
    assert_bits_equal(run_q4mv(m, xb, xs), oracle.q4mv(m, xb, xs), "2^117 %d" % cols)


def test_q4mv_nan_and_inf_propagate():
    rows, cols = 8, 2048
    m = synth.small_product(seed=4, rows=rows, cols=cols, name="nan")
    for bad in (np.inf, -np.inf, np.nan):
        x = m["x"].copy()
        x[700] = bad
        xs = oracle.group_sums(x)
        got, want = run_q4mv(m, x, xs), oracle.q4mv(m, x, xs)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        ok = ~np.isnan(want)
        assert_bits_equal(got[ok], want[ok], "non-NaN outputs with %r" % bad)


def test_q4mv_add_residual():
    m = synth.small_product(seed=4, rows=2048, cols=6144, name="res")
    xs = oracle.group_sums(m["x"])
    r = synth.normal_f32(4, "resid", (2048,), 0.0, 10.0)
    want = oracle.add(r, oracle.q4mv(m, m["x"], xs, NTHREADS))
    assert_bits_equal(run_q4mv(m, m["x"], xs, resid=r), want, "q4mv_add")
    # in place: y is the residual
    q4 = lib()
    W = q4.Q4Matrix.from_host(m)
    h = dev(r)
    q4.q4mv_add(W, dev(m["x"]), dev(xs), h, y=h)
    torch.cuda.synchronize()
    assert_bits_equal(host(h), want, "q4mv_add in place")


def test_q4mv_4096x2048_400_calls_hash():
    """4096 x 2048, 400 calls: every output identical to the oracle; the FNV-1a
    hash of the last output's bits equals the oracle's."""
    q4 = lib()
    m = synth.small_product(seed=synth.DEFAULT_SEED, rows=4096, cols=2048, name="c1")
    xs = oracle.group_sums(m["x"])
    want = oracle.q4mv(m, m["x"], xs, NTHREADS)
    W = q4.Q4Matrix.from_host(m)
    xd, xsd = dev(m["x"]), dev(xs)
    ys = torch.empty(400, 4096, dtype=torch.float32, device="cuda")
    for i in range(400):
        q4.q4mv(W, xd, xsd, y=ys[i])
    torch.cuda.synchronize()
    allb = host(ys).view(np.uint32)
    assert np.all(allb == bits(want)[None, :]), "some of the 400 outputs differ"
    assert oracle.fnv1a32(host(ys[-1])) == oracle.fnv1a32(want)


def test_q4mv_head_248320x2048_full():
    """The 248320 x 2048 output head with x from rmsq; every row bit-exact."""
    q4 = lib()
    h = synth.head_inputs()
    u, us = oracle.rmsq(h["z"], h["wn"], h["eps"])
    W = q4.Q4Matrix.from_host(h)
    ud, usd = q4.rmsq(dev(h["z"]), dev(h["wn"]), float(h["eps"]))
    torch.cuda.synchronize()
    assert_bits_equal(host(ud), u, "rmsq head input")
    assert_bits_equal(host(usd), us, "rmsq head group sums")
    y = q4.q4mv(W, ud, usd)
    torch.cuda.synchronize()
    want = oracle.q4mv(h, u, us, NTHREADS)
    assert_bits_equal(host(y), want, "head")


def test_q4mv_looping_launches_on_two_streams_at_once():
    """Two looping launches (41011 and 20483 rows) issued on two streams so
    that they can run at the same time, each with its own activations:
    the looping kernel's tickets live in each workgroup's LDS, so the
    launches share no state; both fixed-order outputs bit-exact."""
    q4 = lib()
    ms = [synth.small_product(seed=61 + i, rows=rows, cols=2048, name="two%d" % i)
          for i, rows in enumerate((41011, 20483))]
    wants = [oracle.q4mv(m, m["x"], oracle.group_sums(m["x"]), NTHREADS) for m in ms]
    Ws = [q4.Q4Matrix.from_host(m) for m in ms]
    xs = [(dev(m["x"]), dev(oracle.group_sums(m["x"]))) for m in ms]
    ys = [torch.full((m["rows"],), 7.0, device="cuda") for m in ms]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                q4.q4mv(Ws[i], xs[i][0], xs[i][1], ys[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert_bits_equal(host(ys[i]), wants[i], "stream %d rep %d" % (i, rep))


@pytest.mark.parametrize("rows", [20483, 61447])
@pytest.mark.parametrize("with_xsum", [True, False])
def test_q4mv_looping_launch_ragged(rows, with_xsum):
    """More rows than one 4-row block per resident wave, so that the
    looping kernel runs (each workgroup's 16 waves take its blocks by
    tickets; the activations read after the first block's loads), with a
    partial last block; the group sums given, or formed in the kernel.
    Fixed order bit-exact; fast order within its bound."""
    print("q4mv looping %dx2048 xsum %s" % (rows, with_xsum), flush=True)
    m = synth.small_product(seed=21, rows=rows, cols=2048, name="loop%d" % rows)
    xs = oracle.group_sums(m["x"])
    q4 = lib()
    W = q4.Q4Matrix.from_host(m)
    xd = dev(m["x"])
    xsd = dev(xs) if with_xsum else None
    want = oracle.q4mv(m, m["x"], xs, NTHREADS)
    y = q4.q4mv(W, xd, xsd, mode=0)
    torch.cuda.synchronize()
    assert_bits_equal(host(y), want, "looping fixed %d" % rows)
    y = q4.q4mv(W, xd, xsd, mode=1)
    torch.cuda.synchronize()
    got, w64 = host(y).astype(np.float64), want.astype(np.float64)
    rms = np.sqrt(np.mean(w64**2))
    err = np.abs(got - w64)
    assert np.all(err <= 1e-5 * np.abs(w64) + 1e-5 * rms), err.max()


@pytest.mark.parametrize("rows,cols", [(13, 128), (1000, 2048), (31, 6144), (5, 192)])
def test_q4mv_fast_within_tolerance(rows, cols):
    m = synth.small_product(seed=9, rows=rows, cols=cols, name="f%d_%d" % (rows, cols))
    xs = oracle.group_sums(m["x"])
    want = oracle.q4mv(m, m["x"], xs).astype(np.float64)
    got = run_q4mv(m, m["x"], xs, mode=1).astype(np.float64)
    rms = np.sqrt(np.mean(want**2))
    err = np.abs(got - want)
    assert np.all(err <= 1e-5 * np.abs(want) + 1e-5 * rms), err.max()


def test_q4mv_argument_errors():
    q4 = lib()
    m = synth.small_product(seed=1, rows=8, cols=128, name="err")
    W = q4.Q4Matrix.from_host(m)
    x = dev(m["x"])
    xs = dev(oracle.group_sums(m["x"]))
    y = torch.empty(8, device="cuda")
    with pytest.raises(q4.Q4Error):  # x misaligned for 16-byte loads
        big = torch.zeros(129, device="cuda")
        q4.q4mv(W, big[1:], xs, y)
    with pytest.raises(q4.Q4Error):  # y overlaps x
        buf = torch.zeros(256, device="cuda")
        buf[:128] = x
        q4.q4mv(W, buf[:128], xs, buf[64:72])
    with pytest.raises(q4.Q4Error):  # bad mode
        q4.q4mv(W, x, xs, y, mode=7)
    q4.q4mv(W, x, xs, y)  # the library still works afterwards
    torch.cuda.synchronize()


# Shapes whose kernels loop: the split kernel (rows over 2048-column passes)
# takes more than one block of 4 rows per workgroup past 4 x 2048 rows, with
# the next block's loads issued while the current one is summed; the seg
# kernel (rows under 2048 columns) strides over its grid past 16384 rows at
# 31 groups per row and past 32768 at 16.  Ragged tails in every case.
@pytest.mark.parametrize("rows,cols", [(8197, 6144), (8195, 2112), (16411, 1984), (32771, 1024)])
def test_q4mv_split_and_seg_loops(rows, cols):
    print("q4mv loop path %dx%d" % (rows, cols), flush=True)
    m = synth.small_product(seed=23, rows=rows, cols=cols, name="lp%d_%d" % (rows, cols))
    xs = oracle.group_sums(m["x"])
    want = oracle.q4mv(m, m["x"], xs, NTHREADS)
    got = run_q4mv(m, m["x"], xs, mode=0)
    assert_bits_equal(got, want, "loop path %dx%d" % (rows, cols))
    r = synth.normal_f32(23, "lpr%d" % rows, (rows,), 0.0, 2.0)
    q4 = lib()
    y = q4.q4mv_add(q4.Q4Matrix.from_host(m), dev(m["x"]), dev(xs), dev(r))
    torch.cuda.synchronize()
    assert_bits_equal(host(y), oracle.add(r, want), "loop path with residual %dx%d" % (rows, cols))
