"""The kernel designs the pages compare, built into the library as
q4mv_variant: one lane per row ("Array.q4mv on Metal: one kernel thread per
row ..." (#1435), Change) and one wave per row with 1, 2, 4 or 8 rows per
block ("Metal: queued rmsq, swq, gdn and atq kernels and a 4-row q4mv ..."
(#1440), Change and Verification).  Every variant keeps the fixed tree, so
in fixed mode each must equal the oracle bit for bit; in fast mode each is
within the fast-mode bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = 16
VARIANTS = [0, 1, 2, 4, 8]


def _within_fast_bound(got, want):
    got, w64 = np.asarray(got, np.float64), np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(w64**2))
    err = np.abs(got - w64)
    assert np.all(err <= 1e-5 * np.abs(w64) + 1e-5 * rms), err.max()


# 13 rows (one partial block), a ragged count that fills several blocks per
# wave, and one that makes the lane-per-row kernel loop over its grid
@pytest.mark.parametrize("rows", [13, 4099, 530001])
@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_matches_oracle(variant, rows):
    print("q4mv_variant %d, %d x 2048" % (variant, rows), flush=True)
    q4 = lib()
    m = synth.small_product(seed=41, rows=rows, cols=2048, name="var%d" % rows)
    xs = oracle.group_sums(m["x"])
    W = q4.Q4Matrix.from_host(m)
    xd, xsd = dev(m["x"]), dev(xs)
    want = oracle.q4mv(m, m["x"], xs, NTHREADS)
    y = torch.full((rows,), 7.0, device="cuda")
    q4.q4mv_variant(W, xd, xsd, y, variant, mode=q4.FIXED)
    torch.cuda.synchronize()
    assert_bits_equal(host(y), want, "variant %d fixed, %d rows" % (variant, rows))
    y.fill_(7.0)
    q4.q4mv_variant(W, xd, xsd, y, variant, mode=q4.FAST)
    torch.cuda.synchronize()
    _within_fast_bound(host(y), want)


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_large_activations(variant):
    # an activation of 2^120: products near binary32 overflow, the same bits
    # as the oracle
    q4 = lib()
    m = synth.small_product(seed=42, rows=515, cols=2048, name="varbig")
    x = m["x"].copy()
    x[77] = np.float32(2.0**120)
    xs = oracle.group_sums(x)
    W = q4.Q4Matrix.from_host(m)
    y = torch.empty(515, device="cuda")
    q4.q4mv_variant(W, dev(x), dev(xs), y, variant, mode=q4.FIXED)
    torch.cuda.synchronize()
    assert_bits_equal(host(y), oracle.q4mv(m, x, xs), "variant %d with 2^120" % variant)


def test_variant_rejects_other_widths_and_names():
    q4 = lib()
    m = synth.small_product(seed=43, rows=8, cols=1024, name="varw")
    W = q4.Q4Matrix.from_host(m)
    x = dev(m["x"])
    xs = dev(oracle.group_sums(m["x"]))
    y = torch.empty(8, device="cuda")
    for v in (0, 4):
        with pytest.raises(q4.Q4Error):
            q4.q4mv_variant(W, x, xs, y, v)
    m2 = synth.small_product(seed=43, rows=8, cols=2048, name="varn")
    W2 = q4.Q4Matrix.from_host(m2)
    with pytest.raises(q4.Q4Error):
        q4.q4mv_variant(W2, dev(m2["x"]), dev(oracle.group_sums(m2["x"])), y, 3)
