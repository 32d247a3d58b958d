"""q4mv_norm_argmax_noalloc (the head step with the argmax keys in the
library's static device array) against q4mv_norm_argmax with a caller
workspace, through the C ABI: the same logits bits and the same token, on
two calls in a row, the second smaller than the first, so that keys the
first call left in the shared array must not leak into the second."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = 16


def _head(rows: int, seed: int, plant: int, us) -> dict:
    m = synth.q4_matrix(seed, "na%d" % rows, rows, 2048)
    # a clear maximum at row `plant`: biases of 64 with the sign of each
    # group sum add 64 |us_g| over the 32 groups
    m["b"][plant, :] = np.where(us >= 0, np.float32(64.0), np.float32(-64.0))
    return m


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_matches_workspace_entry_point_twice(mode):
    q4 = lib()
    eps = 1e-6
    # first call: a looping launch (more blocks than resident waves), the
    # maximum in a workgroup past every workgroup of the second call
    calls = [(100000, 31, 8000), (3000, 32, 1234)]
    for k, (rows, seed, plant) in enumerate(calls):
        h = synth.normal_f32(seed, "nah", (2048,), 0.0, 1.0)
        wn = synth.normal_f32(seed, "naw", (2048,), 1.0, 0.1)
        u, us = oracle.rmsq(h, wn, eps)
        m = _head(rows, seed, plant, us)
        W = q4.Q4Matrix.from_host(m)
        hd, wnd = dev(h), dev(wn)
        y_ws = torch.empty(rows, device="cuda")
        y_na = torch.empty(rows, device="cuda")
        i_ws = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        i_na = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        q4.q4mv_norm_argmax(W, hd, wnd, eps, y_ws, i_ws, mode=mode)
        q4.q4mv_norm_argmax_noalloc(W, hd, wnd, eps, y_na, i_na, mode=mode)
        torch.cuda.synchronize()
        assert_bits_equal(host(y_na), host(y_ws), "noalloc logits, call %d" % k)
        assert int(host(i_na)[0]) == int(host(i_ws)[0]) == plant, k
        if mode == 0:
            want = oracle.q4mv(m, u, us, NTHREADS)
            assert_bits_equal(host(y_na), want, "noalloc logits against the oracle, call %d" % k)
            assert oracle.argmax(want) == plant


def test_noalloc_rejects_what_the_workspace_call_rejects():
    q4 = lib()
    m = synth.q4_matrix(33, "nr", 64, 1024)  # not 2048 columns
    W = q4.Q4Matrix.from_host(m)
    h = torch.zeros(1024, device="cuda")
    y = torch.empty(64, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.q4mv_norm_argmax_noalloc(W, h, h, 1e-6, y, idx)
    assert e.value.code == q4.Q4_EINVAL
