"""GPU parity of the fused stages against the oracle's separate steps:
group sums formed in the kernel, rmsq as a product's prologue, SwiGLU as an
epilogue over interleaved (gate, up) rows, argmax as the head's epilogue."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = 16


@pytest.mark.parametrize("rows,cols", [(13, 128), (5, 192), (1000, 2048), (31, 6144), (7, 3072),
                                       (3, 32768)])
def test_q4mv_forms_group_sums(rows, cols):
    q4 = lib()
    m = synth.small_product(seed=21, rows=rows, cols=cols, name="xs%d_%d" % (rows, cols))
    want = oracle.q4mv(m, m["x"], oracle.group_sums(m["x"]), NTHREADS)
    W = q4.Q4Matrix.from_host(m)
    y = q4.q4mv(W, dev(m["x"]), None)
    torch.cuda.synchronize()
    assert_bits_equal(host(y), want, "q4mv xsum=None %dx%d" % (rows, cols))
    r = synth.normal_f32(21, "r%d" % rows, (rows,), 0.0, 3.0)
    y2 = q4.q4mv_add(W, dev(m["x"]), None, dev(r))
    torch.cuda.synchronize()
    assert_bits_equal(host(y2), oracle.add(r, want), "q4mv_add xsum=None")


@pytest.mark.parametrize("rows", [1, 13, 4096, 248320])
def test_q4mv_norm_equals_rmsq_then_q4mv(rows):
    q4 = lib()
    m = synth.q4_matrix(22, "norm%d" % rows, rows, 2048)
    h = synth.normal_f32(22, "nh", (2048,), 0.0, 3.0)
    wn = synth.normal_f32(22, "nw", (2048,), 1.0, 0.1)
    u, us = oracle.rmsq(h, wn, 1e-6)
    W = q4.Q4Matrix.from_host(m)
    ud = torch.empty(2048, device="cuda")
    usd = torch.empty(32, device="cuda")
    y = q4.q4mv_norm(W, dev(h), dev(wn), 1e-6, u=ud, usum=usd)
    torch.cuda.synchronize()
    assert_bits_equal(host(ud), u, "q4mv_norm u")
    assert_bits_equal(host(usd), us, "q4mv_norm usum")
    if rows > 100000:
        idx = np.unique(np.concatenate([np.random.default_rng(0).choice(rows, 4096, replace=False),
                                        [0, rows - 1]]))
        assert_bits_equal(host(y)[idx], oracle.q4mv_sample(m, u, us, idx), "q4mv_norm sampled")
    else:
        assert_bits_equal(host(y), oracle.q4mv(m, u, us, NTHREADS), "q4mv_norm y")
    # without the optional outputs
    y2 = q4.q4mv_norm(W, dev(h), dev(wn), 1e-6)
    torch.cuda.synchronize()
    assert_bits_equal(host(y2), host(y), "q4mv_norm without u")


def test_q4mv_norm_other_width_runs_two_steps():
    q4 = lib()
    m = synth.q4_matrix(23, "norm6144", 40, 6144)
    h = synth.normal_f32(23, "h6", (6144,), 0.0, 1.0)
    wn = synth.normal_f32(23, "w6", (6144,), 1.0, 0.1)
    u, us = oracle.rmsq(h, wn, 1e-6)
    W = q4.Q4Matrix.from_host(m)
    ud, usd = torch.empty(6144, device="cuda"), torch.empty(96, device="cuda")
    y = q4.q4mv_norm(W, dev(h), dev(wn), 1e-6, u=ud, usum=usd)
    torch.cuda.synchronize()
    assert_bits_equal(host(y), oracle.q4mv(m, u, us), "q4mv_norm 6144")
    with pytest.raises(q4.Q4Error):  # no scratch for u: refused, nothing launched
        q4.q4mv_norm(W, dev(h), dev(wn), 1e-6)


# n = 20032: 40064 interleaved rows, more than one 4-row block per wave,
# so the launch loops (the SwiGLU batches then span several blocks)
@pytest.mark.parametrize("n", [64, 6144, 20032])
def test_q4mv_norm_swiglu_equals_separate_steps(n):
    q4 = lib()
    from affine_q4_matvec_amd.chain import _interleave_rows
    gate = synth.q4_matrix(24, "g%d" % n, n, 2048, center=7.5)
    up = synth.q4_matrix(24, "u%d" % n, n, 2048, center=7.5)
    h = synth.normal_f32(24, "sh", (2048,), 0.0, 1.0)
    wn = synth.normal_f32(24, "sw", (2048,), 1.0, 0.1)
    u, us = oracle.rmsq(h, wn, 1e-6)
    a = np.concatenate([oracle.q4mv(gate, u, us, NTHREADS), oracle.q4mv(up, u, us, NTHREADS)])
    o, _ = oracle.swq(a, n)
    W = q4.Q4Matrix.from_host(_interleave_rows(gate, up))
    m = q4.q4mv_norm_swiglu(W, dev(h), dev(wn), 1e-6)
    torch.cuda.synchronize()
    assert_bits_equal(host(m), o, "q4mv_norm_swiglu n=%d" % n)
    with pytest.raises(q4.Q4Error):  # odd row count
        odd = synth.q4_matrix(24, "odd", 5, 2048)
        q4.q4mv_norm_swiglu(q4.Q4Matrix.from_host(odd), dev(h), dev(wn), 1e-6)


@pytest.mark.parametrize("rows", [7, 8192, 248320])
def test_q4mv_norm_argmax_repeated_calls(rows):
    q4 = lib()
    m = synth.q4_matrix(25, "am%d" % rows, rows, 2048)
    W = q4.Q4Matrix.from_host(m)
    y = torch.empty(rows, device="cuda")
    idx = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    state = torch.full((q4.q4mv_argmax_ws_bytes() // 8,), -1, dtype=torch.int64, device="cuda")
    for k in range(3):  # several calls on one workspace (left dirty on purpose)
        h = synth.normal_f32(25, "ah%d" % k, (2048,), 0.0, 1.0)
        wn = synth.normal_f32(25, "aw%d" % k, (2048,), 1.0, 0.1)
        u, us = oracle.rmsq(h, wn, 1e-6)
        want = oracle.q4mv(m, u, us, NTHREADS)
        q4.q4mv_norm_argmax(W, dev(h), dev(wn), 1e-6, y, idx, state)
        torch.cuda.synchronize()
        assert_bits_equal(host(y), want, "argmax logits call %d" % k)
        assert int(host(idx)[0]) == oracle.argmax(want), k


def test_q4mv_norm_argmax_ties_and_nan():
    q4 = lib()
    from test_oracle_pins import mat_from
    rows = 3000
    codes = np.zeros((rows, 2048), np.int64)
    b = np.zeros((rows, 32), np.float32)
    b[[2999, 17, 1500], :] = 1.0  # three rows tie at the maximum
    m = mat_from(codes, np.ones((rows, 32)), b)
    W = q4.Q4Matrix.from_host(m)
    h = np.ones(2048, np.float32)
    wn = np.ones(2048, np.float32)
    y = torch.empty(rows, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    q4.q4mv_norm_argmax(W, dev(h), dev(wn), 1e-6, y, idx)
    torch.cuda.synchronize()
    assert int(host(idx)[0]) == oracle.argmax(host(y)) == 17
    # a workspace of 8 bytes: one workgroup does every row
    small = torch.empty(1, dtype=torch.int64, device="cuda")
    q4.q4mv_norm_argmax(W, dev(h), dev(wn), 1e-6, y, idx, small)
    torch.cuda.synchronize()
    assert int(host(idx)[0]) == 17
    h[5] = np.nan
    q4.q4mv_norm_argmax(W, dev(h), dev(wn), 1e-6, y, idx)
    torch.cuda.synchronize()
    assert int(host(idx)[0]) == -1


def test_fused_and_unfused_chain_agree():
    lib()
    from affine_q4_matvec_amd.chain import DecodeChain
    w = synth.chain_weights(seed=26, layers=3, vocab=6000)
    s = torch.cuda.Stream()
    logs = {}
    for fused in (False, True):
        c = DecodeChain(w, fused=fused)
        lg = []
        toks = c.run(w["tok0"], 6, s, on_step=lambda i, ch: lg.append(host(ch.logits)))
        logs[fused] = (toks, lg)
    assert logs[False][0] == logs[True][0]
    for a, b in zip(logs[False][1], logs[True][1]):
        assert_bits_equal(b, a, "fused vs unfused logits")
    want, _ = oracle.chain_step(w, w["tok0"], nthreads=NTHREADS)
    assert_bits_equal(logs[True][1][0], want, "fused chain vs oracle, step 0")
