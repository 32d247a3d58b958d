"""GPU parity of the attention step (q4_atq): one decode token of gated
attention over key/value caches, bit for bit against the oracle's orc_atq
(outputs, group sums and the written cache rows), over positions that
span one to 64 chunks of 64 with ragged last chunks, head groupings from
1 to 8 queries per key/value head, cache lengths that are not multiples of
the chunk, a key row whose terms cancel only in the canonical order,
consecutive tokens that grow the caches in place, graph replays at
positions read on the device, and positions outside the cache."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu


def new_ws(q4, hq, hkv):
    n = q4.q4_atq_ws_bytes(hq, hkv)
    assert n > 0
    return torch.zeros((n + 255) // 256 * 64, dtype=torch.float32, device="cuda")


class Dev:
    """The inputs of one token on the device, and its outputs."""

    def __init__(self, a):
        self.q, self.g, self.k, self.v = (dev(a[n]) for n in ("q", "g", "k", "v"))
        self.wq, self.wk = dev(a["wq"]), dev(a["wk"])
        # the tables of every position; the token's row is the one in a
        # (which a test may have replaced)
        ct, st = a["cos_tab"].copy(), a["sin_tab"].copy()
        ct[a["pos"]], st[a["pos"]] = a["cos"], a["sin"]
        self.cs, self.sn = dev(ct), dev(st)
        self.pos = torch.tensor([a["pos"]], dtype=torch.int32, device="cuda")
        self.kc, self.vc = dev(a["kcache"]), dev(a["vcache"])
        self.o = torch.full((a["hq"] * 128,), 7.0, device="cuda")
        self.os = torch.full((a["hq"] * 2,), 7.0, device="cuda")
        self.eps = float(a["eps"])

    def run(self, q4, ws, stream=None):
        q4.q4_atq(self.q, self.g, self.k, self.v, self.wq, self.wk, self.eps, self.cs, self.sn,
                  self.kc, self.vc, self.pos, self.o, self.os, ws, stream)


def oracle_run(a):
    kc, vc = a["kcache"].copy(), a["vcache"].copy()
    o, os_ = oracle.atq(a["q"], a["g"], a["k"], a["v"], a["wq"], a["wk"], a["eps"], a["cos"],
                        a["sin"], kc, vc, a["pos"])
    return o, os_, kc, vc


def check(a, d, what):
    o, os_, kc, vc = oracle_run(a)
    torch.cuda.synchronize()
    assert_bits_equal(host(d.o), o, what + " o")
    assert_bits_equal(host(d.os), os_, what + " osum")
    assert_bits_equal(host(d.kc).ravel(), kc.ravel(), what + " kcache")
    assert_bits_equal(host(d.vc).ravel(), vc.ravel(), what + " vcache")


@pytest.mark.parametrize("pos", [0, 1, 63, 64, 204, 255, 256, 257, 1000, 4095])
def test_atq_bit_exact_positions(pos):
    q4 = lib()
    print("atq pos %d" % pos, flush=True)
    a = synth.atq_inputs(seed=100 + pos, pos=pos, max_pos=4096)
    d = Dev(a)
    ws = new_ws(q4, 16, 4)
    d.run(q4, ws)
    check(a, d, "pos %d" % pos)
    assert q4.q4_atq_status(ws, 16, 4) == q4.Q4_OK


@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 1), (4, 4), (16, 2), (24, 3), (128, 16)])
def test_atq_head_groups(hq, hkv):
    q4 = lib()
    print("atq hq %d hkv %d" % (hq, hkv), flush=True)
    a = synth.atq_inputs(seed=200 + hq, pos=300, hq=hq, hkv=hkv, max_pos=512)
    d = Dev(a)
    d.run(q4, new_ws(q4, hq, hkv))
    check(a, d, "hq %d hkv %d" % (hq, hkv))


@pytest.mark.parametrize("pos", [70, 99])
def test_atq_ragged_cache_length(pos):
    q4 = lib()
    a = synth.atq_inputs(seed=300 + pos, pos=pos, max_pos=100)
    d = Dev(a)
    d.run(q4, new_ws(q4, 16, 4))
    check(a, d, "max_pos 100 pos %d" % pos)


def test_atq_cancelling_key_row():
    """The score of [2^30, 1 x 63, -2^30, 1 x 63] against a unit query is 0
    in the canonical tree and 63 left to right."""
    q4 = lib()
    a = synth.atq_inputs(seed=79, pos=1, hq=4, hkv=2, max_pos=4)
    a["eps"] = np.float32(0.0)
    for n in ("q", "wq", "k", "cos"):
        a[n] = np.ones_like(a[n])
    a["wk"] = np.zeros_like(a["wk"])
    a["sin"] = np.zeros_like(a["sin"])
    a["g"] = np.full_like(a["g"], 40.0)
    row = np.ones(128, np.float32)
    row[0], row[64] = 2.0 ** 30, -(2.0 ** 30)
    a["kcache"][:, 0] = row
    d = Dev(a)
    d.run(q4, new_ws(q4, 4, 2))
    check(a, d, "cancelling key")


def test_atq_consecutive_tokens_grow_the_cache():
    """Tokens at positions 126..130 (crossing a chunk boundary), each
    writing its row into the caches that the next one reads; one workspace
    for all of them."""
    q4 = lib()
    a = synth.atq_inputs(seed=400, pos=126, max_pos=256)
    d = Dev(a)
    ws = new_ws(q4, 16, 4)
    kc, vc = a["kcache"].copy(), a["vcache"].copy()
    for pos in range(126, 131):
        t = synth.atq_inputs(seed=401 + pos, pos=pos, max_pos=pos + 1)
        b = dict(a, pos=pos, kcache=kc, vcache=vc, cos=t["cos"], sin=t["sin"])
        for n in ("q", "g", "k", "v"):
            b[n] = t[n]
            getattr(d, n).copy_(dev(t[n]))
        d.pos.fill_(pos)
        d.run(q4, ws)
        o, os_ = oracle.atq(b["q"], b["g"], b["k"], b["v"], b["wq"], b["wk"], b["eps"], b["cos"],
                            b["sin"], kc, vc, pos)
        torch.cuda.synchronize()
        assert_bits_equal(host(d.o), o, "token at %d" % pos)
        assert_bits_equal(host(d.os), os_, "token at %d osum" % pos)
    assert_bits_equal(host(d.kc).ravel(), kc.ravel(), "kcache after the tokens")
    assert_bits_equal(host(d.vc).ravel(), vc.ravel(), "vcache after the tokens")


def test_atq_in_graph_replays():
    """One captured q4_atq replayed at positions 204, 205 and 64 (the
    position is read on the device), with new inputs copied in between, and
    eager work and host synchronisations between the replays."""
    q4 = lib()
    a = synth.atq_inputs(seed=500, pos=204, max_pos=512)
    d = Dev(a)
    ws = new_ws(q4, 16, 4)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = q4.Graph(s)
    g.begin()
    try:
        d.run(q4, ws, stream=s)
    finally:
        g.end()
    for seed, pos in ((501, 204), (502, 205), (503, 64)):
        t = synth.atq_inputs(seed=seed, pos=pos, max_pos=512)
        for n in ("q", "g", "k", "v"):
            getattr(d, n).copy_(dev(t[n]))
        d.kc.copy_(dev(t["kcache"]))
        d.vc.copy_(dev(t["vcache"]))
        d.pos.fill_(pos)
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        b = dict(a, pos=pos, cos=t["cos"], sin=t["sin"],
                 **{n: t[n] for n in ("q", "g", "k", "v", "kcache", "vcache")})
        check(b, d, "replay seed %d pos %d" % (seed, pos))
        # eager work between replays: the same step outside the graph
        d.run(q4, new_ws(q4, 16, 4))
        torch.cuda.synchronize()
    g.close()


@pytest.mark.parametrize("pos", [-1, 100])
def test_atq_position_outside_the_cache(pos):
    """A position outside [0, max_pos): no cache row written, o and osum
    NaN."""
    q4 = lib()
    a = synth.atq_inputs(seed=600, pos=50, max_pos=100)
    d = Dev(a)
    d.pos.fill_(pos)
    d.run(q4, new_ws(q4, 16, 4))
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(d.o))) and np.all(np.isnan(host(d.os)))
    assert_bits_equal(host(d.kc).ravel(), a["kcache"].ravel(), "kcache untouched")
    assert_bits_equal(host(d.vc).ravel(), a["vcache"].ravel(), "vcache untouched")


def test_atq_bounded_waits_report_and_recover():
    """With the wait bound at zero (Q4_DECODE_TIMEOUT_MS < 0) the span
    exchanges of position 4095 give up at their first look: the status call
    reports Q4_ETIMEOUT and clears the workspace, and the next call with
    the normal bound is bit-exact."""
    import os
    q4 = lib()
    a = synth.atq_inputs(seed=700, pos=4095, max_pos=4096)
    d = Dev(a)
    ws = new_ws(q4, 16, 4)
    os.environ["Q4_DECODE_TIMEOUT_MS"] = "-1"
    try:
        d.run(q4, ws)
    finally:
        del os.environ["Q4_DECODE_TIMEOUT_MS"]
    assert q4.q4_atq_status(ws, 16, 4) == q4.Q4_ETIMEOUT
    d.kc.copy_(dev(a["kcache"]))
    d.vc.copy_(dev(a["vcache"]))
    d.run(q4, ws)
    check(a, d, "after a timeout")
    assert q4.q4_atq_status(ws, 16, 4) == q4.Q4_OK
