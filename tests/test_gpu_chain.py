"""GPU parity of the ordering layer: the stage queue with one host wait
(the 24-layer product set), graph capture and replay, and the greedy decode
chain compared with the oracle at every step."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "chain_seed%d.json" % synth.DEFAULT_SEED)


def chain_cls():
    lib()
    from affine_q4_matvec_amd.chain import DecodeChain
    return DecodeChain


# ---------------------------------------------------------------------------
# stage queue
# ---------------------------------------------------------------------------

def test_queue_product_set_two_layers_bit_exact():
    q4 = lib()
    ps = synth.product_set(seed=3, layers=2, vocab=4096)
    xs_host = {c: oracle.group_sums(x) for c, x in ps["x"].items()}
    xd = {c: dev(x) for c, x in ps["x"].items()}
    xsd = {c: dev(v) for c, v in xs_host.items()}
    mats, ys = [], []
    queue = q4.Queue()
    stage = 0
    for m in ps["products"]:
        if m["stage"] != stage:
            queue.q4_stage()
            stage = m["stage"]
        W = q4.Q4Matrix.from_host(m)
        y = torch.full((m["rows"],), 7.0, device="cuda")  # sentinel
        queue.q4mv_queue(W, xd[m["cols"]], xsd[m["cols"]], y)
        mats.append(W)
        ys.append(y)
    queue.q4mv_wait()
    for m, y in zip(ps["products"], ys):
        want = oracle.q4mv(m, ps["x"][m["cols"]], xs_host[m["cols"]], NTHREADS)
        assert_bits_equal(host(y), want, m["name"])
    queue.close()


def test_queue_stage_of_looping_products_bit_exact():
    """One stage of three 2048-column products large enough that the
    grouped launch loops (the device's 16-wave workgroups shared among the
    products in proportion, each workgroup's waves taking its blocks by
    tickets), ragged row counts, one wait."""
    q4 = lib()
    x = synth.normal_f32(31, "lx", (2048,), 0.0, 1.0)
    xs = oracle.group_sums(x)
    xd, xsd = dev(x), dev(xs)
    queue = q4.Queue()
    ms, ys, Ws = [], [], []
    for i, rows in enumerate((30001, 4099, 52223)):
        m = synth.q4_matrix(31, "lp%d" % i, rows, 2048)
        W = q4.Q4Matrix.from_host(m)
        y = torch.full((rows,), 7.0, device="cuda")  # sentinel
        queue.q4mv_queue(W, xd, xsd, y)
        ms.append(m)
        ys.append(y)
        Ws.append(W)
    queue.q4mv_wait()
    for i, (m, y) in enumerate(zip(ms, ys)):
        assert_bits_equal(host(y), oracle.q4mv(m, x, xs, NTHREADS), "looping product %d" % i)
    queue.close()


def test_queue_full_product_set_one_wait():
    """24 layers x 7 products + head, 97 stages, one host wait."""
    q4 = lib()
    ps = synth.product_set()
    assert ps["stages"] == 97 and len(ps["products"]) == 169
    xs_host = {c: oracle.group_sums(x) for c, x in ps["x"].items()}
    xd = {c: dev(x) for c, x in ps["x"].items()}
    xsd = {c: dev(v) for c, v in xs_host.items()}
    queue = q4.Queue()
    keep = []
    stage = 0
    for m in ps["products"]:
        if m["stage"] != stage:
            queue.q4_stage()
            stage = m["stage"]
        W = q4.Q4Matrix.from_host(m)
        y = torch.full((m["rows"],), 7.0, device="cuda")
        queue.q4mv_queue(W, xd[m["cols"]], xsd[m["cols"]], y)
        keep.append((m, W, y))
    queue.q4mv_wait()
    rng = np.random.default_rng(0)
    for m, W, y in keep:
        got = host(y)
        assert not np.any(got == 7.0), m["name"]
        idx = rng.choice(m["rows"], size=min(64, m["rows"]), replace=False)
        idx = np.unique(np.concatenate([idx, [0, m["rows"] - 1]]))
        want = oracle.q4mv_sample(m, ps["x"][m["cols"]], xs_host[m["cols"]], idx)
        assert_bits_equal(got[idx], want, m["name"])
    queue.close()


def test_queue_debug_overlap_check():
    q4 = lib()
    os.environ["Q4MV_DEBUG_CHECKS"] = "1"
    try:
        queue = q4.Queue()
    finally:
        del os.environ["Q4MV_DEBUG_CHECKS"]
    m = synth.small_product(seed=1, rows=64, cols=128, name="ov")
    W = q4.Q4Matrix.from_host(m)
    buf = torch.zeros(1024, device="cuda")
    xs = dev(oracle.group_sums(m["x"]))
    buf[:128] = dev(m["x"])
    y1 = buf[256:320]
    queue.q4mv_queue(W, buf[:128], xs, y1)
    # a second product of the same stage writing over the first one's x
    with pytest.raises(q4.Q4Error):
        queue.q4mv_queue(W, buf[512:640], xs, buf[64:128])
    queue.q4_stage()
    # in the next stage the same buffers are fine (ordered after the stage)
    queue.q4mv_queue(W, y1.repeat(2).contiguous(), xs, buf[640:704])
    queue.q4mv_wait()
    queue.close()


def test_wait_inside_capture_is_refused():
    q4 = lib()
    s = torch.cuda.Stream()
    queue = q4.Queue(stream=s)
    m = synth.small_product(seed=2, rows=64, cols=128, name="cap")
    W = q4.Q4Matrix.from_host(m)
    x, xs = dev(m["x"]), dev(oracle.group_sums(m["x"]))
    y = torch.empty(64, device="cuda")
    torch.cuda.synchronize()
    g = q4.Graph(s)
    g.begin()
    try:
        q4.q4mv(W, x, xs, y, stream=s)
        with pytest.raises(q4.Q4Error) as e:
            queue.q4mv_wait()
        assert e.value.code == q4.Q4_ESTATE
    finally:
        g.end()
    g.launch()
    s.synchronize()
    assert_bits_equal(host(y), oracle.q4mv(m, m["x"], oracle.group_sums(m["x"])), "captured q4mv")
    g.close()
    queue.close()


# ---------------------------------------------------------------------------
# the decode chain
# ---------------------------------------------------------------------------

def oracle_chain(w, tok, steps, layers=None):
    toks, logits = [], []
    for _ in range(steps):
        lg, tok = oracle.chain_step(w, tok, nthreads=NTHREADS, layers=layers)
        toks.append(tok)
        logits.append(lg)
    return toks, logits


@pytest.mark.parametrize("persistent", [False, True, "one_launch"])
def test_chain_two_layers_every_step_bit_exact(persistent):
    DecodeChain = chain_cls()
    w = synth.chain_weights(seed=7, layers=2, vocab=8192)
    want_toks, want_logits = oracle_chain(w, w["tok0"], 12)
    assert len(set(want_toks)) > 3
    for use_graph in (False, True):
        chain = DecodeChain(w, persistent=persistent is True,
                            one_launch=persistent == "one_launch")
        got_logits = []
        toks = chain.run(w["tok0"], 12, torch.cuda.Stream(), use_graph=use_graph,
                         on_step=lambda i, c: got_logits.append(host(c.logits)))
        assert toks == want_toks, use_graph
        for i, (g, wl) in enumerate(zip(got_logits, want_logits)):
            assert_bits_equal(g, wl, "logits step %d graph=%s" % (i, use_graph))


def test_chain_graph_replays_match_eager_with_work_between():
    """Replays of one captured step, with eager library work and host waits
    between them, equal eager steps."""
    q4 = lib()
    DecodeChain = chain_cls()
    w = synth.chain_weights(seed=8, layers=2, vocab=4096)
    eager = DecodeChain(w)
    s = torch.cuda.Stream()
    ref = eager.run(w["tok0"], 6, s, use_graph=False)
    graph = DecodeChain(w)
    graph.capture(s)
    graph.set_token(w["tok0"])
    torch.cuda.synchronize()
    other = synth.small_product(seed=9, rows=300, cols=2048, name="between")
    W = q4.Q4Matrix.from_host(other)
    xo, xso = dev(other["x"]), dev(oracle.group_sums(other["x"]))
    for i in range(6):
        graph.graph.launch(s)
        s.synchronize()
        assert int(host(graph.tok)[0]) == ref[i], i
        q4.q4mv(W, xo, xso)  # eager work between replays
        torch.cuda.synchronize()


def test_chain_full_depth_first_steps_bit_exact():
    DecodeChain = chain_cls()
    w = synth.chain_weights()
    want_toks, want_logits = oracle_chain(w, w["tok0"], 3)
    chain = DecodeChain(w)
    got = []
    toks = chain.run(w["tok0"], 3, torch.cuda.Stream(), on_step=lambda i, c: got.append(host(c.logits)))
    assert toks == want_toks
    for i in range(3):
        assert_bits_equal(got[i], want_logits[i], "full chain logits step %d" % i)


@pytest.mark.parametrize("engine", ["fused", "persistent", "one_launch"])
def test_chain_200_tokens_against_oracle_golden(engine):
    """200 greedy steps of the 24-layer chain in one captured graph; every
    token and every step's logits hash equal the oracle's (tests/golden,
    written by tests/golden/make_chain_golden.py from the oracle only)."""
    DecodeChain = chain_cls()
    ref = json.load(open(GOLDEN))
    w = synth.chain_weights(seed=ref["seed"])
    assert w["tok0"] == ref["tok0"]
    chain = DecodeChain(w, persistent=engine == "persistent", one_launch=engine == "one_launch")
    hashes = []
    toks = chain.run(ref["tok0"], len(ref["tokens"]), torch.cuda.Stream(),
                     on_step=lambda i, c: hashes.append(oracle.fnv1a32(host(c.logits))))
    assert toks == ref["tokens"]
    assert hashes == ref["logits_fnv1a32"]
    # resuming from step k (the chain carries only the token) reproduces the rest
    k = 150
    again = chain.run(ref["tokens"][k - 1], 20, torch.cuda.Stream())
    assert again == ref["tokens"][k:k + 20]


def test_two_chains_interleaved_equal_solo_runs():
    DecodeChain = chain_cls()
    w = synth.chain_weights(seed=11, layers=2, vocab=4096)
    s = torch.cuda.Stream()
    solo_a = DecodeChain(w).run(5, 8, s)
    solo_b = DecodeChain(w).run(4000, 8, s)
    a, b = DecodeChain(w), DecodeChain(w)
    ta, tb = 5, 4000
    got_a, got_b = [], []
    for _ in range(8):
        ta = a.run(ta, 1, s)[0]
        tb = b.run(tb, 1, s)[0]
        got_a.append(ta)
        got_b.append(tb)
    assert got_a == solo_a and got_b == solo_b


@pytest.mark.parametrize("mailbox", [False, True])
def test_queue_wait_trace_reports_each_wait(capfd, mailbox):
    """With Q4MV_TRACE=1 each q4mv_wait prints the products it waited for,
    their GPU time and the wall time since the first of them was launched
    ('Array.q4go/Array.q4wait queue Metal Q4 products ...' (#1437), Change:
    the trace of every wait); the products' results are unchanged."""
    import re
    q4 = lib()
    os.environ["Q4MV_TRACE"] = "1"
    try:
        queue = q4.Queue(stream=torch.cuda.Stream())
    finally:
        del os.environ["Q4MV_TRACE"]
    if mailbox:
        queue.set_wait(q4.WAIT_MAILBOX)
    m = synth.small_product(seed=5, rows=4099, cols=2048, name="tr")
    xs = oracle.group_sums(m["x"])
    W = q4.Q4Matrix.from_host(m)
    xd, xsd = dev(m["x"]), dev(xs)
    want = oracle.q4mv(m, m["x"], xs, NTHREADS)
    ys = [torch.empty(4099, device="cuda") for _ in range(6)]
    capfd.readouterr()
    for y in ys[:3]:  # stage 1: three products
        queue.q4mv_queue(W, xd, xsd, y)
    queue.q4_stage()
    for y in ys[3:5]:  # stage 2: two more, then one wait for all five
        queue.q4mv_queue(W, xd, xsd, y)
    queue.q4mv_wait()
    queue.q4mv_queue(W, xd, xsd, ys[5])  # a second wait for one product
    queue.q4mv_wait()
    err = capfd.readouterr().err
    lines = re.findall(r"q4mv_wait: (\d+) products, gpu ([0-9.]+) ms, wall ([0-9.]+) ms", err)
    assert [int(n) for n, _, _ in lines] == [5, 1], err
    for _, gpu, wall in lines:
        assert 0.0 < float(gpu) < 1000.0 and 0.0 < float(wall) < 10000.0
        assert float(wall) >= 0.5 * float(gpu)  # the wall time spans the GPU work
    for y in ys:
        assert_bits_equal(host(y), want, "traced queue product")
    queue.close()
