"""The host flag wait (mailbox): a one-thread kernel copies device values
into pinned host memory and publishes a sequence number the host spins on,
directly, inside captured graphs, and as the decode chain's per-token wait."""
import json
import os

import pytest
import torch

import synth
from gpu_util import lib

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "chain_seed%d.json" % synth.DEFAULT_SEED)


def test_mailbox_posts_in_order_and_times_out():
    q4 = lib()
    mb = q4.Mailbox(3)
    assert mb.seq == 0
    s = torch.cuda.Stream()
    vals = [torch.tensor([i, -i, 7 * i], dtype=torch.int32, device="cuda") for i in range(1, 6)]
    torch.cuda.synchronize()
    for v in vals:
        mb.post(v, stream=s)
    assert mb.wait(5) == [5, -5, 35]
    assert mb.seq == 5
    # a number that is never posted: the bounded spin gives up
    with pytest.raises(q4.Q4Error) as e:
        mb.wait(6, timeout_ms=20)
    assert e.value.code == q4.Q4_ETIMEOUT
    mb.close()


def test_mailbox_post_in_graph_replays():
    q4 = lib()
    mb = q4.Mailbox(1)
    s = torch.cuda.Stream()
    v = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    g = q4.Graph(s)
    g.begin()
    try:
        with torch.cuda.stream(s):
            v.add_(1)  # a device-side counter, read by the post
        mb.post(v, stream=s)
    finally:
        g.end()
    for i in range(1, 6):
        g.launch(s)
        assert mb.wait(i) == [i]
    s.synchronize()
    g.close()
    mb.close()


def test_chain_mailbox_wait_golden_tokens():
    """The persistent chain with the host waiting on the mailbox decodes
    the oracle's golden tokens."""
    from affine_q4_matvec_amd.chain import DecodeChain
    ref = json.load(open(GOLDEN))
    w = synth.chain_weights(seed=ref["seed"])
    chain = DecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    toks = chain.run(ref["tok0"], 40, s, wait="mailbox")
    assert toks == ref["tokens"][:40]
    again = chain.run(ref["tok0"], 5, s, wait="stream")
    assert again == ref["tokens"][:5]


def test_queue_waits_on_mailbox():
    """q4mv_wait on a mailbox: the product set of two layers, one wait,
    every product bit-exact; switching back to the stream wait works."""
    import numpy as np
    import oracle
    from gpu_util import assert_bits_equal, dev, host
    q4 = lib()
    ps = synth.product_set(seed=5, layers=2, vocab=4096)
    xs_host = {c: oracle.group_sums(x) for c, x in ps["x"].items()}
    xd = {c: dev(x) for c, x in ps["x"].items()}
    xsd = {c: dev(v) for c, v in xs_host.items()}
    queue = q4.Queue()
    queue.set_wait(q4.WAIT_MAILBOX, timeout_ms=5000)
    for rep in range(2):
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
        torch.cuda.synchronize()  # the uploads above ran on torch's stream
        queue.q4mv_wait()
        for m, W, y in keep[-3:]:
            got = host(y)
            idx = np.unique(np.linspace(0, m["rows"] - 1, 64).astype(np.int64))
            assert_bits_equal(got[idx], oracle.q4mv_sample(m, ps["x"][m["cols"]],
                                                           xs_host[m["cols"]], idx), m["name"])
        queue.set_wait(q4.WAIT_STREAM if rep == 0 else q4.WAIT_MAILBOX)
    queue.close()
