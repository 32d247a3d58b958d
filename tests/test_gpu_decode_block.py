"""GPU parity of the persistent decoder layers (q4_decode_blocks and
q4_decode_block: the attention block and the MLP block of every layer in
one launch whose stages hand their outputs to each other through tagged
words), driven through AttnDecodeChain(persistent=True): step by step and
as graph replays against the oracle's attn_chain_step, bit for bit, for 1
to 16 key/value heads; 200 tokens of the 24-layer chain against the
oracle's golden file; the hidden state after a stack of layers and after
single-layer launches against the oracle's; the bounded waits; positions
outside the cache."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = 16
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "attn_chain_seed20261202.json")


def oracle_steps(w, steps, pos0=0):
    kc, vc = oracle.attn_caches(w)
    out, tok = [], w["tok0"]
    for pos in range(pos0, pos0 + steps):
        logits, tok = oracle.attn_chain_step(w, tok, pos, kc, vc, nthreads=NTHREADS)
        out.append((tok, logits))
    return out, kc, vc


@pytest.mark.parametrize("hkv,use_graph", [(4, False), (4, True), (1, True), (2, False),
                                           (16, True)])
def test_block_chain_bit_exact(hkv, use_graph):
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    print("decode block: 2 layers, hkv %d, graph %s" % (hkv, use_graph), flush=True)
    w = synth.attn_chain_weights(seed=40 + hkv, layers=2, vocab=4096, hkv=hkv, max_pos=32)
    want, kc, vc = oracle_steps(w, 5)
    chain = AttnDecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    got = []
    toks = chain.run(w["tok0"], 5, s, use_graph=use_graph,
                     on_step=lambda i, c: got.append(host(c.logits)))
    for i, (_, logits) in enumerate(want):
        assert_bits_equal(got[i], logits, "step %d logits" % i)
    assert toks == [t for t, _ in want]
    for l, lw in enumerate(chain.layers):
        assert_bits_equal(host(lw["kc"]).ravel(), kc[l].ravel(), "layer %d kcache" % l)
        assert_bits_equal(host(lw["vc"]).ravel(), vc[l].ravel(), "layer %d vcache" % l)
    assert lib().q4_decode_block_status(chain.block_ws, s) == lib().Q4_OK


def test_block_chain_late_positions():
    """Steps at positions 250..254 of a 256-position cache (the whole span)."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    w = synth.attn_chain_weights(seed=45, layers=2, vocab=4096, max_pos=256)
    want, kc, _ = oracle_steps(w, 5, pos0=250)
    chain = AttnDecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    got = []
    toks = chain.run(w["tok0"], 5, s, pos0=250, on_step=lambda i, c: got.append(host(c.logits)))
    for i, (_, logits) in enumerate(want):
        assert_bits_equal(got[i], logits, "step %d logits" % i)
    assert toks == [t for t, _ in want]
    assert_bits_equal(host(chain.layers[1]["kc"]).ravel(), kc[1].ravel(), "layer 1 kcache")


def test_block_chain_24_layers_golden_tokens():
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    g = json.load(open(GOLDEN))
    print("decode block, 24 layers, %d golden tokens" % len(g["tokens"]), flush=True)
    w = synth.attn_chain_weights(seed=g["seed"])
    chain = AttnDecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    hashes = []
    toks = chain.run(g["tok0"], len(g["tokens"]), s, wait="mailbox",
                     on_step=lambda i, c: hashes.append(oracle.fnv1a32(host(c.logits))))
    assert toks == g["tokens"]
    assert hashes == g["logits_fnv1a32"]
    assert lib().q4_decode_block_status(chain.block_ws, s) == lib().Q4_OK


def test_block_waits_report_and_recover():
    """With the wait bound at zero the hand-offs give up at their first
    look: the status call reports Q4_ETIMEOUT and clears the workspace; the
    next step with the normal bound is bit-exact."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    q4 = lib()
    w = synth.attn_chain_weights(seed=46, layers=2, vocab=4096, max_pos=16)
    want, _, _ = oracle_steps(w, 1)
    chain = AttnDecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    os.environ["Q4_DECODE_TIMEOUT_MS"] = "-1"
    try:
        chain.run(w["tok0"], 1, s, use_graph=False)
    finally:
        del os.environ["Q4_DECODE_TIMEOUT_MS"]
    assert q4.q4_decode_block_status(chain.block_ws, s) == q4.Q4_ETIMEOUT
    got = []
    toks = chain.run(w["tok0"], 1, s, use_graph=False,
                     on_step=lambda i, c: got.append(host(c.logits)))
    assert toks == [want[0][0]]
    assert_bits_equal(got[0], want[0][1], "after a timeout")
    assert q4.q4_decode_block_status(chain.block_ws, s) == q4.Q4_OK


def test_block_position_outside_the_cache():
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    q4 = lib()
    w = synth.attn_chain_weights(seed=47, layers=1, vocab=4096, max_pos=16)
    chain = AttnDecodeChain(w, persistent=True)
    h = dev(np.ones(2048, np.float32))
    pos = torch.tensor([16], dtype=torch.int32, device="cuda")
    q4.q4_decode_block(chain.layers[0]["blk"], chain.eps, h, pos, chain.cos_tab, chain.sin_tab,
                       chain.block_ws)
    assert q4.q4_decode_block_status(chain.block_ws) == q4.Q4_OK
    assert np.all(np.isnan(host(h)))
    assert not np.any(host(chain.layers[0]["kc"]))  # no cache row written


def test_stack_and_single_layer_calls_against_oracle_hidden():
    """Three layers, three steps: the hidden state after every layer, from
    one q4_decode_blocks launch and from three q4_decode_block launches,
    each against the oracle's attn_chain_hidden bit for bit, and the caches
    of both against the oracle's."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    q4 = lib()
    print("decode blocks: stack of 3 layers vs 3 single-layer launches", flush=True)
    w = synth.attn_chain_weights(seed=48, layers=3, vocab=4096, hkv=2, max_pos=24)
    toks = [5, 17, 4000]
    kc, vc = oracle.attn_caches(w)
    want = [oracle.attn_chain_hidden(w, t, p, kc, vc, nthreads=NTHREADS)
            for p, t in enumerate(toks)]
    chain = AttnDecodeChain(w, persistent=True)
    assert len(chain.stacks) == 1
    zc = lambda: torch.zeros_like(chain.layers[0]["kc"])
    single = []
    for lw in chain.layers:
        single.append(q4.AttnBlock(lw["qgkv"], lw["o"], lw["wa"], lw["wq"], lw["wk"], zc(), zc(),
                                   q4.MlpLayer(lw["gu"], lw["down"], lw["wn"])))
    ws2 = torch.zeros_like(chain.block_ws)
    s = torch.cuda.Stream()
    for p, t in enumerate(toks):
        tok = torch.tensor([t], dtype=torch.int32, device="cuda")
        pos = torch.tensor([p], dtype=torch.int32, device="cuda")
        h1 = torch.empty(2048, device="cuda")
        h2 = torch.empty(2048, device="cuda")
        q4.q4_embed(chain.head, tok, h1, stream=s)
        q4.q4_embed(chain.head, tok, h2, stream=s)
        q4.q4_decode_blocks(chain.stacks[0], chain.eps, h1, pos, chain.cos_tab, chain.sin_tab,
                            chain.block_ws, stream=s)
        for blk in single:
            q4.q4_decode_block(blk, chain.eps, h2, pos, chain.cos_tab, chain.sin_tab, ws2,
                               stream=s)
        s.synchronize()
        assert_bits_equal(host(h1), want[p], "stack, step %d" % p)
        assert_bits_equal(host(h2), want[p], "single layers, step %d" % p)
    for l in range(3):
        for name, kt, vt in (("stack", chain.layers[l]["kc"], chain.layers[l]["vc"]),
                             ("single", single[l].kcache, single[l].vcache)):
            assert_bits_equal(host(kt).ravel(), kc[l].ravel(), "%s layer %d kcache" % (name, l))
            assert_bits_equal(host(vt).ravel(), vc[l].ravel(), "%s layer %d vcache" % (name, l))
    assert q4.q4_decode_block_status(chain.block_ws, s) == q4.Q4_OK
    assert q4.q4_decode_block_status(ws2, s) == q4.Q4_OK


def test_stack_position_outside_the_cache():
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    q4 = lib()
    w = synth.attn_chain_weights(seed=49, layers=2, vocab=4096, max_pos=16)
    chain = AttnDecodeChain(w, persistent=True)
    h = dev(np.ones(2048, np.float32))
    pos = torch.tensor([-1], dtype=torch.int32, device="cuda")
    q4.q4_decode_blocks(chain.stacks[0], chain.eps, h, pos, chain.cos_tab, chain.sin_tab,
                        chain.block_ws)
    assert q4.q4_decode_block_status(chain.block_ws) == q4.Q4_OK
    assert np.all(np.isnan(host(h)))
    for lw in chain.layers:
        assert not np.any(host(lw["kc"])) and not np.any(host(lw["vc"]))


@pytest.mark.parametrize("inter", [2048, 4096, 8192])
def test_block_chain_other_widths(inter):
    """The kernel's other MLP widths (1, 2 and 4 passes per down row): two
    layers, three steps against the oracle bit for bit."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    print("decode blocks: inter %d" % inter, flush=True)
    w = synth.attn_chain_weights(seed=50 + inter // 2048, layers=2, vocab=4096, inter=inter,
                                 max_pos=16)
    want, kc, _ = oracle_steps(w, 3)
    chain = AttnDecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    got = []
    toks = chain.run(w["tok0"], 3, s, on_step=lambda i, c: got.append(host(c.logits)))
    for i, (_, logits) in enumerate(want):
        assert_bits_equal(got[i], logits, "inter %d step %d logits" % (inter, i))
    assert toks == [t for t, _ in want]
    assert_bits_equal(host(chain.layers[1]["kc"]).ravel(), kc[1].ravel(), "layer 1 kcache")
    assert lib().q4_decode_block_status(chain.block_ws, s) == lib().Q4_OK


def test_block_chain_fast_mode_equals_stage_kernels():
    """Fast mode: the rows use the per-stage kernels' fast code and the
    attention step its one order, so the persistent engine decodes the same
    bits as the per-stage kernels in fast mode; and its logits stay within
    the fast order's error of the oracle's."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    q4 = lib()
    w = synth.attn_chain_weights(seed=54, layers=3, vocab=4096, max_pos=16)
    want, _, _ = oracle_steps(w, 4)
    s = torch.cuda.Stream()
    logits = {}
    toks = {}
    for persistent in (False, True):
        chain = AttnDecodeChain(w, mode=q4.FAST, persistent=persistent)
        got = []
        toks[persistent] = chain.run(w["tok0"], 4, s,
                                     on_step=lambda i, c: got.append(host(c.logits)))
        logits[persistent] = got
    for i in range(4):
        assert_bits_equal(logits[True][i], logits[False][i], "fast step %d" % i)
    assert toks[True] == toks[False]
    # the first step starts from the same token as the oracle's
    ref = want[0][1].astype(np.float64)
    err = np.abs(logits[True][0].astype(np.float64) - ref)
    assert err.max() <= 1e-4 * np.sqrt(np.mean(ref ** 2)), err.max()


@pytest.mark.parametrize("max_pos,pos0,hkv", [(1024, 254, 4), (1024, 766, 1), (2048, 1790, 16),
                                             (4096, 4092, 4)])
def test_block_chain_several_spans(max_pos, pos0, hkv):
    """Caches of 4 and 16 spans of 256 positions: one workgroup per head
    and span, the span maxima and sums exchanged as tagged words, steps
    that cross from one span into the next, against the oracle bit for
    bit."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    print("decode blocks: max_pos %d from %d, hkv %d" % (max_pos, pos0, hkv), flush=True)
    w = synth.attn_chain_weights(seed=60 + hkv, layers=2, vocab=4096, hkv=hkv, max_pos=max_pos)
    want, kc, vc = oracle_steps(w, 4, pos0=pos0)
    chain = AttnDecodeChain(w, persistent=True)
    s = torch.cuda.Stream()
    got = []
    toks = chain.run(w["tok0"], 4, s, pos0=pos0, on_step=lambda i, c: got.append(host(c.logits)))
    for i, (_, logits) in enumerate(want):
        assert_bits_equal(got[i], logits, "pos %d logits" % (pos0 + i))
    assert toks == [t for t, _ in want]
    for l in range(2):
        assert_bits_equal(host(chain.layers[l]["kc"]).ravel(), kc[l].ravel(), "layer %d kcache" % l)
        assert_bits_equal(host(chain.layers[l]["vc"]).ravel(), vc[l].ravel(), "layer %d vcache" % l)
    assert lib().q4_decode_block_status(chain.block_ws, s) == lib().Q4_OK


def test_stack_rejects_caches_of_other_lengths():
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    q4 = lib()
    w = synth.attn_chain_weights(seed=70, layers=2, vocab=4096, max_pos=32)
    chain = AttnDecodeChain(w, persistent=True)
    lw = chain.layers[1]
    short = q4.AttnBlock(lw["qgkv"], lw["o"], lw["wa"], lw["wq"], lw["wk"],
                         torch.zeros(w["hkv"], 16, 128, device="cuda"),
                         torch.zeros(w["hkv"], 16, 128, device="cuda"),
                         q4.MlpLayer(lw["gu"], lw["down"], lw["wn"]))
    with pytest.raises(ValueError):
        q4.BlockStack([chain.layers[0]["blk"], short])


LONG_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "attn_chain_long_seed20261202.json")


@pytest.mark.parametrize("persistent", [False, True])
def test_attn_chain_long_cache_golden_tokens(persistent):
    """200 tokens at positions 3896..4095 of a 4096-position cache (all 16
    spans of a head in use; earlier rows zero, as the oracle's fresh
    caches), both engines: tokens and logits hashes as the oracle wrote
    them."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    g = json.load(open(LONG_GOLDEN))
    print("attention chain at the end of a %d cache, persistent %s, %d golden tokens"
          % (g["max_pos"], persistent, len(g["tokens"])), flush=True)
    w = synth.attn_chain_weights(seed=g["seed"], max_pos=g["max_pos"])
    chain = AttnDecodeChain(w, persistent=persistent)
    s = torch.cuda.Stream()
    hashes = []
    toks = chain.run(g["tok0"], len(g["tokens"]), s, wait="mailbox", pos0=g["pos0"],
                     on_step=lambda i, c: hashes.append(oracle.fnv1a32(host(c.logits))))
    assert toks == g["tokens"]
    assert hashes == g["logits_fnv1a32"]
    assert lib().q4_atq_status(chain.atq_ws, w["hq"], w["hkv"], s) == lib().Q4_OK
    if persistent:
        assert lib().q4_decode_block_status(chain.block_ws, s) == lib().Q4_OK
