"""GPU parity of the decode chain with an attention block in every layer
(AttnDecodeChain: q4mv_norm of [Q; gate; K; V], q4_atq over per-layer
caches, q4mv_add of O, the fused MLP stages, the head and argmax, the
position advanced on the device): step by step and as replays of one
captured graph against the oracle's attn_chain_step, bit for bit, and 64
tokens of the 24-layer chain against the oracle's golden tokens and
logits hashes."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = 16
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "attn_chain_seed20261202.json")


def small_weights():
    return synth.attn_chain_weights(seed=31, layers=2, vocab=4096, max_pos=16)


@pytest.mark.parametrize("use_graph", [False, True])
def test_attn_chain_steps_bit_exact(use_graph):
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    print("attn chain, 2 layers, graph=%s" % use_graph, flush=True)
    w = small_weights()
    chain = AttnDecodeChain(w)
    s = torch.cuda.Stream()
    kc, vc = oracle.attn_caches(w)
    want_tok, want_logits = [], []
    tok = w["tok0"]
    for pos in range(6):
        logits, tok = oracle.attn_chain_step(w, tok, pos, kc, vc, nthreads=NTHREADS)
        want_tok.append(tok)
        want_logits.append(logits)
    got_logits = []
    toks = chain.run(w["tok0"], 6, s, use_graph=use_graph,
                     on_step=lambda i, c: got_logits.append(host(c.logits)))
    for i in range(6):
        assert_bits_equal(got_logits[i], want_logits[i], "step %d logits" % i)
    assert toks == want_tok
    for l, lw in enumerate(chain.layers):
        assert_bits_equal(host(lw["kc"]).ravel(), kc[l].ravel(), "layer %d kcache" % l)
        assert_bits_equal(host(lw["vc"]).ravel(), vc[l].ravel(), "layer %d vcache" % l)
    assert int(host(chain.pos)[0]) == 6
    ws = chain.atq_ws
    assert lib().q4_atq_status(ws, w["hq"], w["hkv"], s) == lib().Q4_OK


def test_attn_chain_24_layers_golden_tokens():
    """200 tokens of the 24-layer chain with attention through one captured
    graph with the mailbox wait: tokens and logits hashes as the oracle
    wrote them."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    g = json.load(open(GOLDEN))
    print("attn chain, 24 layers, %d golden tokens" % len(g["tokens"]), flush=True)
    w = synth.attn_chain_weights(seed=g["seed"])
    assert w["tok0"] == g["tok0"] and w["max_pos"] == g["max_pos"]
    chain = AttnDecodeChain(w)
    s = torch.cuda.Stream()
    hashes = []
    toks = chain.run(g["tok0"], len(g["tokens"]), s, wait="mailbox",
                     on_step=lambda i, c: hashes.append(oracle.fnv1a32(host(c.logits))))
    assert toks == g["tokens"]
    assert hashes == g["logits_fnv1a32"]


def test_attn_chain_past_one_span():
    """Three steps at positions 700..702 of a 1024-position cache (earlier
    rows zero, as the oracle's fresh caches): the attention step's span
    exchanges run inside the captured graph."""
    from affine_q4_matvec_amd.chain import AttnDecodeChain
    w = synth.attn_chain_weights(seed=33, layers=2, vocab=4096, max_pos=1024)
    chain = AttnDecodeChain(w)
    s = torch.cuda.Stream()
    kc, vc = oracle.attn_caches(w)
    want, tok = [], w["tok0"]
    for pos in range(700, 703):
        logits, tok = oracle.attn_chain_step(w, tok, pos, kc, vc, nthreads=NTHREADS)
        want.append((tok, logits))
    got = []
    toks = chain.run(w["tok0"], 3, s, pos0=700, on_step=lambda i, c: got.append(host(c.logits)))
    assert toks == [t for t, _ in want]
    for i, (_, logits) in enumerate(want):
        assert_bits_equal(got[i], logits, "step %d logits" % i)
    for l, lw in enumerate(chain.layers):
        assert_bits_equal(host(lw["kc"]).ravel(), kc[l].ravel(), "layer %d kcache" % l)
    assert lib().q4_atq_status(chain.atq_ws, w["hq"], w["hkv"], s) == lib().Q4_OK
