"""GPU parity of the persistent decode-layers kernel (q4_decode_layers):
the embedding and every MLP layer of a decode step in one launch whose
workgroups hand m and h to each other through tagged words (h relayed
through each XCD's L2, with a fallback to the device-scope copy), against
the oracle's separate steps (bit-exact in fixed mode), against the
per-stage kernels in fast mode, inside a captured graph, and its bounded
waits."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host, lib

pytestmark = pytest.mark.gpu

NTHREADS = 16


def mlp_layers(q4, w, n=None):
    from affine_q4_matvec_amd.chain import _interleave_rows
    out = []
    for lw in w["layers"][:n]:
        gu = q4.Q4Matrix.from_host(_interleave_rows(lw["gate"], lw["up"]))
        out.append(q4.MlpLayer(gu, q4.Q4Matrix.from_host(lw["down"]), dev(lw["wn"])))
    return out


def new_ws(q4):
    return torch.zeros((q4.q4_decode_layers_ws_bytes() + 7) // 8, dtype=torch.int64,
                       device="cuda")




def run_layers(q4, emb, layers, w, tok, mode=0, ws=None):
    t = torch.tensor([tok], dtype=torch.int32, device="cuda")
    h = torch.full((2048,), 7.0, device="cuda")
    if ws is None:
        ws = new_ws(q4)
    q4.q4_decode_layers(emb, t, layers, w["eps"], h, ws, mode=mode)
    assert q4.q4_decode_layers_status(ws) == q4.Q4_OK
    return host(h), ws


@pytest.mark.parametrize("inter,nlayers", [(2048, 1), (4096, 2), (6144, 3), (8192, 2)])
def test_decode_layers_bit_exact(inter, nlayers):
    q4 = lib()
    w = synth.chain_weights(seed=40 + inter // 2048, layers=nlayers, inter=inter, vocab=3000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    ws = None
    for tok in (w["tok0"], 0, 2999):
        want = oracle.chain_hidden(w, tok, NTHREADS)
        got, ws = run_layers(q4, emb, layers, w, tok, ws=ws)
        print("decode_layers inter=%d layers=%d tok=%d" % (inter, nlayers, tok), flush=True)
        assert_bits_equal(got, want, "h inter=%d layers=%d tok=%d" % (inter, nlayers, tok))


def test_decode_layers_large_m():
    """One value of m near 2^120 (gate and up of one pair near 2^60): down
    products near the top of the binary32 range; every h bit as the
    oracle's."""
    q4 = lib()
    w = synth.chain_weights(seed=47, layers=1, inter=2048, vocab=300)
    tok = 11
    w["head"]["s"][tok, :] = 0.0  # h = the embedding row = all ones
    w["head"]["b"][tok, :] = 1.0
    lw = w["layers"][0]
    for name in ("gate", "up"):
        lw[name]["s"][5, :] = 0.0
        lw[name]["b"][5, :] = np.float32(2.0**49)
    want = oracle.chain_hidden(w, tok, NTHREADS)
    assert np.all(np.isfinite(want)) and np.max(np.abs(want)) > 2.0**100
    got, _ = run_layers(q4, q4.Q4Matrix.from_host(w["head"]), mlp_layers(q4, w), w, tok)
    assert_bits_equal(got, want, "h with m near 2^120")


def test_decode_layers_token_out_of_range_gives_nan():
    q4 = lib()
    w = synth.chain_weights(seed=45, layers=1, vocab=500)
    emb = q4.Q4Matrix.from_host(w["head"])
    got, _ = run_layers(q4, emb, mlp_layers(q4, w), w, 500)
    assert np.all(np.isnan(got))
    got, _ = run_layers(q4, emb, mlp_layers(q4, w), w, -1)
    assert np.all(np.isnan(got))


def test_decode_layers_fast_mode_equals_stage_kernels():
    """Fast mode: the same code as the per-stage fused kernels, so the same
    bits as q4mv_norm_swiglu + q4mv_add in fast mode; and within the fast
    mode's error of the fixed result."""
    q4 = lib()
    w = synth.chain_weights(seed=46, layers=4, vocab=2000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    tok = w["tok0"]
    got, _ = run_layers(q4, emb, layers, w, tok, mode=q4.FAST)
    t = torch.tensor([tok], dtype=torch.int32, device="cuda")
    h = q4.q4_embed(emb, t)
    m = torch.empty(w["inter"], device="cuda")
    for L in layers:
        q4.q4mv_norm_swiglu(L.gate_up, h, L.wn, w["eps"], m, mode=q4.FAST)
        q4.q4mv_add(L.down, m, None, h, h, mode=q4.FAST)
    torch.cuda.synchronize()
    assert_bits_equal(got, host(h), "fast decode_layers vs fast stage kernels")
    want = oracle.chain_hidden(w, tok, NTHREADS)
    err = np.abs(got.astype(np.float64) - want)
    assert err.max() <= 1e-4 * np.sqrt(np.mean(want.astype(np.float64) ** 2)), err.max()


def test_decode_layers_full_depth_matches_oracle():
    """24 layers of 2048 x 6144 (the decode chain's layer stack)."""
    q4 = lib()
    w = synth.chain_weights(vocab=4096)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    want = oracle.chain_hidden(w, w["tok0"], NTHREADS)
    got, ws = run_layers(q4, emb, layers, w, w["tok0"])
    assert_bits_equal(got, want, "h after 24 layers")
    # repeated calls reuse the workspace (the barrier words return to rest)
    for _ in range(3):
        again, ws = run_layers(q4, emb, layers, w, w["tok0"], ws=ws)
        assert_bits_equal(again, want, "h after 24 layers, again")


def test_decode_layers_relay_fallback_gives_the_same_bits():
    """Q4_DECODE_NEAR_US=0: a wait for h reads its XCD's copy for one round
    only, then the producers' device-scope copy (the path of a workgroup
    that no relay serves); the result must not change."""
    q4 = lib()
    w = synth.chain_weights(seed=46, layers=4, vocab=3000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    want = oracle.chain_hidden(w, w["tok0"], NTHREADS)
    os.environ["Q4_DECODE_NEAR_US"] = "0"
    try:
        ws = None
        for i in range(3):
            got, ws = run_layers(q4, emb, layers, w, w["tok0"], ws=ws)
            assert_bits_equal(got, want, "h after 4 layers, relay fallback, call %d" % i)
    finally:
        del os.environ["Q4_DECODE_NEAR_US"]
    got, ws = run_layers(q4, emb, layers, w, w["tok0"], ws=ws)
    assert_bits_equal(got, want, "h after 4 layers, relay")


def test_two_persistent_launches_at_once_end_and_stay_exact():
    """The persistent kernel needs every compute unit (one workgroup each);
    two launches on two streams at once may each get only part of the
    device.  Each must then either finish with the oracle's bits or give up
    through its bounded waits (Q4_ETIMEOUT, here after 200 ms) and leave a
    workspace that the status call makes usable again: never a hang, never
    other bits."""
    q4 = lib()
    w = synth.chain_weights(seed=48, layers=2, vocab=3000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    want = oracle.chain_hidden(w, w["tok0"], NTHREADS)
    t = torch.tensor([w["tok0"]], dtype=torch.int32, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    hs = [torch.full((2048,), 7.0, device="cuda") for _ in streams]
    wss = [new_ws(q4) for _ in streams]
    seen = set()
    os.environ["Q4_DECODE_TIMEOUT_MS"] = "200"
    try:
        for rep in range(6):
            torch.cuda.synchronize()
            for s, h, ws in zip(streams, hs, wss):
                q4.q4_decode_layers(emb, t, layers, w["eps"], h, ws, stream=s)
            for i, (s, h, ws) in enumerate(zip(streams, hs, wss)):
                st = q4.q4_decode_layers_status(ws, stream=s)
                print("concurrent launches, round %d, stream %d: status %d" % (rep, i, st),
                      flush=True)
                assert st in (q4.Q4_OK, q4.Q4_ETIMEOUT)
                seen.add(st)
                if st == q4.Q4_OK:
                    assert_bits_equal(host(h), want, "h, concurrent launch %d/%d" % (rep, i))
    finally:
        del os.environ["Q4_DECODE_TIMEOUT_MS"]
    print("statuses seen:", sorted(seen), flush=True)
    for h, ws in zip(hs, wss):
        got, _ = run_layers(q4, emb, layers, w, w["tok0"], ws=ws)
        assert_bits_equal(got, want, "h after the concurrent launches")


def test_decode_layers_in_graph_replays():
    q4 = lib()
    w = synth.chain_weights(seed=47, layers=3, vocab=3000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    s = torch.cuda.Stream()
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    h = torch.empty(2048, device="cuda")
    ws = new_ws(q4)
    torch.cuda.synchronize()
    g = q4.Graph(s)
    g.begin()
    try:
        q4.q4_decode_layers(emb, t, layers, w["eps"], h, ws, stream=s)
    finally:
        g.end()
    other = synth.small_product(seed=48, rows=200, cols=2048, name="between")
    W = q4.Q4Matrix.from_host(other)
    for tok in (5, 2999, 1234):
        t.fill_(tok)
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        assert_bits_equal(host(h), oracle.chain_hidden(w, tok, NTHREADS), "graph tok %d" % tok)
        q4.q4mv(W, dev(other["x"]), None)  # eager work between replays
        torch.cuda.synchronize()
    assert q4.q4_decode_layers_status(ws) == q4.Q4_OK
    g.close()


def test_decode_layers_error_word_stops_the_kernel_and_is_cleared():
    """A workspace whose error word is set: every workgroup returns at once,
    the status call reports it and clears the workspace, the next call is
    correct."""
    q4 = lib()
    w = synth.chain_weights(seed=49, layers=2, vocab=1000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    t = torch.tensor([3], dtype=torch.int32, device="cuda")
    h = torch.full((2048,), 7.0, device="cuda")
    ws = new_ws(q4)
    # the error word: 32 words before the end of the workspace
    ws.view(torch.int32)[q4.q4_decode_layers_ws_bytes() // 4 - 32] = 1
    q4.q4_decode_layers(emb, t, layers, w["eps"], h, ws)
    assert q4.q4_decode_layers_status(ws) == q4.Q4_ETIMEOUT
    assert np.all(host(h) == 7.0)  # nothing ran
    assert int(np.abs(host(ws)).max()) == 0  # cleared
    got, _ = run_layers(q4, emb, layers, w, 3, ws=ws)
    assert_bits_equal(got, oracle.chain_hidden(w, 3, NTHREADS), "after a cleared error")


def test_decode_layers_wait_timeout_is_reported_and_cleared():
    """No waiting allowed (bound set from the host): the first thread that
    does not find its data at the first look sets the error word, every
    workgroup leaves at its next wait, and the status call reports it.  (A
    run can only escape this if every workgroup found every value it needs
    already written; the 12 layers make that out of reach.)"""
    q4 = lib()
    w = synth.chain_weights(seed=50, layers=12, vocab=1000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    t = torch.tensor([3], dtype=torch.int32, device="cuda")
    h = torch.empty(2048, device="cuda")
    ws = new_ws(q4)
    os.environ["Q4_DECODE_TIMEOUT_MS"] = "-1"
    try:
        q4.q4_decode_layers(emb, t, layers, w["eps"], h, ws)
    finally:
        del os.environ["Q4_DECODE_TIMEOUT_MS"]
    assert q4.q4_decode_layers_status(ws) == q4.Q4_ETIMEOUT
    assert int(np.abs(host(ws)).max()) == 0
    got, _ = run_layers(q4, emb, layers[:2], {**w, "layers": w["layers"][:2]}, 3, ws=ws)
    assert_bits_equal(got, oracle.chain_hidden(w, 3, NTHREADS, layers=2), "after a timeout")


@pytest.mark.parametrize("inter,nlayers,vocab", [(2048, 1, 3001), (6144, 2, 20003), (8192, 1, 7),
                                                 (4096, 3, 9000)])
def test_decode_token_matches_separate_calls_and_oracle(inter, nlayers, vocab):
    """q4_decode_token (the layers, the final norm, the head and its argmax
    in one launch) against q4_decode_layers + q4mv_norm_argmax and the
    oracle: h, every logit and the token bit for bit, over several steps
    on one workspace (the token fed back in place); vocab sizes with a
    ragged last block, fewer blocks than waves, and several per wave."""
    q4 = lib()
    w = synth.chain_weights(seed=60 + nlayers, layers=nlayers, inter=inter, vocab=vocab)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    wf = dev(w["wn_final"])
    tok = torch.tensor([int(w["tok0"])], dtype=torch.int32, device="cuda")
    h = torch.full((2048,), 7.0, device="cuda")
    logits = torch.full((vocab,), 7.0, device="cuda")
    ws = new_ws(q4)
    t_host = int(w["tok0"])
    for step in range(3):
        print("decode_token inter=%d layers=%d vocab=%d step %d" % (inter, nlayers, vocab, step),
              flush=True)
        want_logits, want_tok = oracle.chain_step(w, t_host, NTHREADS)
        q4.q4_decode_token(emb, tok, layers, wf, w["eps"], h, logits, ws)
        assert q4.q4_decode_layers_status(ws) == q4.Q4_OK
        assert_bits_equal(host(h), oracle.chain_hidden(w, t_host, NTHREADS), "h step %d" % step)
        assert_bits_equal(host(logits), want_logits, "logits step %d" % step)
        assert int(host(tok)[0]) == want_tok, step
        # the separate calls give the same
        t2 = torch.tensor([t_host], dtype=torch.int32, device="cuda")
        h2 = torch.empty(2048, device="cuda")
        y2 = torch.empty(vocab, device="cuda")
        q4.q4_decode_layers(emb, t2, layers, w["eps"], h2, new_ws(q4))
        q4.q4mv_norm_argmax(emb, h2, wf, w["eps"], y2, t2)
        torch.cuda.synchronize()
        assert_bits_equal(host(y2), host(logits), "separate calls step %d" % step)
        assert int(host(t2)[0]) == want_tok
        t_host = want_tok


def test_decode_token_nan_logits_give_minus_one():
    q4 = lib()
    w = synth.chain_weights(seed=64, layers=1, inter=2048, vocab=500)
    emb = q4.Q4Matrix.from_host(w["head"])
    tok = torch.tensor([500], dtype=torch.int32, device="cuda")  # outside: h is NaN
    h = torch.empty(2048, device="cuda")
    logits = torch.empty(500, device="cuda")
    ws = new_ws(q4)
    q4.q4_decode_token(emb, tok, mlp_layers(q4, w), dev(w["wn_final"]), w["eps"], h, logits, ws)
    assert q4.q4_decode_layers_status(ws) == q4.Q4_OK
    assert np.all(np.isnan(host(logits)))
    assert int(host(tok)[0]) == -1


def test_decode_token_wait_timeout_is_reported_and_cleared():
    """No waiting allowed: the launch leaves early, the status reports it
    and clears the workspace, and the token is left as it was."""
    q4 = lib()
    w = synth.chain_weights(seed=65, layers=6, vocab=1000)
    emb = q4.Q4Matrix.from_host(w["head"])
    layers = mlp_layers(q4, w)
    tok = torch.tensor([3], dtype=torch.int32, device="cuda")
    h = torch.empty(2048, device="cuda")
    logits = torch.empty(1000, device="cuda")
    ws = new_ws(q4)
    os.environ["Q4_DECODE_TIMEOUT_MS"] = "-1"
    try:
        q4.q4_decode_token(emb, tok, layers, dev(w["wn_final"]), w["eps"], h, logits, ws)
    finally:
        del os.environ["Q4_DECODE_TIMEOUT_MS"]
    assert q4.q4_decode_layers_status(ws) == q4.Q4_ETIMEOUT
    assert int(host(tok)[0]) == 3
    assert int(np.abs(host(ws)).max()) == 0
    q4.q4_decode_token(emb, tok, layers[:1], dev(w["wn_final"]), w["eps"], h, logits, ws)
    assert q4.q4_decode_layers_status(ws) == q4.Q4_OK
    _, want = oracle.chain_step({**w, "layers": w["layers"][:1]}, 3, NTHREADS)
    assert int(host(tok)[0]) == want


def test_decode_token_planted_maxima_every_wave_position():
    """The largest logit placed in rows of the first wave of a workgroup
    (block 5: rows 20..23) and of the last wave (block 2047: rows 8188..8191),
    then in two identical rows (a tie: the lower index wins)."""
    q4 = lib()
    w = synth.chain_weights(seed=66, layers=1, inter=2048, vocab=9000)
    tok = 3
    h = oracle.chain_hidden(w, tok, NTHREADS)
    _, us = oracle.rmsq(h, w["wn_final"], w["eps"])
    lift = np.where(us >= 0, np.float32(64.0), np.float32(-64.0))
    layers = mlp_layers(q4, w)
    wf = dev(w["wn_final"])
    for rows, want in (([21], 21), ([8189], 8189), ([8190, 22], 22)):
        head = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in w["head"].items()}
        for r in rows:
            head["q"][r] = head["q"][rows[0]]
            head["s"][r] = head["s"][rows[0]]
            head["b"][r] = lift
        wm = {**w, "head": head}
        want_logits, want_tok = oracle.chain_step(wm, tok, NTHREADS)
        assert want_tok == want
        emb = q4.Q4Matrix.from_host(head)
        t = torch.tensor([tok], dtype=torch.int32, device="cuda")
        hd = torch.empty(2048, device="cuda")
        logits = torch.empty(9000, device="cuda")
        ws = new_ws(q4)
        q4.q4_decode_token(emb, t, layers, wf, w["eps"], hd, logits, ws)
        assert q4.q4_decode_layers_status(ws) == q4.Q4_OK
        assert_bits_equal(host(logits), want_logits, "planted %s" % rows)
        assert int(host(t)[0]) == want, rows
