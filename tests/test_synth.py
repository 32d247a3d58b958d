"""The seeded input generators: reproducible bytes, independent streams and
the value distributions of the workloads."""
import numpy as np

import synth


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of the published generator
    # (state += 0x9E3779B97F4A7C15, then the finaliser) are fixed numbers.
    key = 0
    outs = []
    state = key
    for _ in range(3):
        state = (state + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
        outs.append(synth._mix64_int(state))
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_same_seed_same_bytes_and_independent_streams():
    a = synth.small_product(seed=1, rows=13, cols=128)
    b = synth.small_product(seed=1, rows=13, cols=128)
    assert synth.sha256(a["q"], a["s"], a["b"], a["x"]) == synth.sha256(b["q"], b["s"], b["b"], b["x"])
    c = synth.small_product(seed=2, rows=13, cols=128)
    assert not np.array_equal(a["q"], c["q"])
    d = synth.draws(1, "one", 1000)
    e = synth.draws(1, "two", 1000)
    assert not np.any(d == e)
    # chunked generation equals one-shot generation
    assert np.array_equal(synth.draws(5, "x", 10, start=7), synth.draws(5, "x", 17)[7:])


def test_distributions():
    m = synth.q4_matrix(3, "dist", 2048, 2048)
    q = m["q"]
    counts = np.bincount(((q[..., None] >> np.arange(0, 32, 4, dtype=np.uint32)) & 15).ravel(), minlength=16)
    assert counts.min() > 0.98 * counts.mean() and counts.max() < 1.02 * counts.mean()
    assert m["s"].min() >= 0.001 and m["s"].max() < 0.02
    resid = m["b"].astype(np.float64) + 8 * m["s"].astype(np.float64)
    assert abs(resid.mean()) < 1e-5 and abs(resid.std() - 1e-3) < 2e-5
    x = synth.normal_f32(3, "n", (200000,), 0.0, 1.0)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01 and np.abs(x).max() <= 6.0
    w = synth.normal_f32(3, "w", (200000,), 1.0, 0.1)
    assert abs(w.mean() - 1.0) < 0.001 and abs(w.std() - 0.1) < 0.001


def test_workload_shapes():
    w = synth.chain_weights(seed=1, layers=1, hidden=128, inter=192, vocab=300)
    assert w["layers"][0]["gate"]["q"].shape == (192, 16)
    assert w["layers"][0]["down"]["s"].shape == (128, 3)
    assert w["head"]["q"].shape == (300, 16) and 0 <= w["tok0"] < 300
    h = synth.head_inputs(seed=1, rows=10, cols=2048)
    assert h["q"].shape == (10, 256) and h["z"].shape == (2048,)


def test_rope_tables_rows_are_the_position_tables():
    ct, st = synth.rope_tables(300)
    assert ct.shape == (300, 64) and st.shape == (300, 64)
    for p in (0, 1, 204, 299):
        c, s = synth.rope_table(p)
        assert np.array_equal(ct[p], c) and np.array_equal(st[p], s)
    assert np.array_equal(ct[0], np.ones(64, np.float32))
    assert np.array_equal(st[0], np.zeros(64, np.float32))
