"""Pins of the CPU oracle against facts that do not come from the oracle.

Each check is chosen so that a plausible mistake in the oracle (a dropped
term, a swapped operand, a wrong split of the summation tree, a fused
multiply-add, the wrong nibble order, eps in the wrong place) fails it:

* brute force: dequantise, then a binary64 dot, within an a-priori rounding
  bound (Higham-style ``gamma_D``);
* closed forms that IEEE-754 arithmetic fixes exactly (identity matrices,
  one-hot activations, power-of-two codes, saturation of the sigmoid);
* adversarial sums whose rounded value reveals the shape of the tree,
  checked against an independent characterisation of that shape;
* invariants (row slicing and permutation, thread count, determinism).
"""
import math

import numpy as np
import pytest

import oracle
import synth

U32 = 2.0**-24  # unit roundoff of binary32


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Test-local packer: column 8j+k goes to bits 4k..4k+3 of word j."""
    codes = np.asarray(codes, dtype=np.uint32)
    rows, cols = codes.shape
    words = np.zeros((rows, cols // 8), dtype=np.uint32)
    for k in range(8):
        words |= codes[:, k::8] << np.uint32(4 * k)
    return words


def unpack_codes(words: np.ndarray, cols: int) -> np.ndarray:
    rows = words.shape[0]
    out = np.zeros((rows, cols), dtype=np.int64)
    for k in range(8):
        out[:, k::8] = (words >> np.uint32(4 * k)) & np.uint32(15)
    return out


def mat_from(codes, s, b):
    rows, cols = codes.shape
    return {"q": pack_codes(codes), "s": np.asarray(s, np.float32),
            "b": np.asarray(b, np.float32), "rows": rows, "cols": cols}


def gamma(k):
    return k * U32 / (1 - k * U32)


# ---------------------------------------------------------------------------
# The canonical tree T
# ---------------------------------------------------------------------------

def meets_before_zero(i, j, n):
    """Independent characterisation of T's shape: do leaves i and j
    (0 < i < j < n) join each other before either joins leaf 0?"""
    lo, size = 0, n
    while True:
        if size & (size - 1) == 0:  # power of two: balanced block [lo, lo+size)
            a, b = i - lo, j - lo
            # they meet at level bitlen(a^b); 0 (the block's first leaf) meets
            # a at level bitlen(a)
            return (a ^ b).bit_length() < a.bit_length()
        m = 1 << ((size - 1).bit_length() - 1)  # largest power of two < size
        if i - lo >= m:
            return True  # both in the right part, which does not hold leaf 0
        if j - lo >= m:
            return False  # i is on leaf 0's side, j is not
        size = m  # both in the left, balanced part


@pytest.mark.parametrize("n", list(range(2, 40)) + [63, 64, 65, 96, 127, 128, 129, 192, 200])
def test_tree_shape_against_characterisation(n):
    big = np.float32(2.0**24)
    pairs = [(i, j) for i in range(1, n) for j in range(i + 1, n)]
    if len(pairs) > 400:
        rng = np.random.default_rng(n)
        pairs = [pairs[k] for k in rng.choice(len(pairs), 400, replace=False)]
    for i, j in pairs:
        v = np.zeros(n, np.float32)
        v[0] = big
        v[i] = 1.0
        v[j] = 1.0
        got = float(oracle.tree(v))
        # 2^24 + 1 rounds back to 2^24 (tie to even); 2^24 + 2 is exact
        want = 2.0**24 + 2.0 if meets_before_zero(i, j, n) else 2.0**24
        assert got == want, (n, i, j, got)


def test_tree_small_closed_forms():
    big = 2.0**24
    assert float(oracle.tree([big, 1, 1])) == big          # (a+b)+c
    assert float(oracle.tree([1, 1, big])) == big + 2      # (a+b)+c
    assert float(oracle.tree([big, 1, 1, 0])) == big        # (a+b)+(c+d)
    assert float(oracle.tree([big, 0, 1, 1])) == big + 2
    assert float(oracle.tree([7.5])) == 7.5
    # T(5) = T(4) + v4
    assert float(oracle.tree([big, 0, 0, 1, 1])) == big


@pytest.mark.parametrize("n", [1, 2, 3, 5, 31, 64, 96, 100, 2048, 6144])
def test_tree_exact_on_integers(n):
    rng = np.random.default_rng(100 + n)
    v = rng.integers(-1000, 1000, n).astype(np.float32)
    assert float(oracle.tree(v)) == float(v.astype(np.int64).sum())


def test_tree_negative_zero_and_signs():
    assert math.copysign(1.0, float(oracle.tree([-0.0, -0.0]))) == -1.0
    assert math.copysign(1.0, float(oracle.tree([-0.0, 0.0]))) == 1.0
    assert float(oracle.tree([1.5, -1.5, 2.0])) == 2.0


def test_group_sums_are_trees_of_64():
    x = np.zeros(192, np.float32)
    x[64] = 2.0**24
    x[65] = 1.0
    x[66] = 1.0  # leaves 1 and 2 of group 1: (v0+v1)+(v2+v3) -> 2^24 + 1 lost
    x[130] = 1.0
    x[131] = 1.0  # leaves 2 and 3 of group 2: meet first -> exact 2
    xs = oracle.group_sums(x)
    assert list(map(float, xs)) == [0.0, 2.0**24, 2.0]


# ---------------------------------------------------------------------------
# q4mv
# ---------------------------------------------------------------------------

def brute_force_bound(m, x, xs):
    codes = unpack_codes(m["q"], m["cols"]).astype(np.float64)
    G = m["cols"] // 64
    s = m["s"].astype(np.float64)
    b = m["b"].astype(np.float64)
    x64 = x.astype(np.float64)
    xs64 = xs.astype(np.float64)
    exact = np.empty(m["rows"])
    mag = np.empty(m["rows"])
    D = 9 + math.ceil(math.log2(G)) if G > 1 else 9
    for r in range(m["rows"]):
        terms, absum = [], 0.0
        for g in range(G):
            qx = codes[r, 64 * g:64 * g + 64] * x64[64 * g:64 * g + 64]
            terms.extend(list(s[r, g] * qx))
            terms.append(b[r, g] * xs64[g])
            absum += abs(s[r, g]) * np.abs(qx).sum() + abs(b[r, g] * xs64[g])
        exact[r] = math.fsum(terms)
        mag[r] = absum
    return exact, gamma(D) * mag


@pytest.mark.parametrize("rows,cols", [(13, 128), (4, 64), (3, 192), (5, 2048), (2, 6144)])
def test_q4mv_brute_force_dequantise_then_dot(rows, cols):
    m = synth.small_product(seed=7, rows=rows, cols=cols, name="p1_%d_%d" % (rows, cols))
    xs = oracle.group_sums(m["x"])
    y = oracle.q4mv(m, m["x"], xs)
    exact, bound = brute_force_bound(m, m["x"], xs)
    assert np.all(np.abs(y.astype(np.float64) - exact) <= bound), np.max(np.abs(y - exact) / bound)
    # the bound is tight enough to see a one-nibble slip
    assert np.all(bound < 1e-3 * (np.abs(exact) + 1.0))


def test_q4mv_identity_codes_zero_bias_one():
    rows, cols = 6, 384
    rng = np.random.default_rng(1)
    codes = np.zeros((rows, cols), np.int64)
    s = rng.uniform(0.001, 0.02, (rows, cols // 64)).astype(np.float32)
    b = np.ones((rows, cols // 64), np.float32)
    m = mat_from(codes, s, b)
    # integer-valued activations: every sum is exact, so y = sum(x)
    x = rng.integers(-50, 50, cols).astype(np.float32)
    xs = oracle.group_sums(x)
    y = oracle.q4mv(m, x, xs)
    assert np.all(y == np.float32(x.astype(np.int64).sum()))
    # random activations: y is the tree of the group sums, close to sum(x)
    x = synth.normal_f32(3, "p2x", (cols,), 0.0, 1.0)
    xs = oracle.group_sums(x)
    y = oracle.q4mv(m, x, xs)
    assert np.all(y == y[0])
    assert abs(float(y[0]) - math.fsum(x.astype(np.float64))) <= gamma(9 + 3) * np.abs(x).sum()


@pytest.mark.parametrize("rows,cols", [(3, 64), (4, 128), (2, 192)])
def test_q4mv_one_hot_recovers_dequantised_columns(rows, cols):
    m = synth.q4_matrix(11, "p3_%d" % cols, rows, cols)
    codes = unpack_codes(m["q"], cols)
    G = cols // 64
    for j in range(cols):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        xs = np.zeros(G, np.float32)
        xs[j // 64] = 1.0
        y = oracle.q4mv(m, x, xs)
        g = j // 64
        for r in range(rows):
            want = np.float32(m["s"][r, g]) * np.float32(codes[r, j])
            want = np.float32(want + np.float32(m["b"][r, g]))
            assert y[r] == want, (j, r)


@pytest.mark.parametrize("c", [1, 2, 4, 8])
def test_q4mv_power_of_two_codes(c):
    rows, cols = 3, 6144
    codes = np.full((rows, cols), c, np.int64)
    m = mat_from(codes, np.ones((rows, 96)), np.zeros((rows, 96)))
    rng = np.random.default_rng(c)
    x = (rng.integers(-64, 64, cols) / 8.0).astype(np.float32)  # dyadic: sums exact
    xs = oracle.group_sums(x)
    y = oracle.q4mv(m, x, xs)
    want = c * (x.astype(np.float64) * 8).astype(np.int64).sum() / 8.0
    assert np.all(y.astype(np.float64) == want)


def test_q4mv_group_level_tree_order_on_96_groups():
    # d_0 = 2^24, d_32 = 1, d_64 = 1: T over 96 groups is (P0+P1)+P2 -> 2^24;
    # a right-nested P0+(P1+P2) would give 2^24+2.
    cols = 6144
    codes = np.ones((1, cols), np.int64)
    m = mat_from(codes, np.ones((1, 96)), np.zeros((1, 96)))
    x = np.zeros(cols, np.float32)
    x[0] = 2.0**24
    x[2048] = 1.0
    x[4096] = 1.0
    y = oracle.q4mv(m, x, oracle.group_sums(x))
    assert float(y[0]) == 2.0**24
    x[4096] = 0.0
    x[4096 + 64] = 1.0  # group 65: still in P2
    assert float(oracle.q4mv(m, x, oracle.group_sums(x))[0]) == 2.0**24
    # groups 1 and 2 in the first 32-block: (t0+t1)+(t2+t3) -> t1 is lost
    x[:] = 0
    x[0] = 2.0**24
    x[64] = 1.0
    x[128] = 1.0
    assert float(oracle.q4mv(m, x, oracle.group_sums(x))[0]) == 2.0**24
    x[64] = 0.0
    x[192] = 1.0  # groups 2 and 3 meet first -> exact
    assert float(oracle.q4mv(m, x, oracle.group_sums(x))[0]) == 2.0**24 + 2


def test_q4mv_code_level_tree_is_balanced_per_group():
    cols = 64
    codes = np.ones((1, cols), np.int64)
    m = mat_from(codes, np.ones((1, 1)), np.zeros((1, 1)))
    x = np.zeros(cols, np.float32)
    x[0] = 2.0**24
    x[2] = 1.0
    x[3] = 1.0  # (p0+p1)+(p2+p3): 1+1 first -> exact
    assert float(oracle.q4mv(m, x, np.zeros(1, np.float32))[0]) == 2.0**24 + 2
    x[3] = 0.0
    x[33] = 1.0  # p2 joins p0's side before p33
    assert float(oracle.q4mv(m, x, np.zeros(1, np.float32))[0]) == 2.0**24


def test_q4mv_affine_step_is_unfused():
    # G = 1, codes 1, x = e_0 * d: d_0 = d.  Then y = RN(RN(s d) + RN(b xs)),
    # which differs from the fused RN(s d + RN(b xs)) for these values.
    s = np.float32(1 + 2.0**-23)
    d = np.float32(1 + 2.0**-22)
    b = np.float32(-1.0)
    xs = np.float32(1.0)
    codes = np.ones((1, 64), np.int64)
    m = mat_from(codes, [[s]], [[b]])
    x = np.zeros(64, np.float32)
    x[0] = d
    y = float(oracle.q4mv(m, x, np.array([xs], np.float32))[0])
    unfused = float(np.float32(np.float32(s * d) + np.float32(b * xs)))
    fused = float(np.float32(float(s) * float(d) + float(b * xs)))  # exact s*d fits in binary64
    assert unfused != fused
    assert y == unfused


def test_q4mv_rows_slice_and_permute():
    m = synth.small_product(seed=5, rows=13, cols=256, name="p5")
    xs = oracle.group_sums(m["x"])
    y = oracle.q4mv(m, m["x"], xs)
    perm = np.random.default_rng(0).permutation(13)
    mp = dict(m, q=m["q"][perm].copy(), s=m["s"][perm].copy(), b=m["b"][perm].copy())
    assert np.array_equal(oracle.q4mv(mp, m["x"], xs).view(np.uint32), y[perm].view(np.uint32))
    for lo, hi in [(0, 8), (8, 12), (12, 13)]:
        ms = dict(m, q=m["q"][lo:hi].copy(), s=m["s"][lo:hi].copy(), b=m["b"][lo:hi].copy(), rows=hi - lo)
        assert np.array_equal(oracle.q4mv(ms, m["x"], xs).view(np.uint32), y[lo:hi].view(np.uint32))
    ys = oracle.q4mv_sample(m, m["x"], xs, [12, 0, 5, 5])
    assert np.array_equal(ys.view(np.uint32), y[[12, 0, 5, 5]].view(np.uint32))


def test_q4mv_threads_and_repeats_do_not_change_bits():
    m = synth.small_product(seed=6, rows=257, cols=2048, name="p6")
    xs = oracle.group_sums(m["x"])
    y1 = oracle.q4mv(m, m["x"], xs, nthreads=1)
    for t in (2, 3, 8):
        assert np.array_equal(oracle.q4mv(m, m["x"], xs, nthreads=t).view(np.uint32), y1.view(np.uint32))
    for _ in range(3):
        assert np.array_equal(oracle.q4mv(m, m["x"], xs).view(np.uint32), y1.view(np.uint32))


def test_code_extraction_low_nibble_first():
    q = np.array([[0x76543210, 0xFEDCBA98]], np.uint32)
    assert [oracle.code(q, 16, 0, c) for c in range(16)] == list(range(16))


# ---------------------------------------------------------------------------
# rmsq
# ---------------------------------------------------------------------------

def test_rmsq_zero_input():
    n = 2048
    w = synth.normal_f32(1, "wn", (n,), 1.0, 0.1)
    u, us = oracle.rmsq(np.zeros(n, np.float32), w, 1e-6)
    assert np.all(u == 0) and np.all(us == 0)


@pytest.mark.parametrize("c", [2.0, 0.75, -3.0])
def test_rmsq_constant_input_closed_form(c):
    n = 2048
    w = synth.normal_f32(2, "wn", (n,), 1.0, 0.1)
    eps = np.float32(1e-6)
    u, us = oracle.rmsq(np.full(n, c, np.float32), w, eps)
    cc = np.float32(c)
    ss = np.float32(cc * cc) * np.float32(n)  # exact: n copies of c^2, power-of-two count
    ms = np.float32(ss / np.float32(n))
    rho = np.float32(np.float32(1.0) / np.sqrt(np.float32(ms + eps)))
    want = (np.float32(cc * rho) * w).astype(np.float32)
    assert np.array_equal(u.view(np.uint32), want.view(np.uint32))


def test_rmsq_against_binary64_within_bound():
    n = 2048
    h = synth.normal_f32(3, "h", (n,), 0.0, 1.0)
    w = synth.normal_f32(3, "wn", (n,), 1.0, 0.1)
    u, us = oracle.rmsq(h, w, 1e-6)
    h64, w64 = h.astype(np.float64), w.astype(np.float64)
    ref = h64 * w64 / math.sqrt(math.fsum(h64 * h64) / n + float(np.float32(1e-6)))
    k = math.ceil(math.log2(n)) + 1
    bound = gamma((k + 2) / 2 + 4) * np.abs(ref)
    assert np.all(np.abs(u - ref) <= bound)
    # group sums: trees of 64 over u
    ref_us = u.astype(np.float64).reshape(-1, 64).sum(axis=1)
    assert np.all(np.abs(us - ref_us) <= gamma(6) * np.abs(u).reshape(-1, 64).sum(axis=1))


def test_rmsq_eps_inside_the_root():
    n = 128
    h = np.full(n, 1e-4, np.float32)  # mean(h^2) = 1e-8 << eps
    u, _ = oracle.rmsq(h, np.ones(n, np.float32), 1e-6)
    want = 1e-4 / math.sqrt(1e-8 + float(np.float32(1e-6)))
    assert abs(float(u[0]) - want) <= 4 * U32 * want
    assert abs(float(u[0]) - 1e-4 / (1e-4 + 1e-6)) > 1e-3  # eps outside the root


def test_rmsq_unit_mean_square():
    n = 2048
    h = synth.normal_f32(4, "h", (n,), 0.0, 1.0)
    u, _ = oracle.rmsq(h, np.ones(n, np.float32), 1e-6)
    assert abs(float(np.mean(u.astype(np.float64) ** 2)) - 1.0) < 1e-5


def test_rmsq_rejects_ragged_length():
    with pytest.raises(ValueError):
        oracle.rmsq(np.ones(100, np.float32), np.ones(100, np.float32), 1e-6)


# ---------------------------------------------------------------------------
# exp and swq
# ---------------------------------------------------------------------------

def ulp64(v):
    return math.ulp(v)


def test_exp_close_to_libm():
    ts = np.concatenate([np.linspace(-745.0, 709.7, 20001), np.linspace(-1, 1, 2001),
                         synth.normal_f64(9, "t", 5000) * 30])
    worst = 0.0
    for t in ts:
        e, ref = oracle.exp(float(t)), math.exp(float(t))
        if ref == 0.0 or ref < 2.3e-308:
            assert abs(e - ref) <= 2 * 5e-324 + 1e-300 * 0
            continue
        worst = max(worst, abs(e - ref) / ulp64(ref))
    assert worst <= 2.0, worst


def test_exp_special_values():
    assert oracle.exp(0.0) == 1.0
    assert oracle.exp(710.0) == math.inf and oracle.exp(1e30) == math.inf
    assert oracle.exp(-746.0) == 0.0 and oracle.exp(-1e30) == 0.0
    assert math.isnan(oracle.exp(math.nan))
    assert abs(oracle.exp(1.0) - math.e) <= ulp64(math.e)
    for k in (-1000, -3, 1, 17, 1000):
        assert abs(oracle.exp(k * math.log(2)) / 2.0**k - 1) < 4e-16 * max(1, abs(k)) * 700


def test_swq_closed_forms():
    n = 64
    a = np.zeros(2 * n, np.float32)
    rng = np.random.default_rng(2)
    a[n:] = rng.normal(size=n).astype(np.float32)
    o, os_ = oracle.swq(a, n)
    assert np.all(o == 0)  # silu(0) = 0
    # gate >= 40: 1 + exp(-a) == 1 in binary64, so o = RN32(a * up) exactly
    a[:n] = rng.uniform(40, 1000, n).astype(np.float32)
    o, _ = oracle.swq(a, n)
    want = (a[:n].astype(np.float64) * a[n:].astype(np.float64)).astype(np.float32)
    assert np.array_equal(o.view(np.uint32), want.view(np.uint32))
    # gate <= -746: exp overflows, silu -> -0, o -> +-0
    a[:n] = -rng.uniform(746, 1e4, n).astype(np.float32)
    o, _ = oracle.swq(a, n)
    assert np.all(o == 0)
    # up == 0 -> o == +-0
    a[:n] = rng.normal(size=n).astype(np.float32)
    a[n:] = 0
    o, _ = oracle.swq(a, n)
    assert np.all(o == 0)


def test_swq_against_libm_reference():
    n = 6144
    a = synth.normal_f32(5, "a", (2 * n,), 0.0, 3.0)
    o, os_ = oracle.swq(a, n)
    g, up = a[:n].astype(np.float64), a[n:].astype(np.float64)
    ref = np.array([gi / (1.0 + math.exp(-gi)) for gi in g]) * up
    ref32 = ref.astype(np.float32)
    diff = np.abs(o.astype(np.float64) - ref32.astype(np.float64))
    ulp = np.array([math.ulp(float(v)) for v in np.abs(ref32).astype(np.float32)])
    ulp32 = np.spacing(np.abs(ref32)).astype(np.float64)
    assert np.all(diff <= ulp32)
    assert np.mean(o == ref32) > 0.999
    del ulp
    ref_os = o.astype(np.float64).reshape(-1, 64).sum(axis=1)
    assert np.all(np.abs(os_ - ref_os) <= gamma(6) * np.abs(o).reshape(-1, 64).sum(axis=1))


def test_swq_rejects_n32():
    with pytest.raises(ValueError):
        oracle.swq(np.ones(64, np.float32), 32)


# ---------------------------------------------------------------------------
# argmax and embed
# ---------------------------------------------------------------------------

def test_argmax_planted():
    v = synth.normal_f32(8, "v", (248320,), 0.0, 1.0)
    v[123456] = 50.0
    assert oracle.argmax(v) == 123456
    v[7] = 50.0
    assert oracle.argmax(v) == 7  # tie: lowest index
    v[200000] = math.nan
    assert oracle.argmax(v) == -1
    assert oracle.argmax(np.full(5, -np.inf, np.float32)) == 0
    assert oracle.argmax(np.array([3.0], np.float32)) == 0


def test_embed_is_dequantised_row():
    m = synth.q4_matrix(12, "emb", 50, 2048)
    codes = unpack_codes(m["q"], 2048)
    for t in (0, 17, 49):
        e = oracle.embed(m, t)
        g = np.arange(2048) // 64
        want = (m["s"][t, g] * codes[t].astype(np.float32)).astype(np.float32) + m["b"][t, g]
        assert np.array_equal(e.view(np.uint32), want.astype(np.float32).view(np.uint32))
        # and equals the one-hot product of that column set (P3 route)
        sq = m["s"][t, g].astype(np.float64) * codes[t]
        ref = sq + m["b"][t, g].astype(np.float64)
        # two roundings; b ~ -8 s cancels, so bound by the operands' size
        assert np.all(np.abs(e - ref) <= gamma(2) * (np.abs(sq) + np.abs(m["b"][t, g])))
    assert np.all(np.isnan(oracle.embed(m, 50))) and np.all(np.isnan(oracle.embed(m, -1)))


# ---------------------------------------------------------------------------
# the decode chain, composed from the pieces above
# ---------------------------------------------------------------------------

def test_chain_step_against_binary64_forward():
    w = synth.chain_weights(seed=21, layers=2, hidden=128, inter=192, vocab=1000)
    tok = w["tok0"]
    for _ in range(3):
        logits, nxt = oracle.chain_step(w, tok)
        # independent binary64 forward of the same chain
        def deq(m):
            c = unpack_codes(m["q"], m["cols"]).astype(np.float64)
            g = np.arange(m["cols"]) // 64
            return c * m["s"][:, g].astype(np.float64) + m["b"][:, g].astype(np.float64)
        h = deq(w["head"])[tok]
        for lw in w["layers"]:
            u = h / math.sqrt(np.mean(h * h) + 1e-6) * lw["wn"]
            a1, a2 = deq(lw["gate"]) @ u, deq(lw["up"]) @ u
            mm = a1 / (1 + np.exp(-a1)) * a2
            h = h + deq(lw["down"]) @ mm
        u = h / math.sqrt(np.mean(h * h) + 1e-6) * w["wn_final"]
        ref = deq(w["head"]) @ u
        assert np.max(np.abs(logits - ref)) < 1e-4 * (np.max(np.abs(ref)) + 1)
        top2 = np.sort(ref)[-2:]
        if top2[1] - top2[0] > 1e-3:
            assert nxt == int(np.argmax(ref))
        # the next step depends only on the token: resuming reproduces it
        assert oracle.chain_step(w, tok)[1] == nxt
        tok = nxt


# ---------------------------------------------------------------------------
# atq: the attention step (readings in oracle/q4_oracle.c), pinned against an
# independent binary64 forward pass and against closed forms
# ---------------------------------------------------------------------------
def _atq_run(a):
    kc, vc = a["kcache"].copy(), a["vcache"].copy()
    o, os_ = oracle.atq(a["q"], a["g"], a["k"], a["v"], a["wq"], a["wk"], a["eps"], a["cos"],
                        a["sin"], kc, vc, a["pos"])
    return o, os_, kc, vc


def _atq_ref64(a):
    D = 128
    hq, hkv, pos = a["hq"], a["hkv"], a["pos"]
    grp = hq // hkv
    eps = float(a["eps"])
    c, s = a["cos"].astype(np.float64), a["sin"].astype(np.float64)

    def norm(x, w):
        x = x.astype(np.float64)
        return x / np.sqrt(np.mean(x * x) + eps) * w.astype(np.float64)

    def rot(x):
        lo, hi = x[:D // 2], x[D // 2:]
        return np.concatenate([lo * c - hi * s, lo * s + hi * c])

    K = a["kcache"].astype(np.float64).copy()
    V = a["vcache"].astype(np.float64).copy()
    for j in range(hkv):
        K[j, pos] = rot(norm(a["k"][j * D:(j + 1) * D], a["wk"]))
        V[j, pos] = a["v"][j * D:(j + 1) * D]
    o = np.empty(hq * D)
    for h in range(hq):
        j = h // grp
        qr = rot(norm(a["q"][h * D:(h + 1) * D], a["wq"]))
        sc = K[j, :pos + 1] @ qr / np.sqrt(D)
        p = np.exp(sc - sc.max())
        w = (p @ V[j, :pos + 1]) / p.sum()
        g = a["g"][h * D:(h + 1) * D].astype(np.float64)
        o[h * D:(h + 1) * D] = w / (1.0 + np.exp(-g))
    return o, K, V


@pytest.mark.parametrize("pos,hq,hkv", [(0, 16, 4), (1, 16, 4), (63, 4, 2), (204, 16, 4),
                                        (300, 2, 2)])
def test_atq_matches_binary64_forward(pos, hq, hkv):
    a = synth.atq_inputs(seed=61 + pos, pos=pos, hq=hq, hkv=hkv, max_pos=512)
    o, os_, kc, vc = _atq_run(a)
    o64, K64, V64 = _atq_ref64(a)
    scale = np.sqrt(np.mean(o64 ** 2))
    assert np.max(np.abs(o - o64)) <= 2e-5 * scale, np.max(np.abs(o - o64)) / scale
    # the new cache rows; every other row untouched
    assert np.max(np.abs(kc[:, pos] - K64[:, pos])) <= 1e-5
    assert np.array_equal(vc[:, pos], a["v"].reshape(hkv, 128))
    keep = np.ones(512, bool)
    keep[pos] = False
    assert np.array_equal(kc[:, keep], a["kcache"][:, keep])
    assert np.array_equal(vc[:, keep], a["vcache"][:, keep])
    # group sums of o
    assert np.array_equal(os_, oracle.group_sums(o))


def test_atq_first_position_is_gated_value():
    """One position: the softmax weight is E(0) = 1 exactly, Z = 1, so o is
    the new value times the sigmoid of the gate."""
    a = synth.atq_inputs(seed=71, pos=0, max_pos=8)
    o, _, _, _ = _atq_run(a)
    v = a["v"].reshape(4, 128)
    sig = (1.0 / (1.0 + np.exp(-a["g"].astype(np.float64)))).astype(np.float32)
    want = np.repeat(v, 4, axis=0).ravel() * sig
    # the sigmoid may differ from libm's in its last bit
    assert np.max(np.abs(o - want) / np.maximum(np.abs(want), 1e-30)) <= 2.5e-7
    # values 1: o is the gate's sigmoid itself, taken in binary64 and rounded
    # once to binary32.  libm's binary64 exp is within an ulp of the fixed
    # exp, far below binary32's rounding step, so the bits agree (a sigmoid
    # evaluated in binary32 differs in a good share of them)
    a["v"] = np.ones_like(a["v"])
    o, _, _, _ = _atq_run(a)
    sig = (1.0 / (1.0 + np.exp(-a["g"].astype(np.float64)))).astype(np.float32)
    assert np.array_equal(o, sig)


def test_atq_equal_keys_weighted_sum_is_the_tree():
    """All keys equal (so every weight is exactly 1 and Z is the count) and
    a saturated gate (sigmoid exactly 1): o is T over the value column
    divided by the count, bit for bit."""
    pos = 37
    a = synth.atq_inputs(seed=72, pos=pos, max_pos=64)
    # the generator's normals sit on a 2^-16 grid, where any summation order
    # is exact; scaling by RN32(1/3) fills the significands, so the order of
    # the value sum shows in the bits
    third = np.float32(1.0 / 3.0)
    a["vcache"] = a["vcache"] * third
    a["v"] = a["v"] * third
    # the key the step writes at position pos, copied into every earlier row
    first = dict(a, pos=0, kcache=np.zeros_like(a["kcache"]), vcache=np.zeros_like(a["vcache"]))
    _, _, k0, _ = _atq_run(first)
    a["kcache"][:, :pos] = k0[:, :1]
    a["g"] = np.full_like(a["g"], 40.0)
    o, _, kc, vc = _atq_run(a)
    assert np.array_equal(kc[:, :pos + 1], np.repeat(k0[:, :1], pos + 1, axis=1))
    for h in range(16):
        j = h // 4
        col = np.array([oracle.tree(vc[j, :pos + 1, i]) for i in range(128)], np.float32)
        want = col / np.float32(pos + 1)
        assert np.array_equal(o[h * 128:(h + 1) * 128].view(np.uint32), want.view(np.uint32)), h


def test_atq_unit_values_give_unit_output():
    """Every value 1 and a saturated gate: the weighted sum and Z are the
    same tree over the same weights, so o is exactly 1 at every position
    count, whatever the scores."""
    for pos in (1, 6, 37, 200):
        a = synth.atq_inputs(seed=75 + pos, pos=pos, max_pos=256)
        a["vcache"][:, :pos] = 1.0
        a["v"] = np.ones_like(a["v"])
        a["g"] = np.full_like(a["g"], 40.0)
        o, _, _, _ = _atq_run(a)
        assert np.array_equal(o, np.ones_like(o)), pos


def test_atq_score_is_the_tree_of_products():
    """A score whose terms cancel only in the canonical tree order.  With
    eps = 0, q = 1 and wq = 1 the normed query is exactly 1; an identity
    rotation (c = 1, s = 0) keeps it; so the score of an earlier key row is
    T(row) * SCALE.  Row [2^30, 1 x 63, -2^30, 1 x 63]: T loses every 1
    against the 2^30 in each half and returns 0 (a left-to-right sum gives
    63).  The new key is zero (wk = 0), so both scores are 0, both weights
    E(0) = 1, and o = (V_0 + V_1) / 2 exactly."""
    a = synth.atq_inputs(seed=79, pos=1, hq=4, hkv=2, max_pos=4)
    a["eps"] = np.float32(0.0)
    a["q"] = np.ones_like(a["q"])
    a["wq"] = np.ones_like(a["wq"])
    a["k"] = np.ones_like(a["k"])
    a["wk"] = np.zeros_like(a["wk"])
    a["cos"] = np.ones_like(a["cos"])
    a["sin"] = np.zeros_like(a["sin"])
    a["g"] = np.full_like(a["g"], 40.0)
    row = np.ones(128, np.float32)
    row[0], row[64] = 2.0 ** 30, -(2.0 ** 30)
    a["kcache"][:, 0] = row
    # value rows on a coarse grid so that (V_0 + V_1) / 2 is exact
    a["vcache"][:, 0] = np.round(a["vcache"][:, 0] * 8) / 8
    a["v"] = np.round(a["v"] * 8) / 8
    o, _, kc, _ = _atq_run(a)
    assert np.array_equal(kc[:, 1].view(np.uint32), np.zeros((2, 128), np.uint32))
    mean = (a["vcache"][:, 0] + a["v"].reshape(2, 128)) / np.float32(2.0)
    want = np.repeat(mean, 2, axis=0).ravel()
    assert np.array_equal(o, want)


def test_atq_large_scores_stay_finite():
    a = synth.atq_inputs(seed=73, pos=100, max_pos=128)
    a["wq"] = a["wq"] * np.float32(30.0)  # scores ~ 30x larger
    o, _, _, _ = _atq_run(a)
    o64, _, _ = _atq_ref64(a)
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - o64)) <= 1e-4 * np.sqrt(np.mean(o64 ** 2))


def test_atq_rejects_shapes_outside_the_readings():
    a = synth.atq_inputs(seed=74, pos=3, hq=4, hkv=4, max_pos=8)
    with pytest.raises(ValueError):
        oracle.atq(a["q"], a["g"], a["k"][:3 * 128], a["v"][:3 * 128], a["wq"], a["wk"],
                   a["eps"], a["cos"], a["sin"], a["kcache"][:3].copy(), a["vcache"][:3].copy(), 3)
    with pytest.raises(ValueError):
        oracle.atq(a["q"], a["g"], a["k"], a["v"], a["wq"], a["wk"], a["eps"], a["cos"],
                   a["sin"], a["kcache"], a["vcache"], 8)


# ---------------------------------------------------------------------------
# the decode chain with attention, composed from the pieces above
# ---------------------------------------------------------------------------
def test_attn_chain_steps_against_binary64_forward():
    """Four steps (positions 0..3) of a 2-layer chain with attention against
    an independent binary64 forward pass that keeps its own caches."""
    w = synth.attn_chain_weights(seed=23, layers=2, hidden=128, inter=192, vocab=1000, hq=2,
                                 hkv=1, max_pos=8)
    D, hq, hkv = 128, 2, 1

    def deq(m):
        c = unpack_codes(m["q"], m["cols"]).astype(np.float64)
        g = np.arange(m["cols"]) // 64
        return c * m["s"][:, g].astype(np.float64) + m["b"][:, g].astype(np.float64)

    def norm(x, wt):
        return x / math.sqrt(np.mean(x * x) + 1e-6) * wt.astype(np.float64)

    def rot(x, pos):
        c, s = w["cos_tab"][pos].astype(np.float64), w["sin_tab"][pos].astype(np.float64)
        lo, hi = x[:D // 2], x[D // 2:]
        return np.concatenate([lo * c - hi * s, lo * s + hi * c])

    kc, vc = oracle.attn_caches(w)
    K64 = [np.zeros((hkv, 8, D)) for _ in range(2)]
    V64 = [np.zeros((hkv, 8, D)) for _ in range(2)]
    tok = w["tok0"]
    for pos in range(4):
        logits, nxt = oracle.attn_chain_step(w, tok, pos, kc, vc)
        h = deq(w["head"])[tok]
        for l, lw in enumerate(w["layers"]):
            y = deq(lw["qgkv"]) @ norm(h, lw["wa"])
            q, g = y[:hq * D], y[hq * D:2 * hq * D]
            k, v = y[2 * hq * D:2 * hq * D + hkv * D], y[2 * hq * D + hkv * D:]
            K64[l][0, pos] = rot(norm(k, lw["wk"]), pos)
            V64[l][0, pos] = v
            o = np.empty(hq * D)
            for hh in range(hq):
                qr = rot(norm(q[hh * D:(hh + 1) * D], lw["wq"]), pos)
                sc = K64[l][0, :pos + 1] @ qr / math.sqrt(D)
                p = np.exp(sc - sc.max())
                o[hh * D:(hh + 1) * D] = (p @ V64[l][0, :pos + 1]) / p.sum() / (
                    1 + np.exp(-g[hh * D:(hh + 1) * D]))
            h = h + deq(lw["o"]) @ o
            u = norm(h, lw["wn"])
            a1, a2 = deq(lw["gate"]) @ u, deq(lw["up"]) @ u
            h = h + deq(lw["down"]) @ (a1 / (1 + np.exp(-a1)) * a2)
        ref = deq(w["head"]) @ norm(h, w["wn_final"])
        assert np.max(np.abs(logits - ref)) < 1e-4 * (np.max(np.abs(ref)) + 1), pos
        top2 = np.sort(ref)[-2:]
        if top2[1] - top2[0] > 1e-3:
            assert nxt == int(np.argmax(ref))
        # the caches hold the rotated keys and the values of every position so far
        assert np.max(np.abs(kc[0][0, :pos + 1] - K64[0][0, :pos + 1])) < 1e-4 * np.max(
            np.abs(K64[0][0, :pos + 1]))
        tok = nxt


# ---------------------------------------------------------------------------
# FNV-1a (32 bit): the hash of an output's bytes that the 400-call product
# check and the chains' per-step logits checks compare.  Pinned by the
# algorithm's published test vectors (Fowler/Noll/Vo reference suite), not
# by a second implementation of it.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("text,want", [
    (b"", 0x811C9DC5),      # the offset basis itself
    (b"a", 0xE40C292C),
    (b"foobar", 0xBF9CF968),
])
def test_fnv1a32_published_vectors(text, want):
    assert oracle.fnv1a32(np.frombuffer(text, dtype=np.uint8)) == want


def test_fnv1a32_hashes_the_little_endian_bytes_of_floats():
    # the same bytes give the same hash whatever the array's type; one
    # flipped bit of one value changes it
    y = synth.normal_f32(3, "fnv.y", (4096,), 0.0, 1.0)
    h = oracle.fnv1a32(y)
    assert h == oracle.fnv1a32(y.view(np.uint8))
    assert h == oracle.fnv1a32(np.frombuffer(y.astype("<f4").tobytes(), dtype=np.uint8))
    z = y.copy()
    z.view(np.uint32)[1234] ^= 1
    assert oracle.fnv1a32(z) != h
