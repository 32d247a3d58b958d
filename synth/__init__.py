"""Seeded synthetic inputs for the affine 4-bit matvec workloads.

This module is shared by the oracle's tests and by the GPU library's tests
and benchmark.  It holds none of the method's arithmetic (no group sums, no
products, no norms): it only draws tensors with the shapes and value
distributions of the workloads.

Generator (counter-based, machine independent):

* SplitMix64.  Stream ``key`` yields ``mix64(key + (i + 1) * GAMMA)`` for
  ``i = 0, 1, ...`` (all arithmetic mod 2**64), with the SplitMix64 finaliser
  ``mix64``.  Each tensor has its own stream; its key is
  ``mix64(mix64(seed + GAMMA) ^ fnv1a64(name))``.
* ``U(lo, hi)``: ``u = (z >> 40) * 2**-24`` and ``RN32(lo + (hi - lo) * u)``
  in binary64.
* ``N(mean, std)``: Irwin-Hall with twelve 16-bit uniforms taken from three
  draws, ``n = sum_k (f_k + 0.5) / 65536 - 6`` (exact in binary64; mean 0,
  variance 1, tails cut at +-6), then ``RN32(mean + std * n)``.  No
  transcendental function is used, so every host produces the same bytes.
* 4-bit codes: word ``2j`` of a code tensor is the low half of draw ``j`` and
  word ``2j + 1`` the high half; every nibble of a word is one code, so codes
  are uniform over 0..15.
* Bias of the affine Q4 matrices: ``RN32(-c * s + N(0, 1e-3))`` in binary64,
  where ``s`` is the binary32 scale of the same group and ``c`` the code
  centre: 8 for the single products (as their configurations state), 7.5
  for the decode chain's matrices (zero-mean dequantised weights).  With
  c = 8 every uniform-code weight carries a -0.5 s offset; in a 24-layer
  chain that rank-one drift dominates the residual stream, the head sees
  almost the same input for every token and greedy decoding sits on one
  token from the first step.
"""
from __future__ import annotations

import hashlib

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

DEFAULT_SEED = 20261202
GROUP = 64

_CHUNK = 1 << 22  # draws per chunk, bounds the temporaries


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def _fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for byte in text.encode():
        h ^= byte
        h = (h * 0x100000001B3) & _MASK64
    return h


def stream_key(seed: int, name: str) -> int:
    """Key of the independent stream of tensor ``name`` under ``seed``."""
    return _mix64_int(_mix64_int(seed + int(GAMMA)) ^ _fnv1a64(name))


def draws(seed: int, name: str, count: int, start: int = 0) -> np.ndarray:
    """Draws ``start .. start+count-1`` of the stream of ``name`` (uint64)."""
    key = np.uint64(stream_key(seed, name))
    out = np.empty(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            hi = min(count, lo + _CHUNK)
            z = np.arange(start + lo + 1, start + hi + 1, dtype=np.uint64)
            z *= GAMMA
            z += key
            z ^= z >> np.uint64(30)
            z *= _C1
            z ^= z >> np.uint64(27)
            z *= _C2
            z ^= z >> np.uint64(31)
            out[lo:hi] = z
    return out


def uniform_f32(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    u = (draws(seed, name, n) >> np.uint64(40)).astype(np.float64) * 2.0**-24
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


def _irwin_hall(z3: np.ndarray) -> np.ndarray:
    """Standard-normal stand-ins from rows of three uint64 draws."""
    total = np.zeros(z3.shape[0], dtype=np.float64)
    for k in range(3):
        z = z3[:, k]
        for sh in (0, 16, 32, 48):
            total += ((z >> np.uint64(sh)) & np.uint64(0xFFFF)).astype(np.float64)
    return (total + 6.0) / 65536.0 - 6.0


def normal_f64(seed: int, name: str, n: int) -> np.ndarray:
    """``n`` draws of N(0, 1) (Irwin-Hall, binary64, exact)."""
    out = np.empty(n, dtype=np.float64)
    per = _CHUNK // 3
    for lo in range(0, n, per):
        hi = min(n, lo + per)
        z = draws(seed, name, 3 * (hi - lo), start=3 * lo).reshape(hi - lo, 3)
        out[lo:hi] = _irwin_hall(z)
    return out


def normal_f32(seed: int, name: str, shape, mean: float, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    v = mean + std * normal_f64(seed, name, n)
    return v.astype(np.float32).reshape(shape)


def codes_u32(seed: int, name: str, rows: int, cols: int) -> np.ndarray:
    """Packed 4-bit codes, ``[rows, cols // 8]`` uint32, uniform 0..15."""
    if cols % 8:
        raise ValueError("cols must be a multiple of 8")
    words = rows * (cols // 8)
    d = draws(seed, name, (words + 1) // 2)
    return d.view(np.uint32)[:words].reshape(rows, cols // 8).copy()


def q4_matrix(seed: int, name: str, rows: int, cols: int,
              s_lo: float = 0.001, s_hi: float = 0.02, b_std: float = 1e-3,
              center: float = 8.0) -> dict:
    """An affine Q4 matrix: codes, fp32 scale U(s_lo, s_hi) and fp32 bias
    RN32(-center s + N(0, b_std)) per group of 64 columns."""
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 64")
    G = cols // GROUP
    q = codes_u32(seed, name + ".q", rows, cols)
    s = uniform_f32(seed, name + ".s", (rows, G), s_lo, s_hi)
    noise = normal_f64(seed, name + ".b", rows * G).reshape(rows, G)
    b = (-center * s.astype(np.float64) + b_std * noise).astype(np.float32)
    return {"q": q, "s": s, "b": b, "rows": rows, "cols": cols}


def randint(seed: int, name: str, high: int) -> int:
    """One integer uniform in [0, high) (by rejection-free modulo; the
    bias is < high / 2**64)."""
    return int(draws(seed, name, 1)[0] % np.uint64(high))


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# The workloads.  Shapes and distributions follow the five configurations:
# a 13x128 product, a 4096x2048 product, the 248320x2048 output head fed by an
# RMS norm, a 24-layer product set, and a 24-layer decode chain.
# ---------------------------------------------------------------------------
HIDDEN = 2048
INTER = 6144
VOCAB = 248320
LAYERS = 24
EPS = 1e-6
CHAIN_CENTER = 7.5


def small_product(seed: int = DEFAULT_SEED, rows: int = 13, cols: int = 128,
                  name: str = "small") -> dict:
    """q4mv inputs with x ~ N(0, 1) (group sums are left to the caller)."""
    m = q4_matrix(seed, name + ".w", rows, cols)
    m["x"] = normal_f32(seed, name + ".x", (cols,), 0.0, 1.0)
    return m


def head_inputs(seed: int = DEFAULT_SEED, rows: int = VOCAB, cols: int = HIDDEN,
                copy: int = 0) -> dict:
    """Output head: Q4 matrix plus the rmsq inputs z ~ N(0,1), wn ~ N(1,0.1).
    ``copy`` selects an independently drawn weight copy (same x)."""
    m = q4_matrix(seed, "head.w%d" % copy if copy else "head.w", rows, cols)
    m["z"] = normal_f32(seed, "head.z", (cols,), 0.0, 1.0)
    m["wn"] = normal_f32(seed, "head.wn", (cols,), 1.0, 0.1)
    m["eps"] = np.float32(EPS)
    return m


PRODUCT_SET_LAYER = (  # (name, rows, cols, stage-in-layer)
    ("q", 2048, 2048, 0), ("k", 512, 2048, 0), ("v", 512, 2048, 0),
    ("o", 2048, 2048, 1),
    ("gate", 6144, 2048, 2), ("up", 6144, 2048, 2),
    ("down", 2048, 6144, 3),
)


def product_set(seed: int = DEFAULT_SEED, layers: int = LAYERS, vocab: int = VOCAB) -> dict:
    """One synthetic decode step's product set: per layer Q, K, V (stage 0),
    O (stage 1), gate and up (stage 2), down (stage 3); then the head in a
    last stage.  Every product reads a fixed seeded x of its width."""
    prods = []
    for l in range(layers):
        for name, rows, cols, st in PRODUCT_SET_LAYER:
            m = q4_matrix(seed, "ps.l%d.%s" % (l, name), rows, cols)
            m["stage"] = 4 * l + st
            m["name"] = "l%d.%s" % (l, name)
            prods.append(m)
    head = q4_matrix(seed, "ps.head", vocab, HIDDEN)
    head["stage"] = 4 * layers
    head["name"] = "head"
    prods.append(head)
    xs = {c: normal_f32(seed, "ps.x%d" % c, (c,), 0.0, 1.0) for c in (HIDDEN, INTER)}
    return {"products": prods, "x": xs, "stages": 4 * layers + 1}


def chain_weights(seed: int = DEFAULT_SEED, layers: int = LAYERS, hidden: int = HIDDEN,
                  inter: int = INTER, vocab: int = VOCAB) -> dict:
    """Decode-chain weights: per layer an RMS-norm weight N(1, 0.1) and
    gate, up (inter x hidden) and down (hidden x inter) Q4 matrices; a final
    norm weight; a vocab x hidden head, also used as the tied embedding.
    The Q4 matrices use the code centre 7.5 (zero-mean weights)."""
    lay = []
    for l in range(layers):
        lay.append({
            "wn": normal_f32(seed, "ch.l%d.wn" % l, (hidden,), 1.0, 0.1),
            "gate": q4_matrix(seed, "ch.l%d.gate" % l, inter, hidden, center=CHAIN_CENTER),
            "up": q4_matrix(seed, "ch.l%d.up" % l, inter, hidden, center=CHAIN_CENTER),
            "down": q4_matrix(seed, "ch.l%d.down" % l, hidden, inter, center=CHAIN_CENTER),
        })
    return {
        "layers": lay,
        "wn_final": normal_f32(seed, "ch.wn_final", (hidden,), 1.0, 0.1),
        "head": q4_matrix(seed, "ch.head", vocab, hidden, center=CHAIN_CENTER),
        "tok0": randint(seed, "ch.tok0", vocab),
        "eps": np.float32(EPS),
        "hidden": hidden, "inter": inter, "vocab": vocab,
    }


ATQ_D = 128
ATQ_HQ = 16       # query heads of the 2048-wide Q product
ATQ_HKV = 4       # key/value heads of the 512-wide K and V products
ATQ_MAX_POS = 4096
ROPE_BASE = 10000.0


def rope_table(pos: int, d: int = ATQ_D, base: float = ROPE_BASE):
    """The rotation table of position ``pos``: cos and sin of
    pos * base^(-2i/d), i < d/2, rounded to binary32 (an input of the
    attention step, like the activations)."""
    i = np.arange(d // 2, dtype=np.float64)
    ang = float(pos) * np.power(base, -2.0 * i / d)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_tables(max_pos: int, d: int = ATQ_D, base: float = ROPE_BASE):
    """The rotation tables of positions 0 .. max_pos-1 as [max_pos, d/2]
    arrays (row p is ``rope_table(p)``)."""
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * np.power(base, -2.0 * i / d)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def atq_inputs(seed: int = DEFAULT_SEED, pos: int = 204, hq: int = ATQ_HQ, hkv: int = ATQ_HKV,
               max_pos: int = ATQ_MAX_POS) -> dict:
    """One decode token of the attention step at position ``pos``: q, gate
    (hq x 128) and k, v (hkv x 128) ~ N(0, 1); norm weights wq, wk ~
    N(1, 0.1); the position's rotation table (and the tables of every
    position of the cache); key and value caches
    [hkv, max_pos, 128] whose rows below ``pos`` hold N(0, 1) values (the
    earlier tokens) and zeros above."""
    kc = np.zeros((hkv, max_pos, ATQ_D), np.float32)
    vc = np.zeros((hkv, max_pos, ATQ_D), np.float32)
    if pos > 0:
        kc[:, :pos] = normal_f32(seed, "atq.kcache", (hkv, pos, ATQ_D), 0.0, 1.0)
        vc[:, :pos] = normal_f32(seed, "atq.vcache", (hkv, pos, ATQ_D), 0.0, 1.0)
    c, s = rope_table(pos)
    ct, st = rope_tables(max_pos)
    return {
        "q": normal_f32(seed, "atq.q", (hq * ATQ_D,), 0.0, 1.0),
        "g": normal_f32(seed, "atq.g", (hq * ATQ_D,), 0.0, 1.0),
        "k": normal_f32(seed, "atq.k", (hkv * ATQ_D,), 0.0, 1.0),
        "v": normal_f32(seed, "atq.v", (hkv * ATQ_D,), 0.0, 1.0),
        "wq": normal_f32(seed, "atq.wq", (ATQ_D,), 1.0, 0.1),
        "wk": normal_f32(seed, "atq.wk", (ATQ_D,), 1.0, 0.1),
        "cos": c, "sin": s, "cos_tab": ct, "sin_tab": st,
        "kcache": kc, "vcache": vc, "pos": pos,
        "eps": np.float32(EPS), "hq": hq, "hkv": hkv, "max_pos": max_pos,
    }


def attn_chain_weights(seed: int = DEFAULT_SEED, layers: int = LAYERS, hidden: int = HIDDEN,
                       inter: int = INTER, vocab: int = VOCAB, hq: int = ATQ_HQ,
                       hkv: int = ATQ_HKV, max_pos: int = 256) -> dict:
    """Decode-chain weights with an attention block in every layer: the MLP
    chain's weights (``chain_weights``), plus per layer an RMS-norm weight
    wa ~ N(1, 0.1), the [Q; gate; K; V] matrix ((2 hq + 2 hkv) * 128 rows x
    hidden), the query and key norm weights wq, wk ~ N(1, 0.1) (128 each)
    and O (hidden x hq * 128), all Q4 matrices with the chain's code centre;
    and the rotation tables of ``max_pos`` positions."""
    w = chain_weights(seed, layers, hidden, inter, vocab)
    rows = (2 * hq + 2 * hkv) * ATQ_D
    for l, lw in enumerate(w["layers"]):
        lw["wa"] = normal_f32(seed, "ach.l%d.wa" % l, (hidden,), 1.0, 0.1)
        lw["qgkv"] = q4_matrix(seed, "ach.l%d.qgkv" % l, rows, hidden, center=CHAIN_CENTER)
        lw["wq"] = normal_f32(seed, "ach.l%d.wq" % l, (ATQ_D,), 1.0, 0.1)
        lw["wk"] = normal_f32(seed, "ach.l%d.wk" % l, (ATQ_D,), 1.0, 0.1)
        lw["o"] = q4_matrix(seed, "ach.l%d.o" % l, hidden, hq * ATQ_D, center=CHAIN_CENTER)
    w["cos_tab"], w["sin_tab"] = rope_tables(max_pos)
    w.update(hq=hq, hkv=hkv, max_pos=max_pos)
    return w
