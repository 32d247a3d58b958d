"""CPU oracle for the affine 4-bit matvec and its producers.

TEST INFRASTRUCTURE ONLY: only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  It is the plain,
slow reference the GPU library is checked against, and shares no code with
that library (it never imports it, and the library never imports this).

The arithmetic lives in ``q4_oracle.c`` (plain C compiled by gcc with
``-ffp-contract=off``); this module only marshals numpy arrays.  The chain
step composes those C functions in the order the decode chain defines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
GROUP = 64

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.orc_tree.argtypes = [_f32p, _i64]
        L.orc_tree.restype = ctypes.c_float
        L.orc_group_sums.argtypes = [_f32p, _i64, _f32p]
        L.orc_group_sums.restype = None
        L.orc_code.argtypes = [_u32p, _i64, _i64, _i64]
        L.orc_code.restype = ctypes.c_uint32
        L.orc_q4mv.argtypes = [_u32p, _f32p, _f32p, _f32p, _f32p, _f32p, _i64, _i64, ctypes.c_int]
        L.orc_q4mv.restype = None
        L.orc_q4mv_sample.argtypes = [_u32p, _f32p, _f32p, _f32p, _f32p, _f32p, _i64, _i64p, _i64]
        L.orc_q4mv_sample.restype = None
        L.orc_rmsq.argtypes = [_f32p, _f32p, _i64, ctypes.c_float, _f32p, _f32p]
        L.orc_rmsq.restype = ctypes.c_int
        L.orc_exp.argtypes = [ctypes.c_double]
        L.orc_exp.restype = ctypes.c_double
        L.orc_swq.argtypes = [_f32p, _i64, _f32p, _f32p]
        L.orc_swq.restype = ctypes.c_int
        L.orc_argmax.argtypes = [_f32p, _i64]
        L.orc_argmax.restype = ctypes.c_int32
        L.orc_embed.argtypes = [_u32p, _f32p, _f32p, _i64, _i64, _i64, _f32p]
        L.orc_embed.restype = None
        L.orc_add.argtypes = [_f32p, _f32p, _f32p, _i64]
        L.orc_add.restype = None
        L.orc_fnv1a32.argtypes = [ctypes.c_void_p, _i64]
        L.orc_atq.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_float, _f32p,
                              _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _f32p, _f32p]
        L.orc_atq.restype = ctypes.c_int
        L.orc_fnv1a32.restype = ctypes.c_uint32
        _lib = L
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def tree(v) -> np.float32:
    """Canonical tree sum T of a non-empty binary32 vector."""
    v = _f32(v).ravel()
    if v.size < 1:
        raise ValueError("T needs at least one value")
    return np.float32(lib().orc_tree(v, v.size))


def group_sums(x) -> np.ndarray:
    """``xs[g] = T(x[64g .. 64g+63])``."""
    x = _f32(x).ravel()
    if x.size % GROUP or x.size == 0:
        raise ValueError("length must be a positive multiple of 64")
    xs = np.empty(x.size // GROUP, np.float32)
    lib().orc_group_sums(x, x.size, xs)
    return xs


def code(q, cols: int, r: int, c: int) -> int:
    return int(lib().orc_code(np.ascontiguousarray(q, dtype=np.uint32).ravel(), cols, r, c))


def _check_mat(m, x, xs):
    rows, cols = m["rows"], m["cols"]
    q = np.ascontiguousarray(m["q"], dtype=np.uint32).ravel()
    s = _f32(m["s"]).ravel()
    b = _f32(m["b"]).ravel()
    x = _f32(x).ravel()
    xs = _f32(xs).ravel()
    G = cols // GROUP
    if cols % GROUP or rows < 1:
        raise ValueError("bad shape")
    if q.size != rows * cols // 8 or s.size != rows * G or b.size != rows * G:
        raise ValueError("matrix arrays do not match rows x cols")
    if x.size != cols or xs.size != G:
        raise ValueError("x / xs do not match cols")
    return q, s, b, x, xs


def q4mv(m: dict, x, xs, nthreads: int = 1) -> np.ndarray:
    """Fixed-order q4mv of every row (rows split over ``nthreads`` threads;
    the bits do not depend on the split)."""
    q, s, b, x, xs = _check_mat(m, x, xs)
    y = np.empty(m["rows"], np.float32)
    lib().orc_q4mv(q, s, b, x, xs, y, m["rows"], m["cols"], int(nthreads))
    return y


def q4mv_sample(m: dict, x, xs, idx) -> np.ndarray:
    """Fixed-order q4mv of the rows listed in ``idx``."""
    q, s, b, x, xs = _check_mat(m, x, xs)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= m["rows"]):
        raise IndexError("row index out of range")
    y = np.empty(idx.size, np.float32)
    lib().orc_q4mv_sample(q, s, b, x, xs, y, m["cols"], idx, idx.size)
    return y


def rmsq(h, w, eps):
    """RMS norm with weights plus group sums: returns ``(u, us)``."""
    h = _f32(h).ravel()
    w = _f32(w).ravel()
    if h.size != w.size:
        raise ValueError("h and w differ in length")
    u = np.empty(h.size, np.float32)
    us = np.empty(max(h.size // GROUP, 1), np.float32)
    if lib().orc_rmsq(h, w, h.size, float(np.float32(eps)), u, us) != 0:
        raise ValueError("rmsq needs a positive multiple of 64 values")
    return u, us


def exp(t: float) -> float:
    """The fixed binary64 exp used by swq."""
    return lib().orc_exp(float(t))


def swq(a, n: int):
    """SwiGLU of ``a = [gate | up]`` (2n values) plus group sums:
    returns ``(o, os)``."""
    a = _f32(a).ravel()
    if a.size != 2 * n:
        raise ValueError("a must hold 2n values")
    o = np.empty(n, np.float32)
    os_ = np.empty(max(n // GROUP, 1), np.float32)
    if lib().orc_swq(a, n, o, os_) != 0:
        raise ValueError("swq needs n to be a positive multiple of 64")
    return o, os_


def argmax(v) -> int:
    v = _f32(v).ravel()
    return int(lib().orc_argmax(v, v.size))


def embed(m: dict, tok: int) -> np.ndarray:
    q = np.ascontiguousarray(m["q"], dtype=np.uint32).ravel()
    e = np.empty(m["cols"], np.float32)
    lib().orc_embed(q, _f32(m["s"]).ravel(), _f32(m["b"]).ravel(),
                    m["rows"], m["cols"], int(tok), e)
    return e


def add(a, b) -> np.ndarray:
    a = _f32(a).ravel()
    b = _f32(b).ravel()
    out = np.empty_like(a)
    lib().orc_add(a, b, out, a.size)
    return out


def fnv1a32(arr) -> int:
    arr = np.ascontiguousarray(arr)
    return int(lib().orc_fnv1a32(arr.ctypes.data, arr.nbytes))


ATQ_D = 128


def atq(q, g, k, v, wq, wk, eps, cos, sin, kcache, vcache, pos: int):
    """One decode token of gated attention over key/value caches (the
    readings in q4_oracle.c): writes row ``pos`` of ``kcache`` and
    ``vcache`` (float32 [hkv, max_pos, 128], updated in place) and returns
    ``(o, os)`` for ``hq = q.size / 128`` query heads."""
    q, g, k, v = (_f32(a).ravel() for a in (q, g, k, v))
    wq, wk, cos, sin = (_f32(a).ravel() for a in (wq, wk, cos, sin))
    if not (kcache.dtype == np.float32 and kcache.flags.c_contiguous and
            vcache.dtype == np.float32 and vcache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous float32 arrays")
    hq, hkv = q.size // ATQ_D, k.size // ATQ_D
    max_pos = kcache.shape[1]
    if kcache.shape != (hkv, max_pos, ATQ_D) or vcache.shape != kcache.shape:
        raise ValueError("caches must be [hkv, max_pos, 128]")
    if g.size != q.size or v.size != k.size or wq.size != ATQ_D or wk.size != ATQ_D:
        raise ValueError("shape mismatch")
    if cos.size != ATQ_D // 2 or sin.size != ATQ_D // 2:
        raise ValueError("rotation tables hold 64 values")
    o = np.empty(q.size, np.float32)
    os_ = np.empty(q.size // GROUP, np.float32)
    if lib().orc_atq(q, g, k, v, wq, wk, float(np.float32(eps)), cos, sin, kcache, vcache,
                     int(pos), int(max_pos), hq, hkv, o, os_) != 0:
        raise ValueError("atq: heads or position outside the readings")
    return o, os_


def chain_hidden(w: dict, tok: int, nthreads: int = 1, layers: int | None = None) -> np.ndarray:
    """The hidden state after the embedding and the MLP layers of one
    decode-chain step: h = embed(head, tok); per layer: u = rmsq(h, wn);
    a = [gate u | up u]; m = swq(a); h = h + down m."""
    L = len(w["layers"]) if layers is None else layers
    inter = w["inter"]
    h = embed(w["head"], tok)
    for l in range(L):
        lw = w["layers"][l]
        u, us = rmsq(h, lw["wn"], w["eps"])
        a = np.empty(2 * inter, np.float32)
        a[:inter] = q4mv(lw["gate"], u, us, nthreads)
        a[inter:] = q4mv(lw["up"], u, us, nthreads)
        m, ms = swq(a, inter)
        h = add(h, q4mv(lw["down"], m, ms, nthreads))
    return h


def attn_caches(w: dict, layers: int | None = None):
    """Empty key and value caches of an attention chain: one float32
    [hkv, max_pos, 128] pair per layer."""
    L = len(w["layers"]) if layers is None else layers
    shape = (w["hkv"], w["max_pos"], ATQ_D)
    return ([np.zeros(shape, np.float32) for _ in range(L)],
            [np.zeros(shape, np.float32) for _ in range(L)])


def attn_chain_hidden(w: dict, tok: int, pos: int, kc: list, vc: list, nthreads: int = 1,
                      layers: int | None = None) -> np.ndarray:
    """The hidden state of one decode step of a chain with attention, at
    position ``pos`` (the caches ``kc``, ``vc`` get row ``pos`` of every
    layer): h = embed(head, tok); per layer: u = rmsq(h, wa); [q; g; k; v]
    = qgkv u; o = atq(q, g, k, v, ...); h = h + O o; then the MLP block of
    ``chain_hidden``."""
    L = len(w["layers"]) if layers is None else layers
    hq, hkv, D = w["hq"], w["hkv"], ATQ_D
    inter = w["inter"]
    h = embed(w["head"], tok)
    for l in range(L):
        lw = w["layers"][l]
        u, us = rmsq(h, lw["wa"], w["eps"])
        y = q4mv(lw["qgkv"], u, us, nthreads)
        q, g = y[:hq * D], y[hq * D:2 * hq * D]
        k, v = y[2 * hq * D:2 * hq * D + hkv * D], y[2 * hq * D + hkv * D:]
        o, os_ = atq(q, g, k, v, lw["wq"], lw["wk"], w["eps"], w["cos_tab"][pos],
                     w["sin_tab"][pos], kc[l], vc[l], pos)
        h = add(h, q4mv(lw["o"], o, os_, nthreads))
        u, us = rmsq(h, lw["wn"], w["eps"])
        a = np.empty(2 * inter, np.float32)
        a[:inter] = q4mv(lw["gate"], u, us, nthreads)
        a[inter:] = q4mv(lw["up"], u, us, nthreads)
        m, ms = swq(a, inter)
        h = add(h, q4mv(lw["down"], m, ms, nthreads))
    return h


def attn_chain_step(w: dict, tok: int, pos: int, kc: list, vc: list, nthreads: int = 1,
                    layers: int | None = None):
    """One step of the chain with attention: ``attn_chain_hidden``, then
    the final norm, the head and argmax.  Returns ``(logits, next_token)``."""
    h = attn_chain_hidden(w, tok, pos, kc, vc, nthreads, layers)
    u, us = rmsq(h, w["wn_final"], w["eps"])
    logits = q4mv(w["head"], u, us, nthreads)
    return logits, argmax(logits)


def chain_step(w: dict, tok: int, nthreads: int = 1, layers: int | None = None):
    """One decode-chain step from token ``tok``: the hidden state of
    ``chain_hidden``, then u = rmsq(h, wn_final), logits = head u, next
    token = argmax(logits).  Returns ``(logits, next_token)``."""
    h = chain_hidden(w, tok, nthreads, layers)
    u, us = rmsq(h, w["wn_final"], w["eps"])
    logits = q4mv(w["head"], u, us, nthreads)
    return logits, argmax(logits)
