"""Affine 4-bit matvec (q4mv) for AMD Instinct MI355X: Python binding.

A thin ctypes layer over ``libq4mv.so`` (the C ABI in ``include/q4mv.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks and marshals torch tensors (device memory) and streams.  There
is no CPU path: if the library is missing, importing this package fails.

Names follow the C ABI: ``q4mv``, ``q4mv_add``, ``rmsq``, ``swq``,
``q4_argmax``, ``q4_embed``, the stage queue ``Queue`` (``q4mv_queue``,
``q4_stage``, ``q4mv_wait``) and graph capture ``Graph``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FIXED", "FAST", "Q4Error", "Q4Matrix", "q4mv", "q4mv_add", "q4mv_norm",
    "q4mv_norm_swiglu", "q4mv_norm_argmax", "q4mv_norm_argmax_noalloc", "q4mv_argmax_ws_bytes",
    "q4mv_variant", "VARIANTS",
    "rmsq", "swq",
    "q4_argmax", "q4_argmax_ws_bytes", "q4_embed", "Queue", "Graph", "q4_sync",
    "MlpLayer", "q4_decode_layers", "q4_decode_layers_ws_bytes", "q4_decode_layers_status",
    "q4_decode_token",
    "Mailbox", "library_path", "q4_atq", "q4_atq_ws_bytes", "q4_atq_status", "q4_pos_advance",
    "AttnBlock", "BlockStack", "q4_decode_block", "q4_decode_blocks", "q4_decode_block_ws_bytes",
    "q4_decode_block_status",
]

FIXED = 0
FAST = 1
WAIT_STREAM, WAIT_MAILBOX = 0, 1
Q4_OK, Q4_EINVAL, Q4_EHIP, Q4_ETIMEOUT, Q4_ESTATE, Q4_ENOMEM = 0, -1, -2, -3, -4, -5
MAX_COLS = 32768
MAX_RMSQ_N = 8192
MAX_DECODE_LAYERS = 32
ATQ_D = 128
ATQ_MAX_POS = 4096

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libq4mv.so")

if not os.path.exists(library_path):
    raise ImportError(
        "libq4mv.so is not built (expected at %s); build it with "
        "`python -c 'import __graft_entry__ as g; g.build()'`" % library_path)


class _Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class _MlpLayer(ctypes.Structure):
    _fields_ = [("gate_up", _Mat), ("down", _Mat), ("wn", ctypes.c_void_p)]


class _AttnBlock(ctypes.Structure):
    _fields_ = [("qgkv", _Mat), ("o", _Mat), ("wa", ctypes.c_void_p), ("wq", ctypes.c_void_p),
                ("wk", ctypes.c_void_p), ("kcache", ctypes.c_void_p),
                ("vcache", ctypes.c_void_p), ("hkv", ctypes.c_int32), ("mlp", _MlpLayer)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_lib = ctypes.CDLL(library_path)
_SIGS = {
    "q4mv": ([ctypes.POINTER(_Mat), _vp, _vp, _vp, ctypes.c_int, _vp], ctypes.c_int),
    "q4mv_add": ([ctypes.POINTER(_Mat), _vp, _vp, _vp, _vp, ctypes.c_int, _vp], ctypes.c_int),
    "q4mv_norm": ([ctypes.POINTER(_Mat), _vp, _vp, ctypes.c_float, _vp, _vp, _vp, ctypes.c_int, _vp],
                  ctypes.c_int),
    "q4mv_norm_swiglu": ([ctypes.POINTER(_Mat), _vp, _vp, ctypes.c_float, _vp, ctypes.c_int, _vp],
                         ctypes.c_int),
    "q4mv_argmax_ws_bytes": ([], ctypes.c_size_t),
    "q4mv_norm_argmax": ([ctypes.POINTER(_Mat), _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                          ctypes.c_size_t, ctypes.c_int, _vp], ctypes.c_int),
    "q4mv_norm_argmax_noalloc": ([ctypes.POINTER(_Mat), _vp, _vp, ctypes.c_float, _vp, _vp,
                                  ctypes.c_int, _vp], ctypes.c_int),
    "q4mv_variant": ([ctypes.POINTER(_Mat), _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp],
                     ctypes.c_int),
    "rmsq": ([_vp, _vp, _i32, ctypes.c_float, _vp, _vp, _vp], ctypes.c_int),
    "swq": ([_vp, _i32, _vp, _vp, ctypes.c_int, _vp], ctypes.c_int),
    "q4_argmax_ws_bytes": ([_i32], ctypes.c_size_t),
    "q4_argmax": ([_vp, _i32, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "q4_embed": ([ctypes.POINTER(_Mat), _vp, _vp, _vp], ctypes.c_int),
    "q4_decode_layers_ws_bytes": ([], ctypes.c_size_t),
    "q4_decode_layers": ([ctypes.POINTER(_Mat), _vp, ctypes.POINTER(_MlpLayer), _i32,
                          ctypes.c_float, _vp, _vp, ctypes.c_size_t, ctypes.c_int, _vp],
                         ctypes.c_int),
    "q4_decode_layers_status": ([_vp, _vp], ctypes.c_int),
    "q4_decode_token": ([ctypes.POINTER(_Mat), _vp, ctypes.POINTER(_MlpLayer), _i32, _vp,
                         ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, ctypes.c_int, _vp],
                        ctypes.c_int),
    "q4_atq_ws_bytes": ([_i32, _i32], ctypes.c_size_t),
    "q4_atq": ([_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _i32,
                _i32, _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "q4_atq_status": ([_vp, _i32, _i32, _vp], ctypes.c_int),
    "q4_pos_advance": ([_vp, _vp], ctypes.c_int),
    "q4_decode_block_ws_bytes": ([], ctypes.c_size_t),
    "q4_decode_block": ([ctypes.POINTER(_AttnBlock), ctypes.c_float, _vp, _vp, _i32, _vp, _vp, _vp,
                         ctypes.c_size_t, ctypes.c_int, _vp], ctypes.c_int),
    "q4_decode_block_status": ([_vp, _vp], ctypes.c_int),
    "q4_block_stack_create": ([ctypes.POINTER(_AttnBlock), _i32, _i32, ctypes.POINTER(_vp)],
                              ctypes.c_int),
    "q4_block_stack_destroy": ([_vp], ctypes.c_int),
    "q4_decode_blocks": ([_vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                          ctypes.c_int, _vp], ctypes.c_int),
    "q4_queue_create": ([_vp, ctypes.c_int, ctypes.POINTER(_vp)], ctypes.c_int),
    "q4_queue_destroy": ([_vp], ctypes.c_int),
    "q4mv_queue": ([_vp, ctypes.POINTER(_Mat), _vp, _vp, _vp], ctypes.c_int),
    "q4_stage": ([_vp], ctypes.c_int),
    "q4mv_wait": ([_vp], ctypes.c_int),
    "q4_capture_begin": ([_vp], ctypes.c_int),
    "q4_capture_end": ([_vp, ctypes.POINTER(_vp)], ctypes.c_int),
    "q4_graph_launch": ([_vp, _vp], ctypes.c_int),
    "q4_graph_destroy": ([_vp], ctypes.c_int),
    "q4_queue_set_wait": ([_vp, ctypes.c_int, _i32], ctypes.c_int),
    "q4_mailbox_create": ([_i32, ctypes.POINTER(_vp)], ctypes.c_int),
    "q4_mailbox_destroy": ([_vp], ctypes.c_int),
    "q4_mailbox_post": ([_vp, _vp, _vp], ctypes.c_int),
    "q4_mailbox_wait": ([_vp, ctypes.c_uint32, _vp, _i32], ctypes.c_int),
    "q4_mailbox_seq": ([_vp], ctypes.c_uint32),
    "q4_sync": ([_vp], ctypes.c_int),
    "q4_strerror": ([ctypes.c_int], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class Q4Error(RuntimeError):
    def __init__(self, call: str, code: int):
        super().__init__("%s: %s (%d)" % (call, _lib.q4_strerror(code).decode(), code))
        self.code = code


def _check(call: str, code: int) -> None:
    if code != Q4_OK:
        raise Q4Error(call, code)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, numel: int | None, what: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % what)
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor" % (what, dtype))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d values, not %d" % (what, numel, t.numel()))
    return t.data_ptr()


class Q4Matrix:
    """An affine Q4 matrix on the GPU: ``q`` int32 view of packed codes
    ``[rows, cols/8]`` (column 8j+k in bits 4k..4k+3 of word j), ``s`` and
    ``b`` float32 ``[rows, cols/64]``."""

    def __init__(self, q: torch.Tensor, s: torch.Tensor, b: torch.Tensor, rows: int, cols: int):
        if cols % 64 or cols < 64 or rows < 1:
            raise ValueError("rows >= 1 and cols a positive multiple of 64 required")
        G = cols // 64
        if q.dtype not in (torch.int32, torch.uint32):
            raise ValueError("q must be a 32-bit integer tensor")
        _dev(q.view(torch.int32), torch.int32, rows * cols // 8, "q")
        _dev(s, torch.float32, rows * G, "s")
        _dev(b, torch.float32, rows * G, "b")
        self.q, self.s, self.b, self.rows, self.cols = q, s, b, rows, cols
        self._c = _Mat(q.data_ptr(), s.data_ptr(), b.data_ptr(), rows, cols)

    @classmethod
    def from_host(cls, m: dict, device="cuda") -> "Q4Matrix":
        """From numpy arrays ``{"q": uint32[rows, cols/8], "s", "b",
        "rows", "cols"}`` (the layout above)."""
        import numpy as np
        q = torch.from_numpy(np.ascontiguousarray(m["q"]).view(np.int32)).to(device)
        s = torch.from_numpy(np.ascontiguousarray(m["s"], dtype=np.float32)).to(device)
        b = torch.from_numpy(np.ascontiguousarray(m["b"], dtype=np.float32)).to(device)
        return cls(q, s, b, int(m["rows"]), int(m["cols"]))

    @property
    def ref(self):
        return ctypes.byref(self._c)


def _opt(t, dtype, numel, what):
    return None if t is None else _dev(t, dtype, numel, what)


def q4mv(w: Q4Matrix, x: torch.Tensor, xsum: torch.Tensor | None, y: torch.Tensor | None = None,
         mode: int = FIXED, stream=None) -> torch.Tensor:
    """``y = W x`` with the activation group sums ``xsum`` (None: formed in
    the kernel); see q4mv.h."""
    if y is None:
        y = torch.empty(w.rows, dtype=torch.float32, device=x.device)
    _check("q4mv", _lib.q4mv(w.ref, _dev(x, torch.float32, w.cols, "x"),
                             _opt(xsum, torch.float32, w.cols // 64, "xsum"),
                             _dev(y, torch.float32, w.rows, "y"), mode, _stream(stream)))
    return y


def q4mv_add(w: Q4Matrix, x: torch.Tensor, xsum: torch.Tensor | None, resid: torch.Tensor,
             y: torch.Tensor | None = None, mode: int = FIXED, stream=None) -> torch.Tensor:
    """``y = resid + W x`` (``y`` may be ``resid``)."""
    if y is None:
        y = torch.empty(w.rows, dtype=torch.float32, device=x.device)
    _check("q4mv_add", _lib.q4mv_add(w.ref, _dev(x, torch.float32, w.cols, "x"),
                                     _opt(xsum, torch.float32, w.cols // 64, "xsum"),
                                     _dev(resid, torch.float32, w.rows, "resid"),
                                     _dev(y, torch.float32, w.rows, "y"), mode, _stream(stream)))
    return y


def q4mv_norm(w: Q4Matrix, h: torch.Tensor, wn: torch.Tensor, eps: float,
              y: torch.Tensor | None = None, u: torch.Tensor | None = None,
              usum: torch.Tensor | None = None, mode: int = FIXED, stream=None) -> torch.Tensor:
    """``y = W rmsq(h, wn)`` in one kernel (2048 columns); optionally also
    writes rmsq's ``u`` and ``usum``."""
    if y is None:
        y = torch.empty(w.rows, dtype=torch.float32, device=h.device)
    _check("q4mv_norm", _lib.q4mv_norm(w.ref, _dev(h, torch.float32, w.cols, "h"),
                                       _dev(wn, torch.float32, w.cols, "wn"), float(eps),
                                       _dev(y, torch.float32, w.rows, "y"),
                                       _opt(u, torch.float32, w.cols, "u"),
                                       _opt(usum, torch.float32, w.cols // 64, "usum"),
                                       mode, _stream(stream)))
    return y


def q4mv_norm_swiglu(w: Q4Matrix, h: torch.Tensor, wn: torch.Tensor, eps: float,
                     m: torch.Tensor | None = None, mode: int = FIXED,
                     stream=None) -> torch.Tensor:
    """``m = swq(W rmsq(h, wn))`` for a matrix of interleaved (gate, up)
    rows, in one kernel."""
    if m is None:
        m = torch.empty(w.rows // 2, dtype=torch.float32, device=h.device)
    _check("q4mv_norm_swiglu",
           _lib.q4mv_norm_swiglu(w.ref, _dev(h, torch.float32, w.cols, "h"),
                                 _dev(wn, torch.float32, w.cols, "wn"), float(eps),
                                 _dev(m, torch.float32, w.rows // 2, "m"), mode, _stream(stream)))
    return m


def q4mv_argmax_ws_bytes() -> int:
    return int(_lib.q4mv_argmax_ws_bytes())


def q4mv_norm_argmax(w: Q4Matrix, h: torch.Tensor, wn: torch.Tensor, eps: float,
                     y: torch.Tensor, idx: torch.Tensor, state: torch.Tensor | None = None,
                     mode: int = FIXED, stream=None) -> torch.Tensor:
    """``y = W rmsq(h, wn)`` and ``idx[0] = argmax(y)``: the product kernel
    plus one small reduction kernel; ``state`` is the key workspace
    (allocated when None)."""
    if state is None:
        state = torch.empty((q4mv_argmax_ws_bytes() + 7) // 8, dtype=torch.int64, device=h.device)
    _check("q4mv_norm_argmax",
           _lib.q4mv_norm_argmax(w.ref, _dev(h, torch.float32, w.cols, "h"),
                                 _dev(wn, torch.float32, w.cols, "wn"), float(eps),
                                 _dev(y, torch.float32, w.rows, "y"),
                                 _dev(idx, torch.int32, 1, "idx"),
                                 _dev(state, state.dtype, None, "state"),
                                 state.numel() * state.element_size(), mode, _stream(stream)))
    return idx


VARIANT_LANE_PER_ROW = 0
VARIANTS = {"lane_per_row": 0, "wave_R1": 1, "wave_R2": 2, "wave_R4": 4, "wave_R8": 8}


def q4mv_variant(w: Q4Matrix, x: torch.Tensor, xsum: torch.Tensor, y: torch.Tensor,
                 variant: int, mode: int = FIXED, stream=None) -> torch.Tensor:
    """``y = W x`` (2048 columns) by one of the kernel designs the pages
    compare: ``variant`` 0 = one lane per row, 1/2/4/8 = one wave per row
    with that many rows per block (4 is what ``q4mv`` runs)."""
    _check("q4mv_variant", _lib.q4mv_variant(w.ref, _dev(x, torch.float32, w.cols, "x"),
                                             _dev(xsum, torch.float32, w.cols // 64, "xsum"),
                                             _dev(y, torch.float32, w.rows, "y"), int(variant),
                                             mode, _stream(stream)))
    return y


def q4mv_norm_argmax_noalloc(w: Q4Matrix, h: torch.Tensor, wn: torch.Tensor, eps: float,
                             y: torch.Tensor, idx: torch.Tensor, mode: int = FIXED,
                             stream=None) -> torch.Tensor:
    """``q4mv_norm_argmax`` with the keys in the library's static device
    array instead of a caller workspace (no allocation by the call); calls
    on one GPU must not overlap in time."""
    _check("q4mv_norm_argmax_noalloc",
           _lib.q4mv_norm_argmax_noalloc(w.ref, _dev(h, torch.float32, w.cols, "h"),
                                         _dev(wn, torch.float32, w.cols, "wn"), float(eps),
                                         _dev(y, torch.float32, w.rows, "y"),
                                         _dev(idx, torch.int32, 1, "idx"), mode,
                                         _stream(stream)))
    return idx


def rmsq(h: torch.Tensor, w: torch.Tensor, eps: float, u: torch.Tensor | None = None,
         usum: torch.Tensor | None = None, stream=None):
    """RMS norm with weights plus group sums; returns ``(u, usum)``."""
    n = h.numel()
    if u is None:
        u = torch.empty(n, dtype=torch.float32, device=h.device)
    if usum is None:
        usum = torch.empty(max(n // 64, 1), dtype=torch.float32, device=h.device)
    _check("rmsq", _lib.rmsq(_dev(h, torch.float32, n, "h"), _dev(w, torch.float32, n, "w"), n,
                             float(eps), _dev(u, torch.float32, n, "u"),
                             _dev(usum, torch.float32, None, "usum"), _stream(stream)))
    return u, usum


def swq(a: torch.Tensor, n: int, o: torch.Tensor | None = None, osum: torch.Tensor | None = None,
        mode: int = FIXED, stream=None):
    """SwiGLU of ``a = [gate | up]`` plus group sums; returns ``(o, osum)``."""
    if o is None:
        o = torch.empty(n, dtype=torch.float32, device=a.device)
    if osum is None:
        osum = torch.empty(max(n // 64, 1), dtype=torch.float32, device=a.device)
    _check("swq", _lib.swq(_dev(a, torch.float32, 2 * n, "a"), n, _dev(o, torch.float32, n, "o"),
                           _dev(osum, torch.float32, None, "osum"), mode, _stream(stream)))
    return o, osum


def q4_argmax_ws_bytes(n: int) -> int:
    return int(_lib.q4_argmax_ws_bytes(n))


def q4_argmax(v: torch.Tensor, idx: torch.Tensor | None = None, ws: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Lowest index of the largest value (-1 on NaN), written on the device
    into ``idx`` (int32[1])."""
    n = v.numel()
    if idx is None:
        idx = torch.empty(1, dtype=torch.int32, device=v.device)
    if ws is None:
        ws = torch.empty((q4_argmax_ws_bytes(n) + 7) // 8, dtype=torch.int64, device=v.device)
    _check("q4_argmax", _lib.q4_argmax(_dev(v, torch.float32, n, "v"), n,
                                       _dev(idx, torch.int32, 1, "idx"),
                                       _dev(ws, ws.dtype, None, "ws"), ws.numel() * ws.element_size(),
                                       _stream(stream)))
    return idx


def q4_embed(w: Q4Matrix, tok: torch.Tensor, e: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """Dequantised row ``tok`` (device int32[1]) of ``w``."""
    if e is None:
        e = torch.empty(w.cols, dtype=torch.float32, device=tok.device)
    _check("q4_embed", _lib.q4_embed(w.ref, _dev(tok, torch.int32, 1, "tok"),
                                     _dev(e, torch.float32, w.cols, "e"), _stream(stream)))
    return e


class MlpLayer:
    """One MLP layer for ``q4_decode_layers``: ``gate_up`` (rows 2*inter,
    2048 columns, gate row i at 2i and up row i at 2i+1), ``down`` (2048
    rows, inter columns) and the norm weights ``wn`` (float32[2048])."""

    def __init__(self, gate_up: Q4Matrix, down: Q4Matrix, wn: torch.Tensor):
        _dev(wn, torch.float32, 2048, "wn")
        self.gate_up, self.down, self.wn = gate_up, down, wn
        self._c = _MlpLayer(gate_up._c, down._c, wn.data_ptr())


def q4_decode_layers_ws_bytes() -> int:
    return int(_lib.q4_decode_layers_ws_bytes())


def q4_decode_layers(emb: Q4Matrix, tok: torch.Tensor, layers: list, eps: float,
                     h: torch.Tensor, ws: torch.Tensor, mode: int = FIXED,
                     stream=None) -> torch.Tensor:
    """``h = embed(emb, tok)``, then per layer ``h += down swq(gate_up
    rmsq(h, wn))``, in one persistent kernel.  ``ws`` is its workspace of
    ``q4_decode_layers_ws_bytes()`` bytes (zero-filled before first use,
    e.g. ``torch.zeros``)."""
    if not layers:
        raise ValueError("at least one layer required")
    arr = (_MlpLayer * len(layers))(*[L._c for L in layers])
    _check("q4_decode_layers",
           _lib.q4_decode_layers(emb.ref, _dev(tok, torch.int32, 1, "tok"), arr, len(layers),
                                 float(eps), _dev(h, torch.float32, 2048, "h"),
                                 _dev(ws, ws.dtype, None, "ws"), ws.numel() * ws.element_size(),
                                 mode, _stream(stream)))
    return h


def q4_decode_token(emb: Q4Matrix, tok: torch.Tensor, layers: list, wn_final: torch.Tensor,
                    eps: float, h: torch.Tensor, logits: torch.Tensor, ws: torch.Tensor,
                    mode: int = FIXED, stream=None) -> torch.Tensor:
    """One greedy decode step in one persistent launch: ``h`` after every
    layer, ``logits = emb rmsq(h, wn_final)`` and the next token written
    over ``tok`` (device int32[1]).  ``ws`` as for ``q4_decode_layers``."""
    if not layers:
        raise ValueError("at least one layer required")
    arr = (_MlpLayer * len(layers))(*[L._c for L in layers])
    _check("q4_decode_token",
           _lib.q4_decode_token(emb.ref, _dev(tok, torch.int32, 1, "tok"), arr, len(layers),
                                _dev(wn_final, torch.float32, 2048, "wn_final"), float(eps),
                                _dev(h, torch.float32, 2048, "h"),
                                _dev(logits, torch.float32, emb.rows, "logits"),
                                _dev(ws, ws.dtype, None, "ws"), ws.numel() * ws.element_size(),
                                mode, _stream(stream)))
    return tok


def q4_decode_layers_status(ws: torch.Tensor, stream=None) -> int:
    """Host wait; Q4_OK, or Q4_ETIMEOUT when a wait of the persistent
    kernel ran out (the workspace is then cleared)."""
    return int(_lib.q4_decode_layers_status(_dev(ws, ws.dtype, None, "ws"), _stream(stream)))


def q4_atq_ws_bytes(hq: int, hkv: int) -> int:
    """Workspace bytes of ``q4_atq`` for these head counts (0: outside the
    limits)."""
    return int(_lib.q4_atq_ws_bytes(int(hq), int(hkv)))


def q4_atq(q: torch.Tensor, g: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
           wq: torch.Tensor, wk: torch.Tensor, eps: float, rope_cos: torch.Tensor,
           rope_sin: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
           pos: torch.Tensor, o: torch.Tensor, osum: torch.Tensor, ws: torch.Tensor,
           stream=None) -> torch.Tensor:
    """Gated attention of one decode token at the position held in ``pos``
    (device int32[1], read on the device): writes that row of the
    ``[hkv, max_pos, 128]`` caches and ``o`` (``hq * 128`` values) with its
    group sums ``osum`` (``hq * 2``).  ``rope_cos``/``rope_sin``: the
    ``[max_pos, 64]`` rotation tables.  ``ws``: ``q4_atq_ws_bytes(hq, hkv)``
    bytes, 256-byte aligned (any fresh torch allocation is), zero-filled
    before its first use (e.g. ``torch.zeros``) and kept for calls of one
    shape."""
    if kcache.dim() != 3 or kcache.shape[2] != ATQ_D or vcache.shape != kcache.shape:
        raise ValueError("caches must be [hkv, max_pos, 128]")
    hkv, max_pos = int(kcache.shape[0]), int(kcache.shape[1])
    hq = q.numel() // ATQ_D
    f = torch.float32
    rn = max_pos * (ATQ_D // 2)
    _check("q4_atq", _lib.q4_atq(
        _dev(q, f, hq * ATQ_D, "q"), _dev(g, f, hq * ATQ_D, "g"), _dev(k, f, hkv * ATQ_D, "k"),
        _dev(v, f, hkv * ATQ_D, "v"), _dev(wq, f, ATQ_D, "wq"), _dev(wk, f, ATQ_D, "wk"),
        float(eps), _dev(rope_cos, f, rn, "rope_cos"), _dev(rope_sin, f, rn, "rope_sin"),
        _dev(kcache, f, None, "kcache"), _dev(vcache, f, None, "vcache"),
        _dev(pos, torch.int32, 1, "pos"), max_pos, hq, hkv,
        _dev(o, f, hq * ATQ_D, "o"), _dev(osum, f, hq * 2, "osum"),
        _dev(ws, ws.dtype, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)))
    return o


def q4_atq_status(ws: torch.Tensor, hq: int, hkv: int, stream=None) -> int:
    """Host wait; Q4_OK, or Q4_ETIMEOUT when a wait of q4_atq ran out (the
    workspace is then cleared)."""
    return int(_lib.q4_atq_status(_dev(ws, ws.dtype, None, "ws"), int(hq), int(hkv),
                                  _stream(stream)))


BLOCK_MAX_POS = 4096
BLOCK_MAX_LAYERS = 32


class AttnBlock:
    """One decoder layer's weights and caches for q4_decode_block: the
    [Q; gate; K; V] and O matrices, the attention, query and key norm
    weights, the caches ``[hkv, max_pos, 128]`` and the MLP layer."""

    def __init__(self, qgkv: Q4Matrix, o: Q4Matrix, wa: torch.Tensor, wq: torch.Tensor,
                 wk: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, mlp: "MlpLayer"):
        f = torch.float32
        # the library trusts max_pos for the caches' sizes: the shapes are
        # checked here, where they are known
        if kcache.dim() != 3 or kcache.shape[2] != ATQ_D or tuple(vcache.shape) != tuple(
                kcache.shape):
            raise ValueError("kcache and vcache must both be [hkv, max_pos, %d]" % ATQ_D)
        self._keep = (qgkv, o, wa, wq, wk, kcache, vcache, mlp)
        self.kcache, self.vcache = kcache, vcache
        self._c = _AttnBlock(qgkv._c, o._c, _dev(wa, f, 2048, "wa"), _dev(wq, f, ATQ_D, "wq"),
                             _dev(wk, f, ATQ_D, "wk"), _dev(kcache, f, None, "kcache"),
                             _dev(vcache, f, None, "vcache"), int(kcache.shape[0]), mlp._c)


def q4_decode_block_ws_bytes() -> int:
    return int(_lib.q4_decode_block_ws_bytes())


def q4_decode_block(blk: AttnBlock, eps: float, h: torch.Tensor, pos: torch.Tensor,
                    rope_cos: torch.Tensor, rope_sin: torch.Tensor, ws: torch.Tensor,
                    mode: int = FIXED, stream=None) -> torch.Tensor:
    """One decoder layer (attention block and MLP block) in one persistent
    launch: ``h`` (2048 values) is read and written in place; the caches
    get row ``pos``.  ``ws``: ``q4_decode_block_ws_bytes()`` bytes,
    zero-filled before first use."""
    max_pos = int(blk.kcache.shape[1])
    f = torch.float32
    rn = max_pos * (ATQ_D // 2)
    _check("q4_decode_block", _lib.q4_decode_block(
        ctypes.byref(blk._c), float(eps), _dev(h, f, 2048, "h"), _dev(pos, torch.int32, 1, "pos"),
        max_pos, _dev(rope_cos, f, rn, "rope_cos"), _dev(rope_sin, f, rn, "rope_sin"),
        _dev(ws, ws.dtype, None, "ws"), ws.numel() * ws.element_size(), mode, _stream(stream)))
    return h


class BlockStack:
    """Decoder layers for one persistent launch (``q4_decode_blocks``): the
    layers' pointers are copied once to a table in device memory (a
    synchronous copy, so not under stream capture).  Holds references to
    the layers, whose arrays must outlive it."""

    def __init__(self, blocks: list):
        blocks = list(blocks)
        if not blocks:
            raise ValueError("no layers")
        self.blocks = blocks
        self.max_pos = int(blocks[0].kcache.shape[1])
        if any(int(b.kcache.shape[1]) != self.max_pos for b in blocks):
            raise ValueError("every layer's caches must hold the same number of positions")
        arr = (_AttnBlock * len(blocks))(*[b._c for b in blocks])
        h = _vp()
        _check("q4_block_stack_create",
               _lib.q4_block_stack_create(arr, len(blocks), self.max_pos, ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _check("q4_block_stack_destroy", _lib.q4_block_stack_destroy(self._h))
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def q4_decode_blocks(stack: BlockStack, eps: float, h: torch.Tensor, pos: torch.Tensor,
                     rope_cos: torch.Tensor, rope_sin: torch.Tensor, ws: torch.Tensor,
                     mode: int = FIXED, stream=None) -> torch.Tensor:
    """Every layer of ``stack`` in one persistent launch, with the bits of
    ``q4_decode_block`` called once per layer: ``h`` is read and written in
    place; each layer's caches get row ``pos``.  ``ws`` as for
    ``q4_decode_block``."""
    f = torch.float32
    rn = stack.max_pos * (ATQ_D // 2)
    _check("q4_decode_blocks", _lib.q4_decode_blocks(
        stack._h, float(eps), _dev(h, f, 2048, "h"), _dev(pos, torch.int32, 1, "pos"),
        _dev(rope_cos, f, rn, "rope_cos"), _dev(rope_sin, f, rn, "rope_sin"),
        _dev(ws, ws.dtype, None, "ws"), ws.numel() * ws.element_size(), mode, _stream(stream)))
    return h


def q4_decode_block_status(ws: torch.Tensor, stream=None) -> int:
    """Host wait; Q4_OK, or Q4_ETIMEOUT when a wait of q4_decode_block ran
    out (the workspace is then cleared)."""
    return int(_lib.q4_decode_block_status(_dev(ws, ws.dtype, None, "ws"), _stream(stream)))


def q4_pos_advance(pos: torch.Tensor, stream=None) -> torch.Tensor:
    """``pos += 1`` on the device (int32[1])."""
    _check("q4_pos_advance", _lib.q4_pos_advance(_dev(pos, torch.int32, 1, "pos"),
                                                 _stream(stream)))
    return pos


class Mailbox:
    """Pinned host mailbox of ``n`` int32 values: ``post`` enqueues a
    one-thread kernel that copies device values into it and publishes the
    next sequence number; ``wait`` spins on the host until the number
    reaches ``target`` (the host waits on a flag, not on the stream)."""

    def __init__(self, n: int):
        h = _vp()
        _check("q4_mailbox_create", _lib.q4_mailbox_create(int(n), ctypes.byref(h)))
        self._h = h
        self.n = int(n)
        self._buf = (ctypes.c_int32 * self.n)()

    def post(self, vals: torch.Tensor, stream=None) -> None:
        _check("q4_mailbox_post", _lib.q4_mailbox_post(self._h, _dev(vals, torch.int32, self.n,
                                                                       "vals"), _stream(stream)))

    def wait(self, target: int, timeout_ms: int = 2000) -> list:
        _check("q4_mailbox_wait", _lib.q4_mailbox_wait(self._h, int(target) & 0xFFFFFFFF,
                                                       ctypes.byref(self._buf), int(timeout_ms)))
        return list(self._buf)

    @property
    def seq(self) -> int:
        return int(_lib.q4_mailbox_seq(self._h))

    def close(self) -> None:
        if self._h:
            _lib.q4_mailbox_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def q4_sync(stream=None) -> None:
    _check("q4_sync", _lib.q4_sync(_stream(stream)))


class Queue:
    """Stage queue over one stream: ``q4mv_queue`` adds a product to the open
    stage, ``q4_stage`` closes it (grouped launches, no host wait),
    ``q4mv_wait`` closes it and waits once.  The queue holds a reference to
    every tensor it was given until ``q4mv_wait`` returns."""

    def __init__(self, mode: int = FIXED, stream=None):
        self._stream = _stream(stream)
        self._h = ctypes.c_void_p()
        _check("q4_queue_create", _lib.q4_queue_create(self._stream, mode, ctypes.byref(self._h)))
        self._keep = []

    def q4mv_queue(self, w: Q4Matrix, x: torch.Tensor, xsum: torch.Tensor, y: torch.Tensor) -> None:
        _check("q4mv_queue", _lib.q4mv_queue(self._h, w.ref, _dev(x, torch.float32, w.cols, "x"),
                                             _dev(xsum, torch.float32, w.cols // 64, "xsum"),
                                             _dev(y, torch.float32, w.rows, "y")))
        self._keep.append((w, x, xsum, y))

    def q4_stage(self) -> None:
        _check("q4_stage", _lib.q4_stage(self._h))

    def set_wait(self, how: int, timeout_ms: int = 10000) -> None:
        """WAIT_STREAM (hipStreamSynchronize) or WAIT_MAILBOX (spin on a
        pinned flag that a one-thread kernel sets after the last stage)."""
        _check("q4_queue_set_wait", _lib.q4_queue_set_wait(self._h, int(how), int(timeout_ms)))

    def q4mv_wait(self) -> None:
        _check("q4mv_wait", _lib.q4mv_wait(self._h))
        self._keep.clear()

    def close(self) -> None:
        if self._h:
            _check("q4_queue_destroy", _lib.q4_queue_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """Records every library call issued on ``stream`` between ``begin`` and
    ``end`` and replays it with ``launch``.  Keep the tensors the recorded
    calls use alive (and at the same addresses) for the graph's lifetime."""

    def __init__(self, stream: torch.cuda.Stream):
        if not isinstance(stream, torch.cuda.Stream):
            raise ValueError("capture needs a torch.cuda.Stream (not the null stream)")
        self.stream = stream
        self._h = ctypes.c_void_p()
        self.keep = []

    def begin(self) -> None:
        _check("q4_capture_begin", _lib.q4_capture_begin(self.stream.cuda_stream))

    def end(self) -> None:
        _check("q4_capture_end", _lib.q4_capture_end(self.stream.cuda_stream, ctypes.byref(self._h)))

    def launch(self, stream=None) -> None:
        _check("q4_graph_launch", _lib.q4_graph_launch(self._h, _stream(stream or self.stream)))

    def close(self) -> None:
        if self._h:
            _check("q4_graph_destroy", _lib.q4_graph_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
