"""The C ABI without a GPU: the library loads, exports every function that
include/q4mv.h declares, and rejects bad arguments before any HIP call
(every call below returns Q4_EINVAL from the host-side checks)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4mv.h")
# Q4MV_TEST_LIB: another build of the library to check (the sanitizer test
# runs this module against a host-sanitized build)
LIB = os.environ.get("Q4MV_TEST_LIB") or os.path.join(ROOT, "affine_q4_matvec_amd", "libq4mv.so")

EINVAL = -1


class Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:int|size_t|uint32_t|const char \*)\s*\**\s*(\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail("libq4mv.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.q4_strerror.restype = ctypes.c_char_p
    lib.q4_argmax_ws_bytes.restype = ctypes.c_size_t
    return lib


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_only_the_c_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    exported = {s for s in syms if not s.startswith("__hip_cuid")}
    assert exported == set(declared_functions())


# fake, never-dereferenced device addresses (16-byte aligned, disjoint)
A = 0x7F0000000000
B = 0x7F0010000000
C = 0x7F0020000000
D = 0x7F0030000000
E = 0x7F0040000000
F = 0x7F0050000000


def mat(q=A, s=B, b=C, rows=8, cols=128):
    return Mat(q, s, b, rows, cols)


@pytest.mark.parametrize("m", [
    mat(q=0), mat(s=0), mat(b=0), mat(rows=0), mat(rows=-3), mat(cols=0), mat(cols=100),
    mat(cols=32), mat(cols=32768 + 64), mat(q=A + 4), mat(s=B + 2),
])
def test_q4mv_rejects_bad_matrix(L, m):
    assert L.q4mv(ctypes.byref(m), ctypes.c_void_p(D), ctypes.c_void_p(E), ctypes.c_void_p(F), 0, None) == EINVAL


def test_q4mv_rejects_bad_vectors_and_mode(L):
    m = mat()
    p = lambda v: ctypes.c_void_p(v)
    assert L.q4mv(None, p(D), p(E), p(F), 0, None) == EINVAL
    assert L.q4mv(ctypes.byref(m), None, p(E), p(F), 0, None) == EINVAL
    assert L.q4mv(ctypes.byref(m), p(D + 4), p(E), p(F), 0, None) == EINVAL  # x not 16-B aligned
    assert L.q4mv(ctypes.byref(m), p(D), p(E), p(F), 2, None) == EINVAL      # mode
    assert L.q4mv(ctypes.byref(m), p(D), p(E), p(D + 64), 0, None) == EINVAL  # y overlaps x
    assert L.q4mv(ctypes.byref(m), p(D), p(E), p(A + 16), 0, None) == EINVAL  # y overlaps q
    # residual that partly overlaps y
    assert L.q4mv_add(ctypes.byref(m), p(D), p(E), p(F + 4), p(F), 0, None) == EINVAL


def test_producers_reject_bad_sizes(L):
    p = lambda v: ctypes.c_void_p(v)
    assert L.rmsq(p(A), p(B), 100, ctypes.c_float(1e-6), p(C), p(D), None) == EINVAL
    assert L.rmsq(p(A), p(B), 8192 + 64, ctypes.c_float(1e-6), p(C), p(D), None) == EINVAL
    assert L.rmsq(p(A), p(B), 2048, ctypes.c_float(1e-6), p(A + 64), p(D), None) == EINVAL
    assert L.swq(p(A), 32, p(B), p(C), 0, None) == EINVAL  # n = 32 is an error
    assert L.swq(p(A), 6144, p(A + 4), p(C), 0, None) == EINVAL  # o inside a
    assert L.swq(p(A), 6144, p(B), p(C), 5, None) == EINVAL


def test_argmax_and_embed_checks(L):
    p = lambda v: ctypes.c_void_p(v)
    need = L.q4_argmax_ws_bytes(248320)
    assert 8 <= need <= 8 * 1024 and L.q4_argmax_ws_bytes(0) == 0
    assert L.q4_argmax(p(A), 248320, p(B), p(C), need - 8, None) == EINVAL
    assert L.q4_argmax(p(A), 0, p(B), p(C), need, None) == EINVAL
    assert L.q4_argmax(p(A), 248320, p(B), p(C + 4), need, None) == EINVAL
    m = mat()
    assert L.q4_embed(ctypes.byref(m), None, p(D), None) == EINVAL
    assert L.q4_embed(ctypes.byref(mat(cols=96)), p(E), p(D), None) == EINVAL


def test_queue_and_graph_argument_checks(L):
    assert L.q4_queue_create(None, 0, None) == EINVAL
    out = ctypes.c_void_p()
    assert L.q4_queue_create(None, 3, ctypes.byref(out)) == EINVAL
    assert L.q4mv_queue(None, None, None, None, None) == EINVAL
    assert L.q4_stage(None) == EINVAL and L.q4mv_wait(None) == EINVAL
    assert L.q4_queue_destroy(None) == EINVAL
    assert L.q4_capture_begin(None) == EINVAL
    assert L.q4_capture_end(None, ctypes.byref(out)) == EINVAL
    assert L.q4_graph_launch(None, None) == EINVAL and L.q4_graph_destroy(None) == EINVAL


def test_strerror(L):
    assert L.q4_strerror(0) == b"ok"
    assert b"invalid" in L.q4_strerror(-1)
    assert L.q4_strerror(12345) == b"unknown status"


class MlpLayer(ctypes.Structure):
    _fields_ = [("gate_up", Mat), ("down", Mat), ("wn", ctypes.c_void_p)]


def test_decode_layers_argument_checks(L):
    p = lambda v: ctypes.c_void_p(v)
    L.q4_decode_layers_ws_bytes.restype = ctypes.c_size_t
    wsb = L.q4_decode_layers_ws_bytes()
    assert 16 * 1024 <= wsb <= 4 * 1024 * 1024
    G = 0x7F1000000000  # a further disjoint region for the layer arrays
    emb = mat(rows=4096, cols=2048)

    def layers(n=2, inter=6144):
        arr = (MlpLayer * n)()
        for i in range(n):
            base = G + i * 0x100000000
            arr[i].gate_up = Mat(base, base + 0x10000000, base + 0x20000000, 2 * inter, 2048)
            arr[i].down = Mat(base + 0x30000000, base + 0x40000000, base + 0x50000000, 2048, inter)
            arr[i].wn = base + 0x60000000
        return arr

    def call(e=emb, tok=D, arr=None, n=2, h=E, ws=F, wsb=wsb, mode=0):
        arr = layers(n) if arr is None else arr
        return L.q4_decode_layers(ctypes.byref(e), p(tok), arr, n, ctypes.c_float(1e-6), p(h),
                                  p(ws), ctypes.c_size_t(wsb), mode, None)

    assert call(n=0) == EINVAL
    assert call(n=33, arr=layers(33)) == EINVAL
    assert call(e=mat(rows=4096, cols=1024)) == EINVAL          # embedding width
    assert call(arr=layers(2, inter=3000)) == EINVAL            # inter not a multiple of 2048
    assert call(arr=layers(2, inter=10240)) == EINVAL           # inter too wide
    bad = layers(2)
    bad[1].down = Mat(G + 0x130000000, G + 0x140000000, G + 0x150000000, 2048, 4096)
    assert call(arr=bad) == EINVAL                              # inter differs between layers
    bad = layers(2)
    bad[0].gate_up = Mat(G, G + 0x10000000, G + 0x20000000, 6144, 2048)
    assert call(arr=bad) == EINVAL                              # gate_up rows != 2 inter
    bad = layers(2)
    bad[1].wn = 0
    assert call(arr=bad) == EINVAL                              # no norm weights
    assert call(h=E + 2) == EINVAL                              # h misaligned
    assert call(h=F + 1024) == EINVAL                           # h inside ws
    assert call(ws=F + 8) == EINVAL                             # ws misaligned
    assert call(wsb=wsb - 8) == EINVAL                          # ws too small
    assert call(tok=0) == EINVAL
    assert call(mode=2) == EINVAL
    assert call(h=G + 0x30000000 + 64) == EINVAL                # h inside a down matrix
    assert call(ws=G + 0x60000000 - 64) == EINVAL               # ws over the norm weights
    assert L.q4_decode_layers_status(None, None) == EINVAL


def test_mailbox_argument_checks(L):
    out = ctypes.c_void_p()
    assert L.q4_mailbox_create(0, ctypes.byref(out)) == EINVAL
    assert L.q4_mailbox_create(1025, ctypes.byref(out)) == EINVAL
    assert L.q4_mailbox_create(4, None) == EINVAL
    assert L.q4_mailbox_destroy(None) == EINVAL
    assert L.q4_mailbox_post(None, ctypes.c_void_p(A), None) == EINVAL
    assert L.q4_mailbox_wait(None, 1, None, 10) == EINVAL
    L.q4_mailbox_seq.restype = ctypes.c_uint32
    assert L.q4_mailbox_seq(None) == 0


def test_queue_set_wait_checks(L):
    assert L.q4_queue_set_wait(None, 0, 10) == EINVAL


def test_atq_argument_checks(L):
    L.q4_atq_ws_bytes.restype = ctypes.c_size_t
    assert L.q4_atq_ws_bytes(16, 4) > 16 * 4096 * 4
    for hq, hkv in ((0, 1), (16, 0), (16, 3), (18, 2), (256, 32), (129, 129)):
        assert L.q4_atq_ws_bytes(hq, hkv) == 0, (hq, hkv)
    wsb = L.q4_atq_ws_bytes(16, 4)
    H = 0x7F0100000000
    f = ctypes.c_float
    base = dict(q=A, g=B, k=C, v=C + 0x100000, wq=C + 0x200000, wk=C + 0x300000,
                cs=C + 0x400000, sn=C + 0x500000, kc=D, vc=E, pos=C + 0x600000, max_pos=4096, hq=16,
                hkv=4, o=F, os=F + 0x100000, ws=H, wsb=wsb)

    def call(**kw):
        a = dict(base, **kw)
        p = ctypes.c_void_p
        return L.q4_atq(p(a["q"]), p(a["g"]), p(a["k"]), p(a["v"]), p(a["wq"]), p(a["wk"]),
                        f(1e-6), p(a["cs"]), p(a["sn"]), p(a["kc"]), p(a["vc"]), p(a["pos"]),
                        a["max_pos"], a["hq"], a["hkv"], p(a["o"]), p(a["os"]), p(a["ws"]),
                        ctypes.c_size_t(a["wsb"]), None)

    assert call(pos=0) == EINVAL                    # no position
    assert call(pos=C + 0x600002) == EINVAL         # position misaligned
    assert call(max_pos=4097) == EINVAL             # cache longer than the limit
    assert call(max_pos=0) == EINVAL
    assert call(o=C + 0x600000) == EINVAL           # o over the position
    assert call(o=C + 0x500000 + 4096 * 256 - 4) == EINVAL   # o over the end of the sin table
    assert call(hq=16, hkv=3) == EINVAL             # heads not in groups
    assert call(hq=32, hkv=2) == EINVAL             # 16 queries per key/value head
    assert call(q=0) == EINVAL
    assert call(q=A + 4) == EINVAL                  # q misaligned
    assert call(kc=D + 8) == EINVAL                 # cache misaligned
    assert call(ws=H + 16) == EINVAL                # workspace misaligned
    assert call(wsb=wsb - 4) == EINVAL              # workspace too small
    assert call(vc=D + 4096 * 512) == EINVAL        # value cache inside the key cache
    assert call(o=A + 512) == EINVAL                # o over q
    assert call(ws=D) == EINVAL                     # workspace over the key cache
    assert call(os=C + 0x400000) == EINVAL          # osum over the rotation table
    assert L.q4_atq_status(None, 16, 4, None) == EINVAL
    assert L.q4_pos_advance(None, None) == EINVAL
    assert L.q4_pos_advance(ctypes.c_void_p(A + 2), None) == EINVAL
    assert L.q4_atq_status(ctypes.c_void_p(H), 16, 3, None) == EINVAL
    assert L.q4_atq_status(ctypes.c_void_p(H + 16), 16, 4, None) == EINVAL


class AttnBlock(ctypes.Structure):
    _fields_ = [("qgkv", Mat), ("o", Mat), ("wa", ctypes.c_void_p), ("wq", ctypes.c_void_p),
                ("wk", ctypes.c_void_p), ("kcache", ctypes.c_void_p), ("vcache", ctypes.c_void_p),
                ("hkv", ctypes.c_int32), ("mlp", MlpLayer)]


def test_decode_block_argument_checks(L):
    L.q4_decode_block_ws_bytes.restype = ctypes.c_size_t
    wsb = L.q4_decode_block_ws_bytes()
    assert 256 * 1024 <= wsb <= 4 * 1024 * 1024
    G = 0x7F2000000000
    slot = lambda i: G + i * 0x10000000  # disjoint 256 MiB regions
    base = dict(hkv=4, qrows=(32 + 8) * 128, qcols=2048, orows=2048, inter=6144, gu_rows=12288,
                wa=slot(9), wq=slot(10), wk=slot(11), kc=slot(12), vc=slot(13), wn=slot(14),
                h=slot(15), pos=slot(16), max_pos=256, cs=slot(17), sn=slot(18), ws=slot(19),
                wsb=wsb, mode=0)

    def block(a):
        b = AttnBlock()
        b.qgkv = Mat(slot(0), slot(1), slot(2), a["qrows"], a["qcols"])
        b.o = Mat(slot(3), slot(4), slot(5), a["orows"], 2048)
        b.wa, b.wq, b.wk = a["wa"], a["wq"], a["wk"]
        b.kcache, b.vcache, b.hkv = a["kc"], a["vc"], a["hkv"]
        b.mlp.gate_up = Mat(slot(6), slot(6) + 0x8000000, slot(7), a["gu_rows"], 2048)
        b.mlp.down = Mat(slot(8), slot(8) + 0x8000000, slot(7) + 0x8000000, 2048, a["inter"])
        b.mlp.wn = a["wn"]
        return b

    def call(blk=True, **kw):
        a = dict(base, **kw)
        p = ctypes.c_void_p
        b = ctypes.byref(block(a)) if blk else None
        return L.q4_decode_block(b, ctypes.c_float(1e-6), p(a["h"]), p(a["pos"]), a["max_pos"],
                                 p(a["cs"]), p(a["sn"]), p(a["ws"]), ctypes.c_size_t(a["wsb"]),
                                 a["mode"], None)

    import torch
    if torch.cuda.device_count() == 0:
        # the unchanged arguments pass every check and fail at the first HIP
        # call, so each rejection below comes from the change it makes
        assert call() not in (EINVAL, 0)
    assert call(mode=2) == EINVAL
    assert call(blk=False) == EINVAL
    for hkv in (0, 3, 32):
        assert call(hkv=hkv) == EINVAL, hkv
    assert call(hkv=2) == EINVAL                        # [Q; gate; K; V] rows are those of 4
    assert call(qcols=1024) == EINVAL
    assert call(orows=4096) == EINVAL
    assert call(inter=3000, gu_rows=6000) == EINVAL     # not a multiple of 2048
    assert call(inter=10240, gu_rows=20480) == EINVAL   # wider than the limit
    assert call(gu_rows=6144) == EINVAL                 # gate/up rows != 2 inter
    assert call(wa=0) == EINVAL
    assert call(wq=slot(10) + 4) == EINVAL              # norm weights misaligned
    assert call(kc=slot(12) + 8) == EINVAL              # cache misaligned
    assert call(h=slot(15) + 4) == EINVAL
    assert call(pos=0) == EINVAL
    assert call(pos=slot(16) + 2) == EINVAL
    assert call(max_pos=0) == EINVAL
    assert call(max_pos=4097) == EINVAL                 # longer than 16 spans
    assert call(cs=0) == EINVAL
    assert call(ws=slot(19) + 8) == EINVAL
    assert call(wsb=wsb - 16) == EINVAL
    assert call(vc=slot(12) + 4096) == EINVAL           # value cache inside the key cache
    assert call(h=slot(19) + 1024) == EINVAL            # h inside the workspace
    assert call(kc=slot(17) + 64) == EINVAL             # key cache over the cos table
    assert call(ws=slot(3) + 4096) == EINVAL            # workspace over the O codes
    assert call(h=slot(8) + 64) == EINVAL               # h inside the down codes
    assert call(pos=slot(15) + 64) == EINVAL            # position inside h
    assert L.q4_decode_block_status(None, None) == EINVAL
    assert L.q4_decode_block_status(ctypes.c_void_p(slot(19) + 4), None) == EINVAL


def test_block_stack_argument_checks(L):
    """q4_block_stack_create rejects bad layer sets before any HIP call."""
    G = 0x7F3000000000
    slot = lambda i: G + i * 0x10000000

    def block(base, hkv=4, inter=6144, kc=None, vc=None):
        b = AttnBlock()
        b.qgkv = Mat(slot(base), slot(base + 1), slot(base + 2), (32 + 2 * hkv) * 128, 2048)
        b.o = Mat(slot(base + 3), slot(base + 4), slot(base + 5), 2048, 2048)
        b.wa, b.wq, b.wk = slot(base + 6), slot(base + 7), slot(base + 8)
        b.kcache = slot(base + 9) if kc is None else kc
        b.vcache = slot(base + 10) if vc is None else vc
        b.hkv = hkv
        b.mlp.gate_up = Mat(slot(base + 11), slot(base + 12), slot(base + 13), 2 * inter, 2048)
        b.mlp.down = Mat(slot(base + 14), slot(base + 15), slot(base + 16), 2048, inter)
        b.mlp.wn = slot(base + 17)
        return b

    def create(blocks, n=None, max_pos=256):
        arr = (AttnBlock * len(blocks))(*blocks)
        out = ctypes.c_void_p()
        return L.q4_block_stack_create(arr, len(blocks) if n is None else n, max_pos,
                                       ctypes.byref(out))

    two = lambda **kw: [block(0), block(20, **kw)]
    import torch
    if torch.cuda.device_count() == 0:
        # a valid set passes every check and fails at the first HIP call
        assert create(two()) not in (EINVAL, 0)
    assert create(two(), n=0) == EINVAL
    assert create([block(20 * i) for i in range(33)]) == EINVAL      # more than 32 layers
    assert create(two(hkv=2)) == EINVAL                               # hkv differs
    assert create(two(inter=4096)) == EINVAL                          # inter differs
    assert create(two(kc=slot(9) + 4096)) == EINVAL                   # caches of two layers overlap
    assert create(two(vc=slot(3))) == EINVAL                          # a cache over layer 0's O codes
    assert create(two(), max_pos=0) == EINVAL
    assert create(two(), max_pos=4097) == EINVAL
    assert create([block(0, hkv=3)]) == EINVAL
    assert L.q4_block_stack_create(None, 1, 16, ctypes.byref(ctypes.c_void_p())) == EINVAL
    arr = (AttnBlock * 1)(block(0))
    assert L.q4_block_stack_create(arr, 1, 16, None) == EINVAL
    assert L.q4_block_stack_destroy(None) == EINVAL
    f = ctypes.c_float(1e-6)
    p = ctypes.c_void_p
    assert L.q4_decode_blocks(None, f, p(A), p(B), p(C), p(D), p(E), ctypes.c_size_t(1 << 21), 0,
                              None) == EINVAL



def test_block_wrapper_checks_cache_shapes():
    """AttnBlock checks what the C ABI takes on trust (the caches' shape
    against max_pos) before touching anything else."""
    import torch
    import affine_q4_matvec_amd as q4
    with pytest.raises(ValueError):
        q4.AttnBlock(None, None, None, None, None, torch.zeros(4, 16, 64), torch.zeros(4, 16, 64),
                     None)
    with pytest.raises(ValueError):
        q4.AttnBlock(None, None, None, None, None, torch.zeros(4, 16, 128), torch.zeros(4, 8, 128),
                     None)


def test_q4mv_variant_rejects_bad_arguments(L):
    p = lambda v: ctypes.c_void_p(v)
    m = mat(cols=2048)
    assert L.q4mv_variant(ctypes.byref(m), p(D), p(E), p(F), 3, 0, None) == EINVAL   # no such variant
    assert L.q4mv_variant(ctypes.byref(m), p(D), None, p(F), 4, 0, None) == EINVAL   # xsum required
    assert L.q4mv_variant(ctypes.byref(m), p(D), p(E), p(F), 4, 2, None) == EINVAL   # mode
    m1 = mat(cols=1024)
    assert L.q4mv_variant(ctypes.byref(m1), p(D), p(E), p(F), 0, 0, None) == EINVAL  # 2048 columns only
    assert L.q4mv_variant(ctypes.byref(m), p(D), p(E), p(D + 64), 4, 0, None) == EINVAL  # y overlaps x


def test_q4mv_norm_argmax_noalloc_rejects_bad_arguments(L):
    p = lambda v: ctypes.c_void_p(v)
    m = mat(cols=2048)
    f = ctypes.c_float(1e-6)
    assert L.q4mv_norm_argmax_noalloc(ctypes.byref(m), p(D), p(E), f, p(F), None, 0, None) == EINVAL
    assert L.q4mv_norm_argmax_noalloc(ctypes.byref(m), p(D + 4), p(E), f, p(F), p(F + 8192), 0,
                                      None) == EINVAL  # h not 16-byte aligned
    assert L.q4mv_norm_argmax_noalloc(ctypes.byref(mat(cols=1024)), p(D), p(E), f, p(F),
                                      p(F + 8192), 0, None) == EINVAL
    assert L.q4mv_norm_argmax_noalloc(ctypes.byref(m), p(D), p(E), f, p(F), p(F + 8192), 5,
                                      None) == EINVAL  # mode
