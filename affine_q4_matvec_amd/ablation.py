"""Rows-per-wave ablation of the q4mv kernel for rows of 2048 columns.

A wave of the row64 kernel keeps one row's worth of activations in its
registers and sums R rows per block ("Metal: queued rmsq, swq, gdn and atq
kernels and a 4-row q4mv, so a decode token is one command buffer with one
wait" (#1440), Change, q4mv bullet: 4 rows per SIMD group, with 2 and 8 no
better).  R is a build-time constant (Q4_ROW64_R), so the ablation builds
the library once per R and times each build's q4mv on the 248320 x 2048
head in fixed and fast mode, the bench's way: two weight copies alternate,
K launches back to back between one pair of HIP events, best of three
interleaved rounds; each build's output is checked against the default
build's bits.

    python -m affine_q4_matvec_amd.ablation build [--dir D] [--rows 1,2,4,8]
    python -m affine_q4_matvec_amd.ablation run   [--dir D] [--steps K]

`build` needs hipcc (no GPU); `run` needs the GPU and the built libraries.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DEFAULT_DIR = os.path.join(ROOT, "_build", "ablation")
ROWS, COLS = 248320, 2048


def lib_path(d: str, r: int) -> str:
    return os.path.join(d, "libq4mv_R%d.so" % r)


def do_build(d: str, rows: list) -> None:
    sys.path.insert(0, HERE)
    import build as b  # the package's build script (no torch needed)
    os.makedirs(d, exist_ok=True)
    for r in rows:
        out = b.build(out=lib_path(d, r), defines=["Q4_ROW64_R=%d" % r])
        print("built", out, flush=True)


class _Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


def do_run(d: str, steps: int, seed: int) -> dict:
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import synth

    libs = {}
    for name in sorted(os.listdir(d)):
        if name.startswith("libq4mv_R") and name.endswith(".so"):
            r = int(name[len("libq4mv_R"):-3])
            lib = ctypes.CDLL(os.path.join(d, name))
            lib.q4mv.argtypes = [ctypes.POINTER(_Mat), ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            lib.rmsq.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            libs[r] = lib
    if not libs:
        raise SystemExit("no libraries in %s: run the build step first" % d)
    torch.cuda.set_device(0)
    st = torch.cuda.current_stream()
    h = synth.head_inputs(seed=seed)
    q0 = torch.from_numpy(np.ascontiguousarray(h["q"]).view(np.int32)).cuda()
    s0 = torch.from_numpy(np.ascontiguousarray(h["s"], dtype=np.float32)).cuda()
    b0 = torch.from_numpy(np.ascontiguousarray(h["b"], dtype=np.float32)).cuda()
    copies = [(q0, s0, b0), (q0.clone(), s0.clone(), b0.clone())]
    mats = [_Mat(q.data_ptr(), s.data_ptr(), b.data_ptr(), ROWS, COLS) for q, s, b in copies]
    z = torch.from_numpy(h["z"]).cuda()
    wn = torch.from_numpy(h["wn"]).cuda()
    x = torch.empty(COLS, device="cuda")
    xs = torch.empty(COLS // 64, device="cuda")
    y = torch.empty(ROWS, device="cuda")
    first = libs[min(libs)]
    rc = first.rmsq(z.data_ptr(), wn.data_ptr(), COLS, float(h["eps"]), x.data_ptr(),
                    xs.data_ptr(), st.cuda_stream)
    assert rc == 0, rc

    def launch(lib, mode, n):
        for i in range(n):
            rc = lib.q4mv(ctypes.byref(mats[i % 2]), x.data_ptr(), xs.data_ptr(), y.data_ptr(),
                          mode, st.cuda_stream)
            assert rc == 0, rc

    ref = {}
    for mode in (0, 1):
        launch(libs[4] if 4 in libs else first, mode, 1)
        torch.cuda.synchronize()
        ref[mode] = y.cpu().numpy().view(np.uint32).copy()
    times = {}
    for rnd in range(3):
        for r, lib in sorted(libs.items()):
            for mode in (0, 1):
                launch(lib, mode, 4)
                a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                launch(lib, mode, steps)
                e.record(st)
                torch.cuda.synchronize()
                times.setdefault((r, mode), []).append(a.elapsed_time(e) / steps * 1e3)
                same = bool(np.array_equal(y.cpu().numpy().view(np.uint32), ref[mode]))
                if not same:
                    raise SystemExit("R=%d mode %d: output bits differ from the default build"
                                     % (r, mode))
    hb = ROWS * (COLS // 2 + 8 * (COLS // 64) + 4) + 4 * COLS + 4 * (COLS // 64)
    out = {"workload": "q4mv 248320x2048 head, x from rmsq", "algorithmic_bytes": hb,
           "steps": steps, "rows_per_block": {}}
    for (r, mode), v in sorted(times.items()):
        best = min(v)
        out["rows_per_block"].setdefault(str(r), {})["fast" if mode else "fixed"] = {
            "us_rounds": [round(t, 2) for t in v], "us_best": round(best, 2),
            "GBps": round(hb / best / 1e3, 1), "pct_of_8TBps": round(hb / best / 1e3 / 80, 1)}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("what", choices=["build", "run"])
    ap.add_argument("--dir", default=DEFAULT_DIR)
    ap.add_argument("--rows", default="1,2,4,8")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--seed", type=int, default=20261202)
    args = ap.parse_args()
    if args.what == "build":
        do_build(args.dir, [int(v) for v in args.rows.split(",")])
        return 0
    print(json.dumps(do_run(args.dir, args.steps, args.seed)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
