"""Builds libq4mv.so (HIP, gfx950) in-tree with hipcc.

Flags:
  -ffp-contract=off          no implicit fused multiply-add: the fixed-order
                             kernels must perform exactly the IEEE operations
                             they spell
  -packed-fp32-ops disabled  (target feature) no packed-fp32 VALU forms
  -fPIC -shared              a C-ABI shared library
  -mllvm -disable-machine-licm
                             (decode_block.hip only) its loop over layers runs
                             whole stages per iteration: constants hoisted out
                             of it (the binary64 exp's coefficients) would be
                             held, or spilled, through every stage

Each source is compiled to an object of its own (in parallel), then linked.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4mv.so")
SOURCES = ["q4mv_kernels.hip", "producers.hip", "decode_layers.hip", "decode_block.hip", "atq.hip",
           "q4mv_api.hip"]
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
EXTRA_FLAGS = {"decode_block.hip": ["-mllvm", "-disable-machine-licm"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l
            and "is not a recognized feature" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False, out: str = LIB, defines=(), extra_flags=()) -> str:
    """Compile every source into affine_q4_matvec_amd/libq4mv.so (or `out`;
    `defines` are extra -D tunables, `extra_flags` extra compile and link
    flags, e.g. host-only sanitizers for a test build)."""
    defs = ["-D" + d for d in defines] + list(extra_flags)
    with tempfile.TemporaryDirectory(prefix="q4mv_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[hipcc(), *FLAGS, *EXTRA_FLAGS.get(s, []), *defs, "-c", "-o", o,
                 os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp%d" % os.getpid()
        _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *extra_flags, "-o", tmp, *objs],
             verbose)
    os.replace(tmp, out)
    return out


def asm(out_path: str, source: str = "q4mv_kernels.hip") -> str:
    """Writes the gfx950 assembly of one source (for inspection)."""
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(source, []), "--cuda-device-only", "-S", "-o",
           out_path, os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
