"""Writes the single-product golden file from the CPU oracle.

For the four product workloads (seeded synthetic inputs, synth/):
  - the 13 x 128 product: x's group sums and every output's bits;
  - the 4096 x 2048 product: x's group sums and the FNV-1a-32 hash of the
    output's bytes;
  - the 248320 x 2048 output head fed by rmsq(z, wn): the hash of the
    output and its greedy argmax;
  - the product set of one decode step (24 layers x {Q, K, V, O, gate, up,
    down} + head): the group sums of the two activation widths and the
    hash of every product's output, in product order.
Only oracle/ and synth/ are used.

    python tests/golden/make_product_golden.py [--seed S] [--threads T]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def hexbits(a) -> list:
    return ["%08x" % v for v in np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=synth.DEFAULT_SEED)
    ap.add_argument("--threads", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    out = args.out or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                   "products_seed%d.json" % args.seed)
    t0 = time.time()
    rec = {"seed": args.seed}

    m = synth.small_product(seed=args.seed)  # 13 x 128
    xs = oracle.group_sums(m["x"])
    y = oracle.q4mv(m, m["x"], xs)
    rec["p13x128"] = {"rows": 13, "cols": 128, "xsum_bits": hexbits(xs), "y_bits": hexbits(y),
                      "y_fnv1a32": oracle.fnv1a32(y)}

    m = synth.small_product(seed=args.seed, rows=4096, cols=2048, name="p4096")
    xs = oracle.group_sums(m["x"])
    y = oracle.q4mv(m, m["x"], xs, args.threads)
    rec["p4096x2048"] = {"rows": 4096, "cols": 2048, "name": "p4096", "xsum_bits": hexbits(xs),
                         "y_fnv1a32": oracle.fnv1a32(y)}
    print("4096 x 2048 done (%.1f s)" % (time.time() - t0), flush=True)

    h = synth.head_inputs(seed=args.seed)
    u, us = oracle.rmsq(h["z"], h["wn"], h["eps"])
    y = oracle.q4mv(h, u, us, args.threads)
    rec["head"] = {"rows": int(h["rows"]), "cols": int(h["cols"]),
                   "y_fnv1a32": oracle.fnv1a32(y), "argmax": oracle.argmax(y)}
    del h, y
    print("head done (%.1f s)" % (time.time() - t0), flush=True)

    ps = synth.product_set(seed=args.seed)
    xsw = {c: oracle.group_sums(x) for c, x in ps["x"].items()}
    hashes = []
    for p in ps["products"]:
        c = p["cols"]
        hashes.append(oracle.fnv1a32(oracle.q4mv(p, ps["x"][c], xsw[c], args.threads)))
    rec["product_set"] = {"products": len(ps["products"]), "stages": ps["stages"],
                          "xsum_bits": {str(c): hexbits(v) for c, v in xsw.items()},
                          "names": [p["name"] for p in ps["products"]],
                          "y_fnv1a32": hashes}
    print("product set done (%.1f s)" % (time.time() - t0), flush=True)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
