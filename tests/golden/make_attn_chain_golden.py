"""Writes the golden file of the decode chain with attention from the CPU
oracle.

The 24-layer chain with an attention block in every layer (hidden 2048,
16 query and 4 key/value heads of 128, SwiGLU width 6144, vocab 248320,
eps 1e-6, rotation tables of 256 positions, seeded synthetic weights) is
run for N greedy steps from its seeded start token at positions 0, 1, ...
with caches that start empty.  For every step the file stores the chosen
token and the FNV-1a-32 hash of the binary32 logits' bytes.  Only oracle/
and synth/ are used.

    python tests/golden/make_attn_chain_golden.py [--seed S] [--steps N] [--threads T]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=synth.DEFAULT_SEED)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--threads", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    out = args.out or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                   "attn_chain_seed%d.json" % args.seed)
    w = synth.attn_chain_weights(seed=args.seed)
    kc, vc = oracle.attn_caches(w)
    tok = w["tok0"]
    rec = {"seed": args.seed, "layers": len(w["layers"]), "hidden": w["hidden"],
           "inter": w["inter"], "vocab": w["vocab"], "hq": w["hq"], "hkv": w["hkv"],
           "max_pos": w["max_pos"], "eps": float(w["eps"]), "tok0": tok, "pos0": 0,
           "tokens": [], "logits_fnv1a32": []}
    t0 = time.time()
    for i in range(args.steps):
        logits, tok = oracle.attn_chain_step(w, tok, i, kc, vc, nthreads=args.threads)
        rec["tokens"].append(int(tok))
        rec["logits_fnv1a32"].append(oracle.fnv1a32(logits))
        print("step %d token %d (%.1f s)" % (i, tok, time.time() - t0), flush=True)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
