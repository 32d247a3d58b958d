"""Writes the golden file of the decode chain with attention from the CPU
oracle.

The 24-layer chain with an attention block in every layer (hidden 2048,
16 query and 4 key/value heads of 128, SwiGLU width 6144, vocab 248320,
eps 1e-6, seeded synthetic weights, caches and rotation tables of
max_pos positions) is run for N greedy steps from its seeded start token at
positions pos0, pos0 + 1, ... with caches that start empty (all zero).
For every step the file stores the chosen token and the FNV-1a-32 hash of
the binary32 logits' bytes.  Only oracle/ and synth/ are used.

    python tests/golden/make_attn_chain_golden.py [--seed S] [--steps N] [--threads T]
        [--max-pos P] [--pos0 Q]

The default (200 steps from position 0, caches of 256) writes
attn_chain_seed<S>.json; --max-pos 4096 --pos0 3896 the end of a full
cache, attn_chain_long_seed<S>.json.
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--max-pos", type=int, default=256)
    ap.add_argument("--pos0", type=int, default=0)
    ap.add_argument("--threads", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    if args.pos0 + args.steps > args.max_pos:
        raise SystemExit("the caches hold %d positions" % args.max_pos)
    name = "attn_chain_seed%d.json" if args.pos0 == 0 else "attn_chain_long_seed%d.json"
    out = args.out or os.path.join(os.path.dirname(os.path.abspath(__file__)), name % args.seed)
    w = synth.attn_chain_weights(seed=args.seed, max_pos=args.max_pos)
    kc, vc = oracle.attn_caches(w)
    tok = w["tok0"]
    rec = {"seed": args.seed, "layers": len(w["layers"]), "hidden": w["hidden"],
           "inter": w["inter"], "vocab": w["vocab"], "hq": w["hq"], "hkv": w["hkv"],
           "max_pos": w["max_pos"], "eps": float(w["eps"]), "tok0": tok, "pos0": args.pos0,
           "tokens": [], "logits_fnv1a32": []}
    t0 = time.time()
    for i in range(args.steps):
        logits, tok = oracle.attn_chain_step(w, tok, args.pos0 + i, kc, vc,
                                             nthreads=args.threads)
        rec["tokens"].append(int(tok))
        rec["logits_fnv1a32"].append(oracle.fnv1a32(logits))
        print("step %d token %d (%.1f s)" % (i, tok, time.time() - t0), flush=True)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
