"""Record the Zipf temperature of the 8192-token prefill chunk's router bias.

The workload asks for Zipf(s=1) expert popularity "so group sizes are skewed
(some experts above 2000 tokens, some at 0)".  The bias is b[e] = beta*ln(p_e)
with p_e proportional to 1/rank_e.  beta = 1 is the plain reading; when the
seed-0 chunk routed by the oracle has no empty expert at beta = 1, beta is
raised in steps of 0.05 until it has one.  The routing is the oracle's (fp64),
so the recorded value depends only on the oracle and the seeded inputs.

Writes tests/golden/zipf_beta.json; synth.ZIPF_BETA must equal its "beta".
Run:  python tests/golden/make_zipf_beta.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def histogram(beta: float, seed: int = 0):
    sh = synth.CONFIGS["c3_prefill8192_bf16"]
    x = synth.make_x(sh, seed)
    wr = synth._store(synth.normal(seed, "wr", (sh.E, sh.H), 0.02), sh.act)
    b = synth.make_bias(sh, seed, beta=beta)
    dummy = np.zeros((sh.E, 1, sh.H), np.uint16)
    dummy_d = np.zeros((sh.E, sh.H, 1), np.uint16)
    L = oracle.Layer(x=x, wr=wr, wg=dummy, wu=dummy, wd=dummy_d, top_k=sh.K, bias=b)
    r = oracle.router(L)
    return np.bincount(r["ids"].ravel(), minlength=sh.E), int(r["near"].sum())


def main():
    beta = 1.0
    trail = []
    while True:
        h, near = histogram(beta)
        trail.append(dict(beta=round(beta, 2), max=int(h.max()), over_2000=int((h > 2000).sum()),
                          empty=int((h == 0).sum()), min=int(h.min()), near_ties=near))
        print(trail[-1], flush=True)
        if (h == 0).any() and (h > 2000).any():
            break
        beta += 0.05
        if beta > 3.0:
            raise SystemExit("no beta up to 3 gives an empty expert")
    out = dict(beta=round(beta, 2), seed=0, config="prefill T=8192, H=2048, E=128, top-8",
               histogram=[int(v) for v in h], trail=trail)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_beta.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("beta =", out["beta"], "->", path)


if __name__ == "__main__":
    main()
