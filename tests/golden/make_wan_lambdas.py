"""Choose the thresholds of the Wan-like sweep from the CPU oracle.

The Wan-like workload (B=1, H=40, S=32760, 21 x 30 x 52 grid, seed 2) is
run at lambda giving skipped-tile fractions of about 0.5, 0.75 and 0.9.  This
script finds those lambdas with the oracle only:

  * fractions reachable with lambda <= 1: from the closed-form prefix-maximum
    margins (oracle.prefix_max_margins_head) of a seeded sample of query
    blocks (16 per head, all 40 heads), inverted by
    oracle.lambda_for_skip_fraction;
  * larger fractions need lambda > 1, where decisions cascade: bisection on
    ln(lambda) with the recurrence itself (oracle.skip_head) on a smaller
    seeded sample (4 query blocks per head, 8 heads).

It writes tests/golden/wan_lambdas.json.  Run: python tests/golden/make_wan_lambdas.py
"""
from __future__ import annotations

import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from skip_softmax_flashattention_amd import inputs  # noqa: E402

S = 32760
TARGETS = (0.5, 0.75, 0.9)


def main():
    t0 = time.time()
    w = inputs.wan()
    q = w.q[0]
    k = w.k[0]
    v = w.v[0]
    H = q.shape[0]
    nqb = -(-S // oracle.BLOCK_Q)
    rng = np.random.default_rng(1234)
    margins = []
    for h in range(H):
        qbs = np.sort(rng.choice(nqb, 16, replace=False))
        margins.append(oracle.prefix_max_margins_head(oracle.from_bf16(q[h]), oracle.from_bf16(k[h]), w.scale, qblocks=qbs))
    margins = np.concatenate(margins)
    out = {"workload": "wan-like B=1 H=40 S=32760 D=128 grid 21x30x52 seed 2", "S": S,
           "sample_closed_form": "16 seeded query blocks per head x 40 heads (seed 1234)",
           "lambda": {}, "estimated_fraction": {}, "method": {}}
    for f in TARGETS:
        try:
            lam = oracle.lambda_for_skip_fraction(margins, f)
            est = float((margins < np.float32(math.log(lam))).mean())
            out["lambda"][str(f)] = lam
            out["estimated_fraction"][str(f)] = est
            out["method"][str(f)] = "closed form (lambda <= 1)"
            print(f"target {f}: lambda {lam:.6g} (closed form, sample fraction {est:.4f})", flush=True)
        except ValueError:
            lam, est = bisect_above_one(w, f, rng)
            out["lambda"][str(f)] = lam
            out["estimated_fraction"][str(f)] = est
            out["method"][str(f)] = "bisection on the recurrence, 4 query blocks x 8 heads (lambda > 1)"
            print(f"target {f}: lambda {lam:.6g} (recurrence, sample fraction {est:.4f})", flush=True)
    out["seconds"] = round(time.time() - t0, 1)
    with open(os.path.join(HERE, "wan_lambdas.json"), "w") as fh:
        json.dump(out, fh, indent=2)
        fh.write("\n")


def bisect_above_one(w, target, rng):
    heads = np.sort(rng.choice(w.q.shape[1], 8, replace=False))
    nqb = -(-S // oracle.BLOCK_Q)
    units = [(h, np.sort(rng.choice(nqb, 4, replace=False))) for h in heads]
    data = [(oracle.from_bf16(w.q[0, h]), oracle.from_bf16(w.k[0, h]), oracle.from_bf16(w.v[0, h]), qbs)
            for h, qbs in units]

    def frac(ln_lam):
        tot = sk = 0
        for qd, kd, vd, qbs in data:
            r = oracle.skip_head(qd, kd, vd, w.scale, np.float32(ln_lam), qblocks=qbs)
            tot += r.skipped.size
            sk += r.skipped.sum()
        return sk / tot

    lo, hi = 0.0, 16.0
    assert frac(hi) >= target, "target fraction not reached even at lambda = e^16"
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        if frac(mid) >= target:
            hi = mid
        else:
            lo = mid
    return math.exp(hi), float(frac(hi))


if __name__ == "__main__":
    main()
