"""Writes exact_tiny.json: exact rational results of tiny cases.

Calls only oracle/exact.py (explicit per-token transition matrices multiplied
out in Fraction arithmetic).  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import exact  # noqa: E402


def case(seed, T, dk, dv, channel):
    r = np.random.Generator(np.random.PCG64(seed))
    fr = lambda lo, hi, den: Fraction(int(r.integers(lo, hi)), den)  # noqa: E731
    q = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-8, 9, 4) for _ in range(dv)] for _ in range(T)]
    if channel:
        alpha = [[fr(1, 9, 8) for _ in range(dk)] for _ in range(T)]
    else:
        alpha = [[fr(1, 9, 8)] * dk for _ in range(T)]
    beta = [fr(0, 9, 8) for _ in range(T)]
    S0 = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(dv)]
    o, st = exact.run(q, k, v, alpha, beta, S0)
    s = lambda m: [[str(x) for x in row] for row in m]  # noqa: E731
    return dict(seed=seed, channel=channel, q=s(q), k=s(k), v=s(v), alpha=s(alpha),
                beta=[str(b) for b in beta], S0=s(S0), o=s(o), S_T=s(st))


if __name__ == "__main__":
    cases = [case(201, 4, 3, 2, False), case(202, 6, 4, 3, True),
             case(203, 3, 2, 4, True), case(204, 5, 5, 2, False)]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_tiny.json")
    with open(out, "w") as fh:
        json.dump(cases, fh, indent=1)
    print("wrote", out)
