"""Writes tests/golden/exact_d4.json from the exact-rational brute force.

Calls only ``oracle.exact``; run from the repository root:
    python tests/golden/make_golden.py
The case: d_k = d_v = 4, 6 tokens, unit keys and queries with rational
entries (Pythagorean quadruples), rational alpha in (0, 1] and beta in [0, 1],
and a non-zero rational initial state, so that every term of the update
(decay, erase, write, inclusive read-out) and the state orientation matter.
"""
import json
import os
import sys
from fractions import Fraction as F

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle.exact import gdn_exact  # noqa: E402

UNIT = [
    [F(1, 3), F(2, 3), F(2, 3), F(0)],
    [F(2, 7), F(3, 7), F(6, 7), F(0)],
    [F(0), F(3, 5), F(4, 5), F(0)],
    [F(1, 2), F(1, 2), F(1, 2), F(1, 2)],
    [F(2, 3), F(-1, 3), F(0), F(2, 3)],
    [F(-6, 7), F(0), F(2, 7), F(3, 7)],
    [F(0), F(0), F(-5, 13), F(12, 13)],
]


def case():
    ks = [UNIT[i] for i in (0, 1, 2, 3, 1, 6)]
    qs = [UNIT[i] for i in (4, 5, 0, 6, 3, 2)]
    vs = [[F(1), F(-2), F(3, 2), F(0)], [F(1, 4), F(1), F(-1), F(2)], [F(0), F(1, 2), F(1, 3), F(-1)],
          [F(2), F(0), F(1), F(1, 5)], [F(-1), F(1), F(1), F(1)], [F(3, 4), F(-3, 4), F(0), F(1, 8)]]
    alphas = [F(1), F(1, 2), F(3, 4), F(1), F(1, 10), F(9, 10)]
    betas = [F(1, 2), F(1), F(1, 4), F(0), F(3, 5), F(1)]
    S0 = [[F(1, 10), F(0), F(-1, 5), F(0)], [F(0), F(1, 2), F(0), F(1, 3)],
          [F(1, 4), F(0), F(0), F(-1, 2)], [F(0), F(-1, 6), F(1, 7), F(0)]]
    return qs, ks, vs, alphas, betas, S0


def main():
    qs, ks, vs, alphas, betas, S0 = case()
    outs, S = gdn_exact(qs, ks, vs, alphas, betas, S0)
    s = lambda x: str(x)  # noqa: E731
    data = {
        "citation": "Exact-rational brute force (oracle/exact.py) of the gated delta rule named by the "
                    "'SANA-WM' cookbook page, table 'Architecture & components', row 'Attention'.",
        "generator": "tests/golden/make_golden.py",
        "q": [[s(x) for x in r] for r in qs], "k": [[s(x) for x in r] for r in ks],
        "v": [[s(x) for x in r] for r in vs], "alpha": [s(x) for x in alphas],
        "beta": [s(x) for x in betas], "state0": [[s(x) for x in r] for r in S0],
        "o": [[s(x) for x in r] for r in outs], "state": [[s(x) for x in r] for r in S],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_d4.json")
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
