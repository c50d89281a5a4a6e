"""Writes tests/golden/exact_tiny.json: a tiny KDA chain solved over exact
rationals by the oracle (oracle/exact.py), with its inputs.

Run from the repository root:  python tests/golden/make_golden.py
The inputs are fixed small rationals (alpha in (0, 1], beta in (0, 1],
keys not normalised); the expected outputs are exact fractions.  Only the
oracle is called.
"""
import json
import os
import sys
from fractions import Fraction as Fr

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))
from oracle.exact import kda_chain_exact  # noqa: E402

T, DK, DV = 6, 3, 2
# A fixed pattern of small rationals (no random generator, so the file is reproducible by eye).
q = [[Fr((3 * t + c) % 5 - 2, 3) for c in range(DK)] for t in range(T)]
k = [[Fr((2 * t + 3 * c) % 7 - 3, 4) for c in range(DK)] for t in range(T)]
v = [[Fr((5 * t + j) % 9 - 4, 2) for j in range(DV)] for t in range(T)]
alpha = [[Fr(1 + (t + c) % 4, 4) for c in range(DK)] for t in range(T)]
beta = [Fr(1 + t % 3, 3) for t in range(T)]
scale = Fr(1, 2)
S0 = [[Fr(c - j, 5) for j in range(DV)] for c in range(DK)]

o, S = kda_chain_exact(q, k, v, alpha, beta, scale, S0)
s = lambda m: [[str(x) for x in row] for row in m]
doc = {
    "about": "KDA chain over exact rationals; alpha given directly (g = log alpha)",
    "source": "oracle/exact.py via tests/golden/make_golden.py",
    "T": T, "dk": DK, "dv": DV, "scale": str(scale),
    "q": s(q), "k": s(k), "v": s(v), "alpha": s(alpha), "beta": [str(b) for b in beta],
    "S0": s(S0), "o": s(o), "S_final": s(S),
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_tiny.json"), "w") as f:
    json.dump(doc, f, indent=1)
print("wrote exact_tiny.json")
