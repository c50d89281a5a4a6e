"""The KDA recurrence over exact rationals (oracle, test infrastructure only).

Same steps as ref.kda_forward ("Understanding Kimi Delta Attention", section
"The KDA Recurrence"; "kimi delta attn from first principles", sections
"KDA" and "three gates"), but every quantity is a fractions.Fraction and the
gate is given directly as alpha (exp of a rational is not rational).  Used on
tiny inputs to bound the fp64 oracle's rounding and to write golden fixtures.
"""
from __future__ import annotations

from fractions import Fraction


def kda_chain_exact(q, k, v, alpha, beta, scale, S0=None):
    """One chain.  q, k, alpha: T lists of dk Fractions; v: T lists of dv;
    beta: T Fractions; scale: Fraction; S0: dk x dv nested lists or None.
    Returns (o: T lists of dv, S_T: dk x dv)."""
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dv for _ in range(dk)] if S0 is None else [list(r) for r in S0]
    out = []
    for t in range(T):
        S = [[alpha[t][c] * S[c][j] for j in range(dv)] for c in range(dk)]          # decay rows
        pred = [sum(S[c][j] * k[t][c] for c in range(dk)) for j in range(dv)]        # S^T k
        u = [beta[t] * (v[t][j] - pred[j]) for j in range(dv)]                        # delta error
        S = [[S[c][j] + k[t][c] * u[j] for j in range(dv)] for c in range(dk)]       # write
        out.append([scale * sum(S[c][j] * q[t][c] for c in range(dk)) for j in range(dv)])
    return out, S
