"""Pure-Python index-loop brute force of the KDA recurrence (tiny inputs only).

TEST INFRASTRUCTURE ONLY.  This follows the coordinate statement of the
factorised update ("Kimi K3: the paper and proofs side by side", section
2.1.1, theorem update_get2): for every key row i and value column j,

    S'[i][j] = alpha[i] * S[i][j]
               - beta * k[i] * (sum_r k[r] * alpha[r] * S[r][j])
               + beta * k[i] * v[j]

followed by the read after the update, o[j] = sum_i S'[i][j] * q[i].  It uses
only Python floats and loops, so it shares nothing with the C oracle beyond the
definition, and is cross-checked against it on tiny shapes.
"""
from __future__ import annotations

import math


def step(S, q, k, v, alpha, beta):
    dk, dv = len(S), len(S[0])
    out = [[0.0] * dv for _ in range(dk)]
    for i in range(dk):
        for j in range(dv):
            old_read = 0.0
            for r in range(dk):
                old_read += k[r] * alpha[r] * S[r][j]
            out[i][j] = alpha[i] * S[i][j] - beta * k[i] * old_read + beta * k[i] * v[j]
    o = [sum(out[i][j] * q[i] for i in range(dk)) for j in range(dv)]
    return out, o


def gate_alpha(z, A, g_min=-5.0):
    """alpha = exp(g_min * sigmoid(exp(A) * z)) for one token's channels."""
    return [math.exp(g_min / (1.0 + math.exp(-math.exp(a) * zz))) for zz, a in zip(z, A)]


def forward(q, k, v, beta, alpha, S0=None):
    """q, k, alpha: [T][dk]; v: [T][dv]; beta: [T] (nested lists or arrays).
    Returns (o [T][dv], S_T [dk][dv]) as nested lists."""
    T = len(k)
    dk = len(k[0]) if T else (len(S0) if S0 is not None else 0)
    dv = len(v[0]) if T else (len(S0[0]) if S0 is not None else 0)
    S = [[float(S0[i][j]) if S0 is not None else 0.0 for j in range(dv)] for i in range(dk)]
    outs = []
    for t in range(T):
        S, o = step(S, [float(x) for x in q[t]], [float(x) for x in k[t]], [float(x) for x in v[t]],
                    [float(x) for x in alpha[t]], float(beta[t]))
        outs.append(o)
    return outs, S
