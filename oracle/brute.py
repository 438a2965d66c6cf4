"""Pure-Python index-loop brute force of the KDA recurrence (tiny inputs only).

TEST INFRASTRUCTURE ONLY.  This follows the coordinate statement of the
factorised update ("Kimi K3: the paper and proofs side by side", section
2.1.1, theorem update_get2): for every key row i and value column j,

    S'[i][j] = alpha[i] * S[i][j]
               - beta * k[i] * (sum_r k[r] * alpha[r] * S[r][j])
               + beta * k[i] * v[j]

followed by the read after the update, o[j] = sum_i S'[i][j] * q[i].  The
same coordinate formula is the scalar step of the CPU laboratory on "Kimi K3:
architecture, derivations and a pinned-source audit" (section "CPU
laboratory: recurrence, depth, experts and replay"); here it is evaluated one
value column at a time, since the columns of the state evolve independently
given (k, beta, alpha).  It uses only Python floats and loops, so it shares
nothing with the C oracle beyond the definition, and is cross-checked against
it on tiny shapes.
"""
from __future__ import annotations

import math


def step(S, q, k, v, alpha, beta):
    """One token: returns (S', o) as nested lists."""
    dk, dv = len(S), len(S[0])
    new = [[0.0] * dv for _ in range(dk)]
    o = [0.0] * dv
    for j in range(dv):
        col = [alpha[i] * S[i][j] for i in range(dk)]  # column j with its key rows decayed
        pred = 0.0
        for i in range(dk):
            pred += k[i] * col[i]                       # what the decayed column predicts at k
        err = v[j] - pred
        for i in range(dk):
            new[i][j] = col[i] + beta * k[i] * err      # erase along k, write v
        acc = 0.0
        for i in range(dk):
            acc += new[i][j] * q[i]                     # the query reads the updated column
        o[j] = acc
    return new, o


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
