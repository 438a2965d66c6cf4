"""fp64 reverse-mode derivative of the KDA forward pass (the oracle of the backward).

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``).

What is differentiated: the fused-gate forward of this package, per batch
entry b and head h, token by token ("Kimi K3: the paper and proofs side by
side", section 2.1.1, Equation 1 and its factorised update; the gate of
"Kimi K3 reading notes", section 2):

    x_t   = e^{A} z_t                   (per key channel)
    g_t   = g_min sigmoid(x_t),  alpha_t = e^{g_t}
    D_t   = Diag(alpha_t) S_{t-1}        decay the key rows
    e_t   = v_t - D_t^T k_t              what the key should read, minus what it reads
    S_t   = D_t + beta_t k_t e_t^T       erase + write
    o_t   = scale S_t^T q_t              read after the update

with a scalar loss L whose gradients dL/do_t (``do``) and dL/dS_T (``dS_out``,
optional) are given.  The pages train through fused KDA kernels and check
gradients against the scalar recurrence ("Kimi K3: architecture, derivations
and a pinned-source audit", CPU laboratory: the analytic derivative of
sum(S_next^2) with respect to the old state, checked by finite differences);
they print no backward formulas, so the ones below are the chain rule applied
to the steps above, in reverse token order, written out by hand:

    dS_t  += scale q_t do_t^T            dq_t = scale S_t do_t
    dbeta_t = k_t^T dS_t e_t             dk_t = beta_t dS_t e_t
    de_t  = beta_t dS_t^T k_t            dv_t = de_t
    dD_t  = dS_t - k_t de_t^T            dk_t -= D_t de_t
    dalpha_t[c] = sum_j dD_t[c, j] S_{t-1}[c, j]
    dS_{t-1} = Diag(alpha_t) dD_t
    dg_t = alpha_t dalpha_t,  dx_t = g_min sigmoid(x_t)(1 - sigmoid(x_t)) dg_t
    dz_t = e^{A} dx_t,        dA  += sum over (b, t) of e^{A} z_t dx_t
    dS_in = dS_0

Every array is fp64; states are kept for all tokens (small test shapes only).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

G_MIN = -5.0


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def forward_states(q, k, v, beta, z, A, g_min: float = G_MIN, S0=None, scale: float = 1.0):
    """The forward above, keeping what the reverse sweep needs.

    q, k, z [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H]; A [H, dk];
    S0 [B, H, dk, dv] or None.  Returns a dict with o [B, T, H, dv], the
    states S [T + 1, B, H, dk, dv] (S[0] = S0), alpha and x [B, T, H, dk]."""
    q, k, v, beta, z, A, S0 = map(_f64, (q, k, v, beta, z, A, S0))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    x = np.exp(A)[None, None] * z
    sig = 1.0 / (1.0 + np.exp(-x))
    alpha = np.exp(g_min * sig)
    S = np.zeros((T + 1, B, H, dk, dv))
    if S0 is not None:
        S[0] = S0
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        D = alpha[:, t, :, :, None] * S[t]                       # [B, H, dk, dv]
        e = v[:, t] - np.einsum("bhc,bhcj->bhj", k[:, t], D)      # [B, H, dv]
        S[t + 1] = D + beta[:, t, :, None, None] * k[:, t, :, :, None] * e[:, :, None, :]
        o[:, t] = scale * np.einsum("bhcj,bhc->bhj", S[t + 1], q[:, t])
    return {"o": o, "S": S, "alpha": alpha, "x": x, "sig": sig}


def backward_z(q, k, v, beta, z, A, do, dS_out=None, g_min: float = G_MIN, S0=None,
               scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Gradients of L given do = dL/do [B, T, H, dv] and dS_out = dL/dS_T
    [B, H, dk, dv] (None: the final state does not enter L).

    Returns dq, dk, dz [B, T, H, dk]; dv [B, T, H, dv]; dbeta [B, T, H];
    dA [H, dk]; dS_in [B, H, dk, dv]; and the forward's o and S_T."""
    q, k, v, beta, z, A, do, dS_out, S0 = map(_f64, (q, k, v, beta, z, A, do, dS_out, S0))
    f = forward_states(q, k, v, beta, z, A, g_min, S0, scale)
    S, alpha, sig = f["S"], f["alpha"], f["sig"]
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dx = np.zeros_like(z)
    dS = np.zeros((B, H, dk, dv)) if dS_out is None else dS_out.copy()
    for t in range(T - 1, -1, -1):
        kt, qt, bt = k[:, t], q[:, t], beta[:, t]
        St, Sp = S[t + 1], S[t]
        D = alpha[:, t, :, :, None] * Sp
        e = v[:, t] - np.einsum("bhc,bhcj->bhj", kt, D)
        # o_t = scale S_t^T q_t
        dS = dS + scale * qt[:, :, :, None] * do[:, t][:, :, None, :]
        dq[:, t] = scale * np.einsum("bhcj,bhj->bhc", St, do[:, t])
        # S_t = D_t + beta_t k_t e_t^T
        dbeta[:, t] = np.einsum("bhc,bhcj,bhj->bh", kt, dS, e)
        dkt = bt[:, :, None] * np.einsum("bhcj,bhj->bhc", dS, e)
        de = bt[:, :, None] * np.einsum("bhcj,bhc->bhj", dS, kt)
        # e_t = v_t - D_t^T k_t
        dv_[:, t] = de
        dD = dS - kt[:, :, :, None] * de[:, :, None, :]
        dkt = dkt - np.einsum("bhcj,bhj->bhc", D, de)
        dk_[:, t] = dkt
        # D_t = Diag(alpha_t) S_{t-1}
        dalpha = np.sum(dD * Sp, axis=-1)                          # [B, H, dk]
        dS = alpha[:, t, :, :, None] * dD
        # alpha = e^g, g = g_min sigmoid(x)
        dg = alpha[:, t] * dalpha
        dx[:, t] = g_min * sig[:, t] * (1.0 - sig[:, t]) * dg
    eA = np.exp(A)
    dz = eA[None, None] * dx
    dA = np.einsum("bthc,bthc->hc", dx, z) * eA
    return {"dq": dq, "dk": dk_, "dv": dv_, "dbeta": dbeta, "dz": dz, "dA": dA, "dS_in": dS,
            "o": f["o"], "S_T": S[T]}


def loss(o, S_T, w_o, w_S=None) -> float:
    """The linear test loss sum(w_o * o) + sum(w_S * S_T): its do is w_o and its dS_out is w_S."""
    val = float(np.sum(w_o * o))
    if w_S is not None:
        val += float(np.sum(w_S * S_T))
    return val
