"""fp64 chunkwise (WY/UT) form of the KDA recurrence -- an algebra check.

TEST INFRASTRUCTURE ONLY, and NOT the parity oracle (the token loop in
kda_oracle.c is).  The pages name a chunkwise form ("Kimi K3: architecture,
derivations and a pinned-source audit", section 4.5, whose equations are
stripped; the reading notes, section 2, name the reciprocal cumulative-decay
key rescaling).  The form below is derived from Eq. 1 and is tested against
the token loop; it documents the regrouping the GPU kernels use.

For one chunk of C tokens with entry state S, per key channel c:
  G_t = sum_{u<=t} g_u (chunk-local), Gamma_t = exp(G_t),
  u_t = beta_t (v_t - (Diag(alpha_t) S_{t-1})^T k_t)  so S_t = Diag(alpha_t) S_{t-1} + k_t u_t^T,
  L[t,s] = beta_t sum_c k_tc k_sc exp(G_tc - G_sc)       (s < t, else 0)
  (I + L) U = Diag(beta) (V - (K*Gamma) S)
  Tm = (I + L)^-1 Diag(beta),  W = Tm (K*Gamma),  Ut = Tm V,  U = Ut - W S
  P[t,s] = sum_c q_tc k_sc exp(G_tc - G_sc)              (s <= t, else 0)
  O = (Q*Gamma) S + P U
  S_C = Diag(Gamma_C) S + (K * exp(G_C - G))^T U
"""
from __future__ import annotations

import numpy as np


def chunk_forward(q, k, v, beta, g, S0=None, chunk: int = 64, scale: float = 1.0):
    """q, k, g: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; S0: [B,H,dk,dv].
    Returns (o, S_T) in fp64."""
    q, k, v, beta, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, g))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_out = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                K = k[b, t0:t1, h]
                Q = q[b, t0:t1, h]
                V = v[b, t0:t1, h]
                bt = beta[b, t0:t1, h]
                G = np.cumsum(g[b, t0:t1, h], axis=0)
                n = t1 - t0
                D = np.exp(G[:, None, :] - G[None, :, :])       # [t, s, c] = exp(G_tc - G_sc)
                KK = np.einsum("tc,sc,tsc->ts", K, K, D)
                QK = np.einsum("tc,sc,tsc->ts", Q, K, D)
                L = np.tril(bt[:, None] * KK, -1)
                P = np.tril(QK, 0)
                Tm = np.linalg.solve(np.eye(n) + L, np.diag(bt))
                Gam = np.exp(G)
                W = Tm @ (K * Gam)
                Ut = Tm @ V
                U = Ut - W @ S
                o[b, t0:t1, h] = scale * ((Q * Gam) @ S + P @ U)
                S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ U
            S_out[b, h] = S
    return o, S_out
