"""fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package; the HIP product path never does, and
this package never imports the HIP path.

What it computes (definitions cited by page title and section):

* Recurrence (Eq. 1), "Kimi K3: the paper and proofs side by side", section
  2.1.1 (Equation 1) and its factorised ``update``: per (batch, head), token
  by token, decay the key rows of S by alpha_t, read the decayed state with
  k_t, subtract beta_t k_t (x) read, add beta_t k_t (x) v_t; then the query
  reads the updated state, o_t = S_t^T q_t.  Implemented in C
  (kda_oracle.c), fp64 throughout.
* Gate (Eq. 5), "Kimi K3 reading notes", section 2: g = g_min *
  sigmoid(exp(A^h) z), alpha = exp(g), g_min = -5.
* Decode: one step of the same recurrence per sequence, state carried.
* Fused prologue (the step before the recurrence): queries and keys get the
  regularised L2 normalisation of "the paper and proofs side by side",
  section 2.1.1 (Equations 2-6, "Preparing the queries, keys, values, and
  decay"), and the write strength beta, which must lie in (0, 1)
  ("architecture, derivations and a pinned-source audit", section 4.2), is
  taken from a logit through the logistic sigmoid.  Plain numpy in fp64,
  followed by the C recurrence.
* Draft replay, "Kimi K3: architecture, derivations and a pinned-source
  audit", section 10.3 (KDA state replay for speculative decoding): the
  drafted tokens of each sequence run from a cached state that is itself
  left unchanged; every drafted token's output is produced, and the state
  committed is the one after the accepted prefix.

Every entry point takes fp64 numpy arrays in the layouts of kda_oracle.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

G_MIN = -5.0
L2_EPS = 1e-6   # the regulariser of the query/key normalisation (paper-and-proofs page, section 2.1.1)

_DP = ctypes.POINTER(ctypes.c_double)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_DP)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def default_threads() -> int:
    """Worker threads of the C recurrence when a call passes nthreads = 0: the
    CPUs this process may run on, capped by OMP_NUM_THREADS when that is set
    (a host shared by several jobs sets it to each job's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _threads(n: int) -> int:
    return int(n) if int(n) > 0 else default_threads()


def l2_normalise(x: np.ndarray) -> np.ndarray:
    """Regularised L2 normalisation over the last axis, in fp64.

    "Kimi K3: the paper and proofs side by side", section 2.1.1 (Equations
    2-6): each coordinate is divided by a regularised norm with 1e-6 inside,
    so the result has norm strictly below one and a zero vector stays zero.
    The divisor itself did not survive extraction; the reading taken is
    sqrt(sum of squares + 1e-6), the one form with both stated properties
    whose regulariser is a plain additive 1e-6."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic sigmoid 1 / (1 + e^-x) in fp64: the map from a write-strength
    logit onto (0, 1) (the pages fix beta in (0, 1), not the map; this is
    the reading taken)."""
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def prologue(q_raw, k_raw, beta_logit) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The fused prologue: (q_hat, k_hat, beta) from un-normalised q, k [..., dk]
    and beta logits [...]."""
    return l2_normalise(q_raw), l2_normalise(k_raw), sigmoid(beta_logit)


class Oracle:
    """ctypes view of one build of kda_oracle.c (the default build, or a
    variant library built by a test from a modified copy of the source)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        L = ctypes.c_long
        lib.kda_oracle_gate.argtypes = [_DP, _DP, ctypes.c_double, L, L, L, L, L, _DP]
        lib.kda_oracle_gate.restype = ctypes.c_int
        lib.kda_oracle_recurrence.argtypes = [_DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP, L, L, L, L, L,
                                              ctypes.c_double, ctypes.c_int]
        lib.kda_oracle_recurrence.restype = ctypes.c_int
        lib.kda_oracle_forward_z.argtypes = [_DP, _DP, _DP, _DP, _DP, _DP, ctypes.c_double, _DP, _DP, _DP,
                                             L, L, L, L, L, ctypes.c_double, ctypes.c_int]
        lib.kda_oracle_forward_z.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def gate(self, z: np.ndarray, A: np.ndarray, g_min: float = G_MIN, chunk: int = 1) -> np.ndarray:
        """G [B,T,H,dk]: chunk-local inclusive sums of g = g_min*sigmoid(exp(A) z)
        over chunks of ``chunk`` tokens (chunk=1 gives g itself)."""
        z = _f64(z)
        A = _f64(A)
        B, T, H, dk = z.shape
        G = np.empty_like(z)
        rc = self.lib.kda_oracle_gate(_p(z), _p(A), float(g_min), B, T, H, dk, int(chunk), _p(G))
        if rc != 0:
            raise ValueError("kda_oracle_gate: bad arguments")
        return G

    def recurrence(self, q, k, v, beta, g, S0=None, scale: float = 1.0,
                   nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Eq. 1 token by token with per-token log-decay g (alpha = exp(g)).
        Returns (o [B,T,H,dv], S_T [B,H,dk,dv])."""
        q, k, v, beta, g, S0 = map(_f64, (q, k, v, beta, g, S0))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        o = np.zeros((B, T, H, dv))
        S = np.zeros((B, H, dk, dv))
        rc = self.lib.kda_oracle_recurrence(_p(q), _p(k), _p(v), _p(beta), _p(g), _p(S0), _p(o), _p(S),
                                            B, T, H, dk, dv, float(scale), _threads(nthreads))
        if rc != 0:
            raise ValueError("kda_oracle_recurrence: bad arguments")
        return o, S

    def forward_z(self, q, k, v, beta, z, A, g_min: float = G_MIN, S0=None, scale: float = 1.0,
                  nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Gate from decay logits z, then Eq. 1.  Returns (o, S_T)."""
        q, k, v, beta, z, A, S0 = map(_f64, (q, k, v, beta, z, A, S0))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        o = np.zeros((B, T, H, dv))
        S = np.zeros((B, H, dk, dv))
        rc = self.lib.kda_oracle_forward_z(_p(q), _p(k), _p(v), _p(beta), _p(z), _p(A), float(g_min),
                                           _p(S0), _p(o), _p(S), B, T, H, dk, dv, float(scale), _threads(nthreads))
        if rc != 0:
            raise ValueError("kda_oracle_forward_z: bad arguments")
        return o, S

    def replay(self, q, k, v, z, beta, A, S_snapshot, accepted, g_min: float = G_MIN, scale: float = 1.0,
               nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Speculative-decoding replay of ``n_draft`` drafted tokens per sequence.

        q, k, z: [n_draft, N, H, dk]; v: [n_draft, N, H, dv]; beta: [n_draft, N, H];
        S_snapshot: [N, H, dk, dv], the state before the drafts (not modified);
        accepted: [N] integers in [0, n_draft], the accepted prefix length of
        each sequence.  The drafts run one token at a time from the snapshot
        exactly as in ``decode``.  Returns (o [n_draft, N, H, dv] for every
        drafted token, the state of each sequence after its first accepted[n]
        tokens: the snapshot itself where accepted[n] == 0)."""
        q, k, v, z, beta, A = map(_f64, (q, k, v, z, beta, A))
        S = _f64(S_snapshot).copy()
        acc = np.asarray(accepted, dtype=np.int64)
        n_draft, N = q.shape[0], S.shape[0]
        if acc.shape != (N,) or np.any(acc < 0) or np.any(acc > n_draft):
            raise ValueError("accepted must hold N values in [0, n_draft]")
        committed = S.copy()
        outs = []
        for s in range(n_draft):
            o, S = self.forward_z(q[s][:, None], k[s][:, None], v[s][:, None], beta[s][:, None], z[s][:, None],
                                  A, g_min, S, scale, nthreads)
            outs.append(o[:, 0])
            done = acc == s + 1
            committed[done] = S[done]
        o = np.stack(outs) if outs else np.zeros((0,) + S.shape[:2] + (S.shape[-1],))
        return o, committed


    def forward_z_prologue(self, q_raw, k_raw, v, beta_logit, z, A, g_min: float = G_MIN, S0=None,
                           scale: float = 1.0, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """``prologue`` then ``forward_z``: the prefill of the fused-prologue entry point."""
        q, k, beta = prologue(q_raw, k_raw, beta_logit)
        return self.forward_z(q, k, v, beta, z, A, g_min, S0, scale, nthreads)

    def decode_prologue(self, q_raw, k_raw, v, z, beta_logit, A, S0, g_min: float = G_MIN, scale: float = 1.0,
                        nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """``prologue`` then the decode protocol (``decode``): [steps, N, H, ...] inputs."""
        q, k, beta = prologue(q_raw, k_raw, beta_logit)
        return _decode(self, q, k, v, z, beta, A, S0, g_min, scale, nthreads)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def gate(z, A, g_min: float = G_MIN, chunk: int = 1):
    return default().gate(z, A, g_min, chunk)


def recurrence(q, k, v, beta, g, S0=None, scale: float = 1.0, nthreads: int = 0):
    return default().recurrence(q, k, v, beta, g, S0, scale, nthreads)


def forward_z(q, k, v, beta, z, A, g_min: float = G_MIN, S0=None, scale: float = 1.0, nthreads: int = 0):
    return default().forward_z(q, k, v, beta, z, A, g_min, S0, scale, nthreads)


def decode(q, k, v, z, beta, A, S0, g_min: float = G_MIN, scale: float = 1.0,
           nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Decode protocol on the default build (see ``_decode``)."""
    return _decode(default(), q, k, v, z, beta, A, S0, g_min, scale, nthreads)


def _decode(orc: "Oracle", q, k, v, z, beta, A, S0, g_min: float = G_MIN, scale: float = 1.0,
            nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Decode protocol: ``steps`` consecutive single-token updates.

    q, k, z: [steps, N, H, dk]; v: [steps, N, H, dv]; beta: [steps, N, H];
    S0: [N, H, dk, dv].  Each step advances every sequence's state by one
    token (the same recurrence with T = 1) and reads it.
    Returns (o [steps, N, H, dv], S after the last step)."""
    q, k, v, z, beta, A, S = map(_f64, (q, k, v, z, beta, A, S0))
    steps = q.shape[0]
    outs = []
    for s in range(steps):
        # [N, H, d] -> [B=N, T=1, H, d]
        o, S = orc.forward_z(q[s][:, None], k[s][:, None], v[s][:, None], beta[s][:, None], z[s][:, None], A,
                             g_min, S, scale, nthreads)
        outs.append(o[:, 0])
    return np.stack(outs) if outs else np.zeros((0,) + S.shape[:2] + (S.shape[-1],)), S



def replay(q, k, v, z, beta, A, S_snapshot, accepted, g_min: float = G_MIN, scale: float = 1.0,
           nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Speculative-decoding replay (see ``Oracle.replay``) on the default build."""
    return default().replay(q, k, v, z, beta, A, S_snapshot, accepted, g_min, scale, nthreads)


def forward_z_prologue(q_raw, k_raw, v, beta_logit, z, A, g_min: float = G_MIN, S0=None, scale: float = 1.0,
                       nthreads: int = 0):
    return default().forward_z_prologue(q_raw, k_raw, v, beta_logit, z, A, g_min, S0, scale, nthreads)


def decode_prologue(q_raw, k_raw, v, z, beta_logit, A, S0, g_min: float = G_MIN, scale: float = 1.0,
                    nthreads: int = 0):
    return default().decode_prologue(q_raw, k_raw, v, z, beta_logit, A, S0, g_min, scale, nthreads)
