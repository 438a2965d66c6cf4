"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when it disagrees with a printed value, a closed form, an invariant, a special
case or a brute-force computation.  tests/test_oracle_pins.py runs them on the
oracle; tests/test_oracle_mutations.py runs them on deliberately broken builds
of the oracle source and requires each broken build to fail at least one.
"""
from __future__ import annotations

import math
import os

import numpy as np

from oracle import brute, chunk_form

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def _rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _kv(name):
    out = {}
    for line in _rows(name):
        key, val = [x.strip() for x in line.split("=", 1)]
        if ";" in val:
            out[key] = np.array([[float(x) for x in r.split()] for r in val.split(";")])
        else:
            out[key] = np.array([float(x) for x in val.split()])
    return out


def run1(orc, q, k, v, alpha, beta, S0=None, scale=1.0):
    """One (batch, head) sequence: q, k, alpha [T, dk]; v [T, dv]; beta [T]."""
    q = np.asarray(q, float)[None, :, None, :]
    k = np.asarray(k, float)[None, :, None, :]
    v = np.asarray(v, float)[None, :, None, :]
    g = np.log(np.asarray(alpha, float))[None, :, None, :]
    beta = np.asarray(beta, float)[None, :, None]
    S = None if S0 is None else np.asarray(S0, float)[None, None]
    o, S = orc.recurrence(q, k, v, beta, g, S, scale)
    return o[0, :, 0], S[0, 0]


def _rand_seq(rng, T, dk, dv, unit_keys=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.05, 0.99, (T, dk))
    beta = rng.uniform(0.05, 0.95, T)
    S0 = rng.standard_normal((dk, dv))
    return q, k, v, alpha, beta, S0


def _dense_step(S, k, v, alpha, beta):
    """Eq. 1 as written with matrices: (I - beta k k^T) Diag(alpha) S + beta k v^T."""
    dk = len(k)
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(alpha) @ S + beta * np.outer(k, v)


# ----------------------------------------------------------------------------
# printed values
# ----------------------------------------------------------------------------
def pin_scalar_delta_step(orc):
    """Paper-and-proofs page, 2.1.1: s=6, alpha=.8, v=10, beta=.5 -> 7.4 (and the
    beta=1 / beta=0 limits)."""
    for line in _rows("scalar_delta_step.txt"):
        s_prev, alpha, v, beta, s_next = map(float, line.split())
        o, S = run1(orc, [[1.0]], [[1.0]], [[v]], [[alpha]], [beta], S0=[[s_prev]])
        assert abs(S[0, 0] - s_next) < 1e-12, (line, S)
        assert abs(o[0, 0] - s_next) < 1e-12, (line, o)


def pin_token_order(orc):
    """Paper-and-proofs page, 2.1.1: values 2 then 10 -> 5.25; 10 then 2 -> 2.25."""
    for line in _rows("token_order.txt"):
        alpha, beta, v1, v2, s_final = map(float, line.split())
        o, S = run1(orc, [[1.0], [1.0]], [[1.0], [1.0]], [[v1], [v2]], [[alpha], [alpha]], [beta, beta])
        assert abs(S[0, 0] - s_final) < 1e-12, (line, S)


def pin_lean_one_token(orc):
    """Paper-and-proofs page, "Writing the model in Lean": output 3.000000."""
    d = _kv("lean_one_token.txt")
    o, S = run1(orc, [d["q"]], [d["k"]], [d["v"]], [d["alpha"]], [d["beta"][0]], S0=np.zeros((2, 1)))
    assert f"{o[0, 0]:.6f}" == f"{d['o0'][0]:.6f}", o


def pin_worked_2x2(orc):
    """Derivations page, "Worked KDA state update and limits"."""
    d = _kv("worked_2x2_update.txt")
    o, S = run1(orc, [d["q"]], [d["k"]], [d["v"]], [d["alpha"]], [d["beta"][0]], S0=d["S"])
    np.testing.assert_allclose(S, d["S_next"], atol=1e-12)
    np.testing.assert_allclose(o[0], d["o"], atol=1e-12)


def pin_gate_slider(orc):
    """Paper-and-proofs page, 2.1.1 Eqs. 2-6 slider: z = 0 -> g = -2.5000,
    alpha = 0.0821, for any A (sigmoid(0) = 1/2 exactly)."""
    z0, g_p, a_p, dec = _rows("gate_slider.txt")[0].split()
    dec = int(dec)
    A = np.array([[-3.0, -0.4, 0.0, 0.7, 2.0]])
    z = np.full((1, 1, 1, A.shape[1]), float(z0))
    g = orc.gate(z, A, -5.0, 1)[0, 0, 0]
    for gi in g:
        assert f"{gi:.{dec}f}" == g_p
        assert f"{math.exp(gi):.{dec}f}" == a_p
        assert gi == -2.5


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------
def pin_gate_closed_form(orc):
    """g = g_min * sigmoid(exp(A) z): exact values where the sigmoid is rational.
    exp(A) z = ln 3 gives sigmoid 3/4; = -ln 3 gives 1/4."""
    A = np.array([[0.0, math.log(2.0), -math.log(4.0), 0.0]])
    z = np.array([[[[math.log(3.0), math.log(3.0) / 2, 4 * math.log(3.0), -math.log(3.0)]]]])
    g = orc.gate(z, A, -5.0, 1)[0, 0, 0]
    np.testing.assert_allclose(g, [-3.75, -3.75, -3.75, -1.25], rtol=1e-14)
    # other floors scale linearly
    g2 = orc.gate(z, A, -2.0, 1)[0, 0, 0]
    np.testing.assert_allclose(g2, [-1.5, -1.5, -1.5, -0.5], rtol=1e-14)
    # limits: z -> +inf saturates at g_min, z -> -inf at 0
    zl = np.array([[[[1e3, -1e3, 1e3, -1e3]]]])
    gl = orc.gate(zl, A, -5.0, 1)[0, 0, 0]
    np.testing.assert_allclose(gl, [-5.0, 0.0, -5.0, 0.0], atol=1e-300)


def pin_gate_chunk_sums(orc):
    """The chunk-local sums restart at every chunk start and add up g."""
    rng = np.random.default_rng(5)
    z = rng.standard_normal((2, 37, 3, 4))
    A = rng.standard_normal((3, 4))
    g = orc.gate(z, A, -5.0, 1)
    for chunk in (1, 4, 16, 64):
        G = orc.gate(z, A, -5.0, chunk)
        for t in range(37):
            t0 = t - t % chunk
            np.testing.assert_allclose(G[:, t], g[:, t0:t + 1].sum(axis=1), rtol=1e-13, atol=1e-13)


def pin_closed_form_single_step(orc):
    """Factorised update == dense (I - beta k k^T) Diag(alpha) S + beta k v^T."""
    rng = np.random.default_rng(11)
    for trial in range(5):
        dk, dv = 7, 5
        q, k, v, alpha, beta, S0 = _rand_seq(rng, 1, dk, dv, unit_keys=(trial % 2 == 0))
        o, S = run1(orc, q, k, v, alpha, beta, S0=S0)
        Sd = _dense_step(S0, k[0], v[0], alpha[0], beta[0])
        np.testing.assert_allclose(S, Sd, atol=1e-13, rtol=1e-13)
        np.testing.assert_allclose(o[0], Sd.T @ q[0], atol=1e-13, rtol=1e-13)


def pin_deltanet_reduction(orc):
    """alpha == 1 (g == 0) is the delta rule: S_t = (I - beta k k^T) S + beta k v^T
    (derivations page, section 4.2)."""
    rng = np.random.default_rng(12)
    q, k, v, _, beta, S0 = _rand_seq(rng, 20, 6, 4)
    alpha = np.ones((20, 6))
    o, S = run1(orc, q, k, v, alpha, beta, S0=S0)
    Sr = S0.copy()
    for t in range(20):
        Sr = (np.eye(6) - beta[t] * np.outer(k[t], k[t])) @ Sr + beta[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(o[t], Sr.T @ q[t], atol=1e-12)
    np.testing.assert_allclose(S, Sr, atol=1e-12)


def pin_pure_decay(orc):
    """beta == 0 leaves only the decay (paper-and-proofs page, 2.1.1)."""
    rng = np.random.default_rng(13)
    q, k, v, alpha, _, S0 = _rand_seq(rng, 15, 5, 3)
    beta = np.zeros(15)
    o, S = run1(orc, q, k, v, alpha, beta, S0=S0)
    Sr = S0.copy()
    for t in range(15):
        Sr = alpha[t][:, None] * Sr
        np.testing.assert_allclose(o[t], Sr.T @ q[t], atol=1e-13)
    np.testing.assert_allclose(S, Sr, atol=1e-13)


def pin_overwrite(orc):
    """beta = 1, alpha = 1, unit k: the state then returns v_t at key k_t exactly
    (a write strength of one replaces the prediction)."""
    rng = np.random.default_rng(14)
    T, dk, dv = 12, 8, 5
    _, k, v, _, _, S0 = _rand_seq(rng, T, dk, dv)
    o, S = run1(orc, k, k, v, np.ones((T, dk)), np.ones(T), S0=S0)
    np.testing.assert_allclose(o, v, atol=1e-12)


def pin_constant_input_scalar(orc):
    """d_k = d_v = 1, k = q = 1, constant alpha, beta, v: s_t = a^t s_0 +
    beta v (1 - a^t)/(1 - a) with a = alpha (1 - beta); checked at T = 10^6."""
    T = 1_000_000
    alpha, beta, v, s0 = 0.999995, 0.3, 1.7, -2.0
    ones = np.ones((T, 1))
    o, S = run1(orc, ones, ones, np.full((T, 1), v), np.full((T, 1), alpha), np.full(T, beta), S0=[[s0]])
    a = alpha * (1 - beta)
    for t in (1, 2, 10, 1000, T):
        ref = a ** t * s0 + beta * v * (1 - a ** t) / (1 - a)
        assert abs(o[t - 1, 0] - ref) <= 1e-12 * max(1.0, abs(ref)), (t, o[t - 1, 0], ref)


def pin_scale(orc):
    """The output scale multiplies o only (power of two: bitwise)."""
    rng = np.random.default_rng(15)
    q, k, v, alpha, beta, S0 = _rand_seq(rng, 9, 4, 3)
    o1, S1 = run1(orc, q, k, v, alpha, beta, S0=S0, scale=1.0)
    o2, S2 = run1(orc, q, k, v, alpha, beta, S0=S0, scale=0.25)
    assert np.array_equal(o2, 0.25 * o1) and np.array_equal(S1, S2)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def pin_gate_and_tile_ranges(orc):
    """g in [g_min, 0] (open interval where the sigmoid does not saturate in
    fp64), alpha in [e^-5, 1], and every 16-token window of log-decay in
    [-80, 0] (reading notes, section 2; paper-and-proofs page slider note)."""
    rng = np.random.default_rng(16)
    z = 6.0 * rng.standard_normal((2, 200, 3, 16))
    A = rng.standard_normal((3, 16))
    g = orc.gate(z, A, -5.0, 1)
    assert np.all(g >= -5.0) and np.all(g <= 0.0)
    x = np.exp(A)[None, None] * z
    inner = np.abs(x) < 30
    assert np.all(g[inner] > -5.0) and np.all(g[inner] < 0.0)
    alpha = np.exp(g)
    assert np.all(alpha >= math.exp(-5.0)) and np.all(alpha <= 1.0)
    G16 = orc.gate(z, A, -5.0, 16)
    assert np.all(G16 >= -80.0) and np.all(G16 <= 0.0)
    cs = np.cumsum(g, axis=1)
    win = cs[:, 15:] - np.concatenate([np.zeros_like(cs[:, :1]), cs[:, :-16]], axis=1)
    assert np.all(win >= -80.0) and np.all(win <= 0.0)


def pin_chunk_split(orc):
    """Carrying the state across a split changes neither outputs nor the final
    state (paper-and-proofs page, "Streaming, full sequences, and chunk
    boundaries", run_append) -- bitwise in fp64."""
    rng = np.random.default_rng(17)
    q, k, v, alpha, beta, S0 = _rand_seq(rng, 50, 6, 5)
    o, S = run1(orc, q, k, v, alpha, beta, S0=S0)
    for cut in (0, 1, 17, 49, 50):
        oa, Sa = run1(orc, q[:cut], k[:cut], v[:cut], alpha[:cut], beta[:cut], S0=S0)
        ob, Sb = run1(orc, q[cut:], k[cut:], v[cut:], alpha[cut:], beta[cut:], S0=Sa)
        assert np.array_equal(np.concatenate([oa, ob]), o), cut
        assert np.array_equal(Sb, S), cut


def pin_superposition(orc):
    """At fixed k, beta, alpha the map (S_in, V) -> (S_T, O) is linear:
    run(S, V) = run(0, V) + run(S, 0); the state part is S~ + M S (the
    fragment decomposition of the reading notes, section 7)."""
    rng = np.random.default_rng(18)
    q, k, v, alpha, beta, S0 = _rand_seq(rng, 30, 5, 4)
    o, S = run1(orc, q, k, v, alpha, beta, S0=S0)
    o1, S1 = run1(orc, q, k, v, alpha, beta, S0=np.zeros_like(S0))
    o2, S2 = run1(orc, q, k, v * 0, alpha, beta, S0=S0)
    np.testing.assert_allclose(o, o1 + o2, atol=1e-12)
    np.testing.assert_allclose(S, S1 + S2, atol=1e-12)


def pin_affine_composition(orc):
    """Each token is the affine map S -> M_t S + U_t with M_t = (I - beta k k^T)
    Diag(alpha) and U_t = beta k v^T (derivations page, section 4.5, which
    regroups these compositions into chunks; the CPU laboratory on the same page,
    "CPU laboratory: recurrence, depth, experts and replay", composes them too).
    Written as the linear map [[M_t, U_t], [0, I]] on [S; I] (a (dk + dv) x dv
    block matrix), the ordered product over all tokens applied to [S_0; I] is
    [S_T; I] of the oracle, and the product over a sequence equals the product of
    the products over any two consecutive pieces of it: the regrouping the
    chunked and segment-parallel forms rely on."""
    rng = np.random.default_rng(19)
    T, dk, dv = 9, 4, 3
    q, k, v, alpha, beta, S0 = _rand_seq(rng, T, dk, dv)
    o, S = run1(orc, q, k, v, alpha, beta, S0=S0)

    def block(t):
        X = np.zeros((dk + dv, dk + dv))
        X[:dk, :dk] = (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(alpha[t])
        X[:dk, dk:] = beta[t] * np.outer(k[t], v[t])
        X[dk:, dk:] = np.eye(dv)
        return X

    def product(t0, t1):  # tokens t0 .. t1-1, the latest applied last (leftmost)
        X = np.eye(dk + dv)
        for t in range(t0, t1):
            X = block(t) @ X
        return X

    whole = product(0, T)
    out = whole @ np.vstack([S0, np.eye(dv)])
    np.testing.assert_allclose(out[:dk], S, atol=1e-12)
    np.testing.assert_allclose(out[dk:], np.eye(dv), atol=0)
    for cut in range(T + 1):
        np.testing.assert_allclose(product(cut, T) @ product(0, cut), whole, atol=1e-12)


def pin_brute_force(orc):
    """Pure-Python index loops vs the C oracle on tiny shapes (<= 1e-12)."""
    rng = np.random.default_rng(20)
    for T, dk, dv in ((24, 6, 5), (7, 3, 2), (1, 16, 16)):
        q, k, v, alpha, beta, S0 = _rand_seq(rng, T, dk, dv)
        o, S = run1(orc, q, k, v, alpha, beta, S0=S0)
        ob, Sb = brute.forward(q, k, v, beta, alpha, S0)
        np.testing.assert_allclose(o, np.array(ob), atol=1e-12)
        np.testing.assert_allclose(S, np.array(Sb), atol=1e-12)


def pin_contraction(orc):
    """|k| <= 1, beta in (0,1), alpha <= 1, v = 0: each transition is a
    contraction, so the Frobenius norm of S never grows."""
    rng = np.random.default_rng(21)
    T, dk, dv = 40, 6, 4
    q, k, v, alpha, beta, S0 = _rand_seq(rng, T, dk, dv)
    S = S0
    prev = np.linalg.norm(S)
    for t in range(T):
        _, S = run1(orc, q[t:t + 1], k[t:t + 1], 0 * v[t:t + 1], alpha[t:t + 1], beta[t:t + 1], S0=S)
        cur = np.linalg.norm(S)
        assert cur <= prev * (1 + 1e-14), (t, cur, prev)
        prev = cur


def pin_causality_and_independence(orc):
    """Changing a later token leaves earlier outputs unchanged; permuting heads
    or batch entries permutes the results (heads are independent: the packed
    update of the paper-and-proofs page acts head by head)."""
    rng = np.random.default_rng(22)
    B, T, H, dk, dv = 2, 12, 3, 4, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) / 2
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.uniform(0, 3, (B, T, H, dk))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.recurrence(q, k, v, beta, g, S0)
    v2 = v.copy()
    v2[:, 7:] += 1.0
    o2, _ = orc.recurrence(q, k, v2, beta, g, S0)
    assert np.array_equal(o[:, :7], o2[:, :7]) and not np.allclose(o[:, 7:], o2[:, 7:])
    ph, pb = [2, 0, 1], [1, 0]
    o3, S3 = orc.recurrence(q[pb][:, :, ph], k[pb][:, :, ph], v[pb][:, :, ph], beta[pb][:, :, ph],
                            g[pb][:, :, ph], S0[pb][:, ph])
    assert np.array_equal(o3, o[pb][:, :, ph]) and np.array_equal(S3, S[pb][:, ph])


def pin_chunk_form(orc):
    """The derived chunkwise WY/UT regrouping equals the token loop (<= 1e-12),
    with an incoming state and a ragged last chunk."""
    rng = np.random.default_rng(23)
    for B, T, H, dk, dv, C in ((1, 150, 2, 8, 6, 64), (2, 40, 1, 16, 16, 16)):
        q = rng.standard_normal((B, T, H, dk))
        k = rng.standard_normal((B, T, H, dk))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, T, H, dv))
        g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dk))))
        beta = rng.uniform(0.05, 0.95, (B, T, H))
        S0 = rng.standard_normal((B, H, dk, dv))
        o, S = orc.recurrence(q, k, v, beta, g, S0)
        oc, Sc = chunk_form.chunk_forward(q, k, v, beta, g, S0, chunk=C)
        assert np.linalg.norm(oc - o) <= 1e-12 * np.linalg.norm(o)
        assert np.linalg.norm(Sc - S) <= 1e-12 * np.linalg.norm(S)


def pin_forward_z_matches_gate_then_recurrence(orc):
    """The fused oracle entry (gate inside the token loop) equals gate() then
    recurrence() exactly."""
    rng = np.random.default_rng(24)
    B, T, H, dk, dv = 1, 20, 2, 5, 3
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) / 3
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk))
    A = rng.standard_normal((H, dk))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    o1, S1 = orc.forward_z(q, k, v, beta, z, A, -5.0)
    o2, S2 = orc.recurrence(q, k, v, beta, orc.gate(z, A, -5.0, 1))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def pin_replay(orc):
    """Draft replay ("architecture, derivations and a pinned-source audit" page,
    section 10.3, and its CPU laboratory): from a snapshot, the committed state is
    the state after the accepted prefix, the same as running those tokens from the
    start; rejecting drafts changes it; the snapshot is left as it was; every
    drafted token gets its output.  Checked against the pure-Python token loop."""
    rng = np.random.default_rng(23)
    n_draft, N, H, dk, dv = 6, 4, 2, 5, 4
    q = rng.standard_normal((n_draft, N, H, dk)) * 0.4
    k = rng.standard_normal((n_draft, N, H, dk)) * 0.4
    v = rng.standard_normal((n_draft, N, H, dv))
    z = rng.standard_normal((n_draft, N, H, dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((n_draft, N, H))))
    A = rng.standard_normal((H, dk)) * 0.5
    snap = rng.standard_normal((N, H, dk, dv)) * 0.3
    snap_copy = snap.copy()
    accepted = np.array([0, 2, 5, 6])
    o, S = orc.replay(q, k, v, z, beta, A, snap, accepted)
    assert np.array_equal(snap, snap_copy)              # snapshot untouched
    assert np.array_equal(S[0], snap[0])                # nothing accepted: the snapshot itself
    for n in range(N):
        for h in range(H):
            alpha = [brute.gate_alpha(z[t, n, h], A[h]) for t in range(n_draft)]
            ob, _ = brute.forward(q[:, n, h], k[:, n, h], v[:, n, h], beta[:, n, h], alpha, snap[n, h])
            np.testing.assert_allclose(o[:, n, h], np.array(ob), rtol=0, atol=1e-12)
            m = accepted[n]
            _, Sm = brute.forward(q[:m, n, h], k[:m, n, h], v[:m, n, h], beta[:m, n, h], alpha[:m], snap[n, h])
            np.testing.assert_allclose(S[n, h], np.array(Sm), rtol=0, atol=1e-12)
            if m < n_draft:                              # the rejected drafts would have moved the state
                _, Sall = brute.forward(q[:, n, h], k[:, n, h], v[:, n, h], beta[:, n, h], alpha, snap[n, h])
                assert not np.allclose(np.array(Sall), S[n, h])


# ----------------------------------------------------------------------------
# fused prologue: regularised L2 normalisation of q, k and beta from a logit
# ----------------------------------------------------------------------------
def pin_prologue_normalisation(orc):
    """Paper-and-proofs page, section 2.1.1 (Equations 2-6): the normalised
    vector keeps its direction, has norm strictly below one, and a zero
    vector stays zero; with the regulariser eps = 1e-6 under the root, the
    squared norm of the result is s / (s + eps) for s = |x|^2, so a vector of
    norm 1e-3 comes out with norm 1/sqrt(2), a large one with norm 1 - eps/(2s),
    and a tiny one is scaled by 1/sqrt(eps) = 1000.  Normalisation is per token
    row (the last axis), never across tokens."""
    import oracle as O
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 7, 2, 16))
    x *= 10.0 ** rng.uniform(-5, 3, (3, 7, 2, 1))
    x[1, 3, 0] = 0.0
    y = O.l2_normalise(x)
    assert np.array_equal(y[1, 3, 0], np.zeros(16))                     # zero stays zero
    n_in = np.linalg.norm(x, axis=-1)
    n_out = np.linalg.norm(y, axis=-1)
    assert np.all(n_out < 1.0)
    s = n_in ** 2
    np.testing.assert_allclose(n_out ** 2, s / (s + 1e-6), rtol=1e-13, atol=0)
    nz = n_in > 0
    cosine = np.sum(x * y, axis=-1)[nz] / (n_in[nz] * n_out[nz])
    np.testing.assert_allclose(cosine, 1.0, rtol=0, atol=1e-14)       # direction kept
    e = np.zeros(16)
    e[0] = 1e-3
    assert abs(np.linalg.norm(O.l2_normalise(e)) - 1.0 / math.sqrt(2.0)) < 1e-12
    e[0] = 1e4
    assert abs(O.l2_normalise(e)[0] - (1.0 - 0.5e-14)) < 1e-15
    e[0] = 1e-9
    assert abs(O.l2_normalise(e)[0] / 1e-9 - 1000.0) < 1e-6
    # rows are independent: scaling one token's row leaves the others unchanged
    x2 = x.copy()
    x2[0, 2, 1] *= 7.0
    y2 = O.l2_normalise(x2)
    mask = np.ones(x.shape[:-1], bool)
    mask[0, 2, 1] = False
    assert np.array_equal(y2[mask], y[mask])


def pin_prologue_beta(orc):
    """beta in (0, 1) ("architecture, derivations and a pinned-source audit",
    section 4.2) from its logit by the logistic sigmoid: 1/2 at 0, symmetric
    (sigma(-x) = 1 - sigma(x)), increasing, and inverted by the log-odds."""
    import oracle as O
    assert O.sigmoid(0.0) == 0.5
    x = np.linspace(-30, 30, 601)
    b = O.sigmoid(x)
    assert np.all((b > 0) & (b < 1)) and np.all(np.diff(b) > 0)
    np.testing.assert_allclose(O.sigmoid(-x) + b, 1.0, rtol=0, atol=1e-15)
    mid = np.abs(x) < 15
    np.testing.assert_allclose(np.log(b[mid] / (1 - b[mid])), x[mid], rtol=0, atol=1e-9)


def pin_prologue_forward(orc):
    """The prefill with the prologue fused: for rows of large norm the
    regulariser is negligible, so it equals the plain prefill on exactly
    unit-normalised q, k with beta = e^x / (1 + e^x) computed apart; scaling
    the raw rows by any factor above that regime changes nothing; and the
    decode form steps the same recurrence token by token."""
    rng = np.random.default_rng(43)
    B, T, H, dk, dv = 2, 9, 2, 6, 5
    q = rng.standard_normal((B, T, H, dk)) * 50.0
    k = rng.standard_normal((B, T, H, dk)) * 50.0
    v = rng.standard_normal((B, T, H, dv))
    bl = rng.standard_normal((B, T, H)) * 2.0
    z = rng.standard_normal((B, T, H, dk))
    A = rng.standard_normal((H, dk)) * 0.5
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    o, S = orc.forward_z_prologue(q, k, v, bl, z, A, -5.0, S0)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    ou, Su = orc.forward_z(unit(q), unit(k), v, np.exp(bl) / (1.0 + np.exp(bl)), z, A, -5.0, S0)
    np.testing.assert_allclose(o, ou, rtol=0, atol=1e-8)
    np.testing.assert_allclose(S, Su, rtol=0, atol=1e-8)
    o3, S3 = orc.forward_z_prologue(q * 1e3, k * 1e3, v, bl, z, A, -5.0, S0)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-9)
    np.testing.assert_allclose(S3, S, rtol=0, atol=1e-9)
    # decode form: [steps, N, H, ...] with the batch entries as sequences
    tm = lambda x: np.ascontiguousarray(np.moveaxis(x, 1, 0))
    od, Sd = orc.decode_prologue(tm(q), tm(k), tm(v), tm(z), tm(bl), A, S0)
    np.testing.assert_allclose(od, tm(o), rtol=0, atol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# backward (oracle.backward): the derivative of the forward
# ----------------------------------------------------------------------------
def _bwd_case(rng, B=2, T=7, H=2, dk=5, dv=4):
    q = rng.standard_normal((B, T, H, dk)) * 0.5
    k = rng.standard_normal((B, T, H, dk)) * 0.4
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    z = rng.standard_normal((B, T, H, dk))
    A = rng.standard_normal((H, dk)) * 0.5
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    return dict(q=q, k=k, v=v, beta=beta, z=z, A=A, S0=S0)


def pin_backward_finite_differences(orc):
    """Every gradient of the backward against central finite differences of the
    C forward (an independent implementation): for L = sum(w_o o) + sum(w_S S_T)
    and a random direction d in each input, (L(x + eps d) - L(x - eps d)) / 2 eps
    equals <grad, d>.  The CPU laboratory of "architecture, derivations and a
    pinned-source audit" checks its analytic state derivative the same way."""
    import oracle.backward as OB
    rng = np.random.default_rng(51)
    c = _bwd_case(rng)
    scale = 0.7
    o, S = orc.forward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], -5.0, c["S0"], scale)
    w_o = rng.standard_normal(o.shape)
    w_S = rng.standard_normal(S.shape)
    g = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], w_o, w_S, -5.0, c["S0"], scale)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "z": "dz", "A": "dA", "S0": "dS_in"}
    eps = 1e-6
    for x, gname in names.items():
        d = rng.standard_normal(c[x].shape)
        lo = dict(c)
        hi = dict(c)
        lo[x] = c[x] - eps * d
        hi[x] = c[x] + eps * d
        Lh = OB.loss(*orc.forward_z(hi["q"], hi["k"], hi["v"], hi["beta"], hi["z"], hi["A"], -5.0, hi["S0"], scale),
                     w_o, w_S)
        Ll = OB.loss(*orc.forward_z(lo["q"], lo["k"], lo["v"], lo["beta"], lo["z"], lo["A"], -5.0, lo["S0"], scale),
                     w_o, w_S)
        fd = (Lh - Ll) / (2 * eps)
        an = float(np.sum(g[gname] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (x, fd, an)


def pin_backward_state_derivative_printed(orc):
    """The CPU laboratory's analytic derivative ("architecture, derivations and a
    pinned-source audit"): for one step S_1 = M S_0 + U with M = (I - beta k k^T)
    Diag(alpha) and U = beta k v^T, the gradient of sum(S_1^2) with respect to S_0
    is 2 M^T (M S_0 + U)."""
    import oracle.backward as OB
    rng = np.random.default_rng(52)
    c = _bwd_case(rng, B=1, T=1, H=1, dk=4, dv=3)
    f = OB.forward_states(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], -5.0, c["S0"])
    S1 = f["S"][1]
    g = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], np.zeros((1, 1, 1, 3)), 2.0 * S1, -5.0,
                      c["S0"])
    k = c["k"][0, 0, 0]
    b = c["beta"][0, 0, 0]
    alpha = f["alpha"][0, 0, 0]
    M = (np.eye(4) - b * np.outer(k, k)) @ np.diag(alpha)
    U = b * np.outer(k, c["v"][0, 0, 0])
    expected = 2 * M.T @ (M @ c["S0"][0, 0] + U)
    np.testing.assert_allclose(g["dS_in"][0, 0], expected, rtol=0, atol=1e-13)


def pin_backward_autograd(orc):
    """Every gradient against torch's reverse-mode automatic differentiation (fp64,
    CPU) of the same forward written as plain tensor operations, and the
    backward's own forward against the C oracle."""
    import torch
    import oracle.backward as OB
    rng = np.random.default_rng(53)
    c = _bwd_case(rng, B=2, T=9, H=3, dk=6, dv=5)
    scale = 1.3
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in c.items()}
    S = t["S0"]
    outs = []
    for i in range(c["q"].shape[1]):
        a = torch.exp(-5.0 * torch.sigmoid(torch.exp(t["A"]) * t["z"][:, i]))     # [B, H, dk]
        D = a[..., None] * S
        e = t["v"][:, i] - torch.einsum("bhc,bhcj->bhj", t["k"][:, i], D)
        S = D + t["beta"][:, i, :, None, None] * t["k"][:, i, :, :, None] * e[:, :, None, :]
        outs.append(scale * torch.einsum("bhcj,bhc->bhj", S, t["q"][:, i]))
    o = torch.stack(outs, dim=1)
    w_o = torch.tensor(rng.standard_normal(tuple(o.shape)), dtype=torch.float64)
    w_S = torch.tensor(rng.standard_normal(tuple(S.shape)), dtype=torch.float64)
    (torch.sum(w_o * o) + torch.sum(w_S * S)).backward()
    g = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], w_o.numpy(), w_S.numpy(), -5.0, c["S0"],
                      scale)
    for n, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("z", "dz"), ("A", "dA"),
                     ("S0", "dS_in")):
        np.testing.assert_allclose(g[gname], t[n].grad.numpy(), rtol=0, atol=1e-11, err_msg=n)
    oc, Sc = orc.forward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], -5.0, c["S0"], scale)
    np.testing.assert_allclose(g["o"], oc, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["S_T"], Sc, rtol=0, atol=1e-12)


def pin_backward_special_cases(orc):
    """beta = 0 leaves only the decay, so nothing flows to v and k (dv = dk = 0);
    with every cotangent zero every gradient is zero; gradients are linear in
    the cotangents (do, dS_out)."""
    import oracle.backward as OB
    rng = np.random.default_rng(54)
    c = _bwd_case(rng)
    w1 = rng.standard_normal((2, 7, 2, 4))
    w2 = rng.standard_normal((2, 7, 2, 4))
    s1 = rng.standard_normal((2, 2, 5, 4))
    b0 = OB.backward_z(c["q"], c["k"], c["v"], np.zeros_like(c["beta"]), c["z"], c["A"], w1, s1, -5.0, c["S0"])
    assert np.array_equal(b0["dv"], np.zeros_like(c["v"])) and np.array_equal(b0["dk"], np.zeros_like(c["k"]))
    z0 = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], np.zeros_like(w1), None, -5.0, c["S0"])
    for key in ("dq", "dk", "dv", "dbeta", "dz", "dA", "dS_in"):
        assert np.array_equal(z0[key], np.zeros_like(z0[key]))
    ga = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], w1, s1, -5.0, c["S0"])
    gb = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], w2, None, -5.0, c["S0"])
    gs = OB.backward_z(c["q"], c["k"], c["v"], c["beta"], c["z"], c["A"], 2 * w1 - 3 * w2, 2 * s1, -5.0, c["S0"])
    for key in ("dq", "dk", "dv", "dbeta", "dz", "dA", "dS_in"):
        np.testing.assert_allclose(gs[key], 2 * ga[key] - 3 * gb[key], rtol=0, atol=1e-11)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
