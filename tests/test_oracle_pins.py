"""The fp64 oracle against printed values, closed forms, special cases,
invariants and brute force (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_decode_protocol_equals_prefill():
    """Decode steps carry the state token by token: 6 steps of the decode
    protocol equal one 6-token prefill per sequence, bitwise in fp64."""
    rng = np.random.default_rng(3)
    steps, N, H, dk, dv = 6, 3, 2, 5, 4
    q = rng.standard_normal((steps, N, H, dk))
    k = rng.standard_normal((steps, N, H, dk)) / 3
    v = rng.standard_normal((steps, N, H, dv))
    z = rng.standard_normal((steps, N, H, dk))
    beta = rng.uniform(0.1, 0.9, (steps, N, H))
    A = rng.standard_normal((H, dk))
    S0 = rng.standard_normal((N, H, dk, dv))
    od, Sd = oracle.decode(q, k, v, z, beta, A, S0)
    tm = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 1))  # [steps, N, ...] -> [N, steps, ...]
    op, Sp = oracle.forward_z(tm(q), tm(k), tm(v), tm(beta), tm(z), A, -5.0, S0)
    assert np.array_equal(od, np.moveaxis(op, 1, 0)) and np.array_equal(Sd, Sp)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(4)
    B, T, H, dk, dv = 2, 33, 3, 8, 40
    q, k, z = (rng.standard_normal((B, T, H, dk)) for _ in range(3))
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    A = rng.standard_normal((H, dk))
    o1, S1 = oracle.forward_z(q, k, v, beta, z, A, nthreads=1)
    o2, S2 = oracle.forward_z(q, k, v, beta, z, A, nthreads=7)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_state_aliasing_and_empty():
    rng = np.random.default_rng(6)
    B, T, H, dk, dv = 1, 0, 2, 4, 3
    S0 = rng.standard_normal((B, H, dk, dv))
    e = np.zeros((B, T, H, dk))
    o, S = oracle.forward_z(e, e, np.zeros((B, T, H, dv)), np.zeros((B, T, H)), e,
                            rng.standard_normal((H, dk)), -5.0, S0)
    assert o.shape == (B, 0, H, dv) and np.array_equal(S, S0)
