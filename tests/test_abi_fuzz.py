"""Property-based checks of the C ABI's host validation (CPU only).

Every entry point is called with arguments drawn from mixes of valid, boundary
and invalid values (sizes, dtype codes, floats, and fake device addresses:
NULL, aligned, misaligned, or the same address as another argument).  For any
combination the call must return one of the documented status codes without
stopping the process; a bad dtype code is reported as KDA_ERR_DTYPE; and KDA_OK
never comes back for a negative size or an unknown dtype.

The fake addresses are never valid memory.  On this container a call that
passes validation fails at its first HIP call and returns KDA_ERR_HIP; where a
GPU is visible the test does not run, since such a call would launch kernels
on them.
"""
import ctypes
import math

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import gated_delta_rule_11_amd as kda  # noqa: E402

# status codes (include/kda.h): 0 on success, negative on error
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_ALIAS, ERR_ALIGN = 0, -1, -2, -3, -4, -5, -6, -7, -8
STATUSES = (OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_ALIAS, ERR_ALIGN)


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses must not reach a real launch")

SIZES = st.sampled_from([-(1 << 31), -3, -1, 0, 1, 2, 3, 7, 16, 17, 64, 100, 1 << 20, (1 << 31) - 1])
DIMS = st.sampled_from([-16, -1, 0, 1, 8, 16, 24, 32, 48, 64, 96, 128, 256, 1 << 30])
CHUNKS = st.sampled_from([-64, 0, 1, 15, 16, 32, 64, 128])
DTYPES = st.sampled_from([-1, 0, 1, 2, 1 << 20])
FLOATS = st.sampled_from([-math.inf, -6.0, -5.5, -5.4, -5.0, -1.0, -0.0, 0.0, 0.5, 1.0, math.inf, math.nan])
SCALES = st.sampled_from([1.0, 0.0, -2.0, 1e30, math.inf, math.nan])


@st.composite
def pointers(draw, n):
    """n fake device addresses: NULL, 16-byte aligned and far apart, misaligned, or
    another argument's address."""
    out = []
    for i in range(n):
        kind = draw(st.sampled_from(["aligned", "aligned", "aligned", "null", "odd", "same"]))
        base = 0x10000000 * (i + 1)
        if kind == "null":
            out.append(None)
        elif kind == "odd":
            out.append(ctypes.c_void_p(base + draw(st.sampled_from([1, 2, 4, 8]))))
        elif kind == "same" and i > 0:
            out.append(out[draw(st.integers(0, i - 1))])
        else:
            out.append(ctypes.c_void_p(base))
    return out


@pytest.fixture(scope="module")
def L():
    from gated_delta_rule_11_amd import _build
    if _build.is_stale():
        _build.build()
    return kda.lib()


def _check(status, dtypes, sizes):
    assert status in STATUSES, status
    if any(t not in (0, 1) for t in dtypes):
        assert status == ERR_DTYPE, status
    if status == OK:
        assert all(s >= 0 for s in sizes)


FUZZ = settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])


@FUZZ
@given(p=pointers(3), zt=DTYPES, gmin=FLOATS, B=SIZES, T=SIZES, H=SIZES, dk=DIMS, chunk=CHUNKS)
def test_fuzz_gate(L, p, zt, gmin, B, T, H, dk, chunk):
    s = L.kda_gate(p[0], zt, p[1], gmin, B, T, H, dk, chunk, p[2], None)
    _check(s, [zt], [B, T, H])


WSB = st.sampled_from([0, 16, 1 << 20, 1 << 40])


@FUZZ
@given(p=pointers(10), it=DTYPES, ot=DTYPES, gmin=FLOATS, scale=SCALES, B=SIZES, T=SIZES, H=SIZES, dk=DIMS,
       dv=DIMS, chunk=CHUNKS, fused=st.booleans(), wsb=WSB)
def test_fuzz_chunk(L, p, it, ot, gmin, scale, B, T, H, dk, dv, chunk, fused, wsb):
    need = L.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk)
    if fused:
        s = L.kda_chunk_fwd_z(p[0], p[1], p[2], p[3], p[4], it, p[5], gmin, p[6], p[7], ot, p[8], B, T, H, dk, dv,
                              chunk, scale, p[9], wsb, None)
    else:
        s = L.kda_chunk_fwd(p[0], p[1], p[2], p[3], it, p[4], p[6], p[7], ot, p[8], B, T, H, dk, dv, chunk, scale,
                            p[9], wsb, None)
    _check(s, [it, ot], [B, T, H])
    if s == OK and B > 0 and H > 0:
        assert wsb >= need


@FUZZ
@given(p=pointers(8), it=DTYPES, ot=DTYPES, gmin=FLOATS, scale=SCALES, Nn=SIZES, H=SIZES, dk=DIMS, dv=DIMS,
       prologue=st.booleans())
def test_fuzz_decode(L, p, it, ot, gmin, scale, Nn, H, dk, dv, prologue):
    f = L.kda_decode_step_prologue if prologue else L.kda_decode_step
    s = f(p[0], p[1], p[2], p[3], p[4], it, p[5], gmin, p[6], p[7], ot, Nn, H, dk, dv, scale, None)
    _check(s, [it, ot], [Nn, H])


@FUZZ
@given(p=pointers(10), it=DTYPES, ot=DTYPES, gmin=FLOATS, scale=SCALES, nd=SIZES, Nn=SIZES, H=SIZES, dk=DIMS,
       dv=DIMS)
def test_fuzz_replay(L, p, it, ot, gmin, scale, nd, Nn, H, dk, dv):
    s = L.kda_decode_replay(p[0], p[1], p[2], p[3], p[4], it, p[5], gmin, p[6], p[7], p[8], ot, p[9], nd, Nn, H, dk,
                            dv, scale, None)
    _check(s, [it, ot], [nd, Nn, H])


@FUZZ
@given(p=pointers(10), it=DTYPES, ot=DTYPES, gmin=FLOATS, scale=SCALES, B=SIZES, T=SIZES, H=SIZES, dk=DIMS,
       dv=DIMS, chunk=CHUNKS, segs=SIZES, wsb=st.sampled_from([0, 16, 1 << 20, 1 << 40]))
def test_fuzz_segmented(L, p, it, ot, gmin, scale, B, T, H, dk, dv, chunk, segs, wsb):
    L.kda_chunk_fwd_z_segmented_workspace_bytes(B, H, dk, dv, segs)
    s = L.kda_chunk_fwd_z_segmented(p[0], p[1], p[2], p[3], p[4], it, p[5], gmin, p[6], p[7], ot, p[8], B, T, H, dk,
                                    dv, chunk, scale, segs, p[9], wsb, None)
    _check(s, [it, ot], [B, T, H])


@FUZZ
@given(p=pointers(10), it=DTYPES, ot=DTYPES, gmin=FLOATS, scale=SCALES, B=SIZES, T=SIZES, H=SIZES, dk=DIMS,
       dv=DIMS, chunk=CHUNKS, wsb=WSB)
def test_fuzz_prologue(L, p, it, ot, gmin, scale, B, T, H, dk, dv, chunk, wsb):
    s = L.kda_chunk_fwd_z_prologue(p[0], p[1], p[2], p[3], p[4], it, p[5], gmin, p[6], p[7], ot, p[8], B, T, H, dk,
                                   dv, chunk, scale, p[9], wsb, None)
    _check(s, [it, ot], [B, T, H])


@FUZZ
@given(p=pointers(16), it=DTYPES, dt=DTYPES, gmin=FLOATS, scale=SCALES, B=SIZES, T=SIZES, H=SIZES, dk=DIMS,
       dv=DIMS, wsb=st.sampled_from([0, 16, 1 << 20, 1 << 40]))
def test_fuzz_backward(L, p, it, dt, gmin, scale, B, T, H, dk, dv, wsb):
    L.kda_chunk_bwd_z_workspace_bytes(B, T, H, dk, dv)
    s = L.kda_chunk_bwd_z(p[0], p[1], p[2], p[3], p[4], it, p[5], gmin, p[6], p[7], dt, p[8], p[9], p[10], p[11],
                          p[12], p[13], p[14], p[15], B, T, H, dk, dv, scale, p[0], wsb, None)
    _check(s, [it, dt], [B, T, H])
