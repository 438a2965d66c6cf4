"""The C ABI on the CPU: libkda.so loads, exports every symbol include/kda.h
declares, and rejects bad arguments on the host without launching anything
(no compute call is made here: every call below fails validation or has
nothing to do)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_11_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

# status codes: 0 on success, negative on error (include/kda.h)
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_ALIAS, ERR_ALIGN = 0, -1, -2, -3, -4, -5, -6, -7, -8
STATUSES = (OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_ALIAS, ERR_ALIGN)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def L():
    from gated_delta_rule_11_amd import _build
    if _build.is_stale():
        _build.build()
    return kda.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_gate", "kda_chunk_fwd", "kda_chunk_fwd_z", "kda_decode_step", "kda_decode_replay",
              "kda_chunk_fwd_z_prologue", "kda_decode_step_prologue", "kda_chunk_fwd_z_segmented",
              "kda_chunk_bwd_z",
              "kda_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_codes_match_the_header(L):
    """The numeric values above are the header's (the contract is negative codes)."""
    text = open(HEADER).read()
    names = {"OK": OK, "ERR_NULL": ERR_NULL, "ERR_SHAPE": ERR_SHAPE, "ERR_DTYPE": ERR_DTYPE,
             "ERR_WORKSPACE": ERR_WORKSPACE, "ERR_UNSUPPORTED": ERR_UNSUPPORTED, "ERR_HIP": ERR_HIP,
             "ERR_ALIAS": ERR_ALIAS, "ERR_ALIGN": ERR_ALIGN}
    for n, val in names.items():
        m = re.search(r"\bKDA_" + n + r"\s*=\s*(-?\d+)", text)
        assert m and int(m.group(1)) == val, n
        assert L.kda_status_string(val).decode().startswith("KDA_" + n)


def test_status_strings(L):
    for s in STATUSES:
        assert L.kda_status_string(s).decode().startswith("KDA_")
    assert b"unknown" in L.kda_status_string(99)
    assert b"unknown" in L.kda_status_string(1)
    assert L.kda_version() >= 200


# Fake device addresses: validation must reject before any of them is used.
def P(i):
    return ctypes.c_void_p(0x10000000 * (i + 1))


N = None


def gate(L, z=P(0), zt=BF16, A=P(1), gmin=-5.0, B=1, T=64, H=2, dk=128, chunk=64, G=P(2)):
    return L.kda_gate(z, zt, A, gmin, B, T, H, dk, chunk, G, N)


def chunk(L, q=P(0), k=P(1), v=P(2), beta=P(3), it=BF16, G=P(4), S_in=P(5), o=P(6), ot=BF16, S_out=P(7),
          B=1, T=64, H=2, dk=128, dv=128, c=64, scale=1.0, ws=None, wsb=0):
    return L.kda_chunk_fwd(q, k, v, beta, it, G, S_in, o, ot, S_out, B, T, H, dk, dv, c, scale, ws, wsb, N)


def chunk_z(L, q=P(0), k=P(1), v=P(2), beta=P(3), z=P(4), it=BF16, A=P(8), gmin=-5.0, S_in=P(5), o=P(6), ot=BF16,
            S_out=P(7), B=1, T=64, H=2, dk=128, dv=128, c=64, scale=1.0, ws=None, wsb=0):
    return L.kda_chunk_fwd_z(q, k, v, beta, z, it, A, gmin, S_in, o, ot, S_out, B, T, H, dk, dv, c, scale, ws, wsb,
                             N)


def decode(L, q=P(0), k=P(1), v=P(2), z=P(3), beta=P(4), it=BF16, A=P(5), gmin=-5.0, S=P(6), o=P(7), ot=BF16,
           Nn=4, H=2, dk=128, dv=128, scale=1.0):
    return L.kda_decode_step(q, k, v, z, beta, it, A, gmin, S, o, ot, Nn, H, dk, dv, scale, N)


def test_gate_validation(L):
    assert gate(L, zt=7) == ERR_DTYPE
    assert gate(L, B=-1) == ERR_SHAPE
    assert gate(L, T=-5) == ERR_SHAPE
    assert gate(L, H=0) == ERR_SHAPE
    assert gate(L, dk=48) == ERR_UNSUPPORTED
    assert gate(L, chunk=32) == ERR_UNSUPPORTED
    assert gate(L, gmin=1.0) == ERR_UNSUPPORTED
    assert gate(L, gmin=float("nan")) == ERR_UNSUPPORTED
    assert gate(L, gmin=-5.5) == ERR_UNSUPPORTED     # 16 g_min >= -80: tile decays stay normal fp32
    assert gate(L, gmin=-5.01) == ERR_UNSUPPORTED
    assert gate(L, gmin=-5.0, z=None) == ERR_NULL    # the floor itself is accepted
    assert gate(L, z=None) == ERR_NULL
    assert gate(L, G=None) == ERR_NULL
    assert gate(L, A=None) == ERR_NULL
    assert gate(L, G=P(0)) == ERR_ALIAS          # G overlaps z
    assert gate(L, G=ctypes.c_void_p(0x30000008)) == ERR_ALIGN
    assert gate(L, B=0) == OK                    # nothing to do, nothing launched
    assert gate(L, T=0, z=None, G=None) == OK


def test_chunk_validation(L):
    assert chunk(L, it=3) == ERR_DTYPE
    assert chunk(L, ot=-1) == ERR_DTYPE
    assert chunk(L, B=-1) == ERR_SHAPE
    assert chunk(L, T=-1) == ERR_SHAPE
    assert chunk(L, H=0) == ERR_SHAPE
    assert chunk(L, B=1 << 20, H=1 << 12) == ERR_SHAPE
    assert chunk(L, dk=96) == ERR_UNSUPPORTED
    assert chunk(L, dv=256) == ERR_UNSUPPORTED
    assert chunk(L, c=32) == ERR_UNSUPPORTED
    assert chunk(L, c=1) == ERR_UNSUPPORTED
    assert chunk(L, scale=float("inf")) == ERR_UNSUPPORTED
    for name in ("q", "k", "v", "beta", "G", "o"):
        assert chunk(L, **{name: None}) == ERR_NULL, name
    assert chunk(L, o=P(0)) == ERR_ALIAS                 # o overlaps q
    assert chunk(L, S_out=P(4)) == ERR_ALIAS             # S_out overlaps G
    assert chunk(L, S_out=ctypes.c_void_p(0x60000000 + 256)) == ERR_ALIAS  # partial overlap with S_in
    assert chunk(L, S_in=ctypes.c_void_p(0x60000004)) == ERR_ALIGN
    assert chunk(L, q=ctypes.c_void_p(0x10000002)) == ERR_ALIGN
    assert chunk(L, beta=ctypes.c_void_p(0x40000001)) == ERR_ALIGN
    # a 2-byte-aligned bf16 beta passes the alignment check (and then fails on the overlap)
    assert chunk(L, beta=ctypes.c_void_p(0x40000002), o=P(0)) == ERR_ALIAS
    assert chunk(L, B=0) == OK
    assert chunk_z(L, gmin=-6.0) == ERR_UNSUPPORTED
    assert chunk_z(L, gmin=-5.5) == ERR_UNSUPPORTED
    assert chunk_z(L, gmin=-5.4) == ERR_UNSUPPORTED
    assert chunk_z(L, gmin=-5.0, q=None) == ERR_NULL
    assert chunk_z(L, gmin=0.5) == ERR_UNSUPPORTED
    assert chunk_z(L, z=None) == ERR_NULL
    assert chunk_z(L, A=None) == ERR_NULL
    assert chunk_z(L, o=P(4)) == ERR_ALIAS               # o overlaps z
    assert chunk_z(L, B=0) == OK


def test_decode_validation(L):
    assert decode(L, it=2) == ERR_DTYPE
    assert decode(L, Nn=-1) == ERR_SHAPE
    assert decode(L, dk=8) == ERR_UNSUPPORTED
    assert decode(L, gmin=3.0) == ERR_UNSUPPORTED
    for name in ("q", "k", "v", "z", "beta", "A", "S", "o"):
        assert decode(L, **{name: None}) == ERR_NULL, name
    assert decode(L, o=P(6)) == ERR_ALIAS                # o overlaps S
    assert decode(L, S=P(2)) == ERR_ALIAS                # S overlaps v
    assert decode(L, S=ctypes.c_void_p(0x70000008)) == ERR_ALIGN
    assert decode(L, Nn=0) == OK


def test_binding_refuses_cpu_tensors(L):
    import torch
    z = torch.zeros(1, 4, 1, 16)
    A = torch.zeros(1, 16)
    with pytest.raises(kda.KDAError):
        kda.gate(z, A, chunk=1, out=torch.zeros(1, 4, 1, 16))


def test_binding_checks_shapes_and_dtypes():
    """The library takes raw pointers and trusts the sizes it is given; the binding
    refuses tensors whose shape or dtype disagree with the call before passing a
    pointer (checked with CPU tensors: the shape check comes first)."""
    import torch
    B, T, H, dk, dv = 1, 8, 2, 16, 32
    q = torch.zeros(B, T, H, dk, dtype=torch.bfloat16)
    v = torch.zeros(B, T, H, dv, dtype=torch.bfloat16)
    beta = torch.zeros(B, T, H, dtype=torch.bfloat16)
    A = torch.zeros(H, dk)
    cases = [
        (lambda: kda.gate(q, A, out=torch.zeros(B, T, H, dk - 1)), "out has shape"),
        (lambda: kda.gate(q, A.bfloat16()), "A has dtype"),
        (lambda: kda.chunk_fwd_z(q, q[:, :4], v, beta, q, A), "k has shape"),
        (lambda: kda.chunk_fwd_z(q, q.float(), v, beta, q, A), "k has dtype"),
        (lambda: kda.chunk_fwd_z(q, q, v, beta[..., :1], q, A), "beta has shape"),
        (lambda: kda.chunk_fwd_z(q, q, v, beta, q, A, S_in=torch.zeros(B, H, dv, dk)), "S_in has shape"),
        (lambda: kda.chunk_fwd_z(q, q, v, beta, q, A, o=torch.zeros(B, T, H, dk)), "o has shape"),
        (lambda: kda.chunk_fwd(q, q, v, beta, q, 16), "G has dtype"),
        (lambda: kda.chunk_bwd_z(q, q, v, beta, q, A, q), "d_o has shape"),
        (lambda: kda.decode_step(q[0], q[0], v[0], q[0], beta[0], A, torch.zeros(T, H, dk, dk)), "S has shape"),
        (lambda: kda.decode_replay(q, q, v, q, beta, A, torch.zeros(T, H, dk, dv), torch.zeros(T, dtype=torch.int64)),
         "accepted has dtype"),
    ]
    for call, msg in cases:
        with pytest.raises(kda.KDAError, match=msg):
            call()


def replay(L, q=P(0), k=P(1), v=P(2), z=P(3), beta=P(4), it=BF16, A=P(5), gmin=-5.0, S_snap=P(6),
           acc=P(7), o=P(8), ot=BF16, S_commit=P(9), n_draft=4, Nn=4, H=2, dk=128, dv=128, scale=1.0):
    return L.kda_decode_replay(q, k, v, z, beta, it, A, gmin, S_snap, acc, o, ot, S_commit, n_draft, Nn, H, dk, dv,
                               scale, N)


def test_replay_validation(L):
    assert replay(L, it=5) == ERR_DTYPE
    assert replay(L, n_draft=-1) == ERR_SHAPE
    assert replay(L, Nn=-2) == ERR_SHAPE
    assert replay(L, dv=48) == ERR_UNSUPPORTED
    assert replay(L, gmin=0.5) == ERR_UNSUPPORTED
    for name in ("A", "S_snap", "acc", "S_commit", "q", "k", "v", "z", "beta", "o"):
        assert replay(L, **{name: None}) == ERR_NULL, name
    # with nothing drafted only the state buffers and accepted are needed (still rejected on overlap)
    assert replay(L, n_draft=0, q=None, k=None, v=None, z=None, beta=None, o=None, S_commit=P(6)) == ERR_ALIAS
    assert replay(L, S_commit=P(6)) == ERR_ALIAS      # commit over the snapshot
    assert replay(L, o=P(7)) == ERR_ALIAS             # output over accepted
    assert replay(L, S_commit=P(8)) == ERR_ALIAS      # commit over the output
    assert replay(L, acc=ctypes.c_void_p(0x80000002)) == ERR_ALIGN
    assert replay(L, S_snap=ctypes.c_void_p(0x70000008)) == ERR_ALIGN
    assert replay(L, Nn=0) == OK



def chunk_seg(L, segs=4, ws=P(10), wsb=1 << 30, B=1, T=1024, H=2, c=64, it=BF16, dk=128, **kw):
    args = dict(q=P(0), k=P(1), v=P(2), beta=P(3), z=P(4), A=P(8), S_in=P(5), o=P(6), S_out=P(7))
    args.update(kw)
    return L.kda_chunk_fwd_z_segmented(args["q"], args["k"], args["v"], args["beta"], args["z"], it, args["A"], -5.0,
                                       args["S_in"], args["o"], BF16, args["S_out"], B, T, H, dk, 128, c, 1.0,
                                       segs, ws, wsb, N)


def test_segmented_validation(L):
    need = L.kda_chunk_fwd_z_segmented_workspace_bytes(1, 2, 128, 128, 4)
    # end states and transitions of every segment but the last, entry states of all
    assert need == 1 * 2 * (3 * (128 * 128 + 128 * 128) + 4 * 128 * 128) * 4
    assert L.kda_chunk_fwd_z_segmented_workspace_bytes(1, 2, 128, 128, 1) == 0
    assert L.kda_chunk_fwd_z_segmented_workspace_bytes(1, 2, 128, 128, 0) == 0
    assert chunk_seg(L, segs=0) == ERR_SHAPE
    assert chunk_seg(L, ws=None) == ERR_NULL
    assert chunk_seg(L, wsb=need - 4) == ERR_WORKSPACE
    assert chunk_seg(L, ws=ctypes.c_void_p(0xa0000008)) == ERR_ALIGN
    assert chunk_seg(L, ws=P(6)) == ERR_ALIAS                     # workspace over the output
    # every shape and dtype takes segments (these get past validation; without a GPU
    # they stop at their first HIP call)
    assert chunk_seg(L, it=F32) == ERR_HIP
    assert chunk_seg(L, dk=64, wsb=L.kda_chunk_fwd_z_segmented_workspace_bytes(1, 2, 64, 128, 4)) == ERR_HIP
    assert chunk_seg(L, dk=48) == ERR_UNSUPPORTED
    assert chunk_seg(L, B=0) == OK


def test_prologue_validation(L):
    """The fused-prologue entry points validate exactly as the plain ones."""
    def chunk(**kw):
        a = dict(q=P(0), k=P(1), v=P(2), beta=P(3), z=P(4), A=P(8), S_in=P(5), o=P(6), S_out=P(7), B=1, T=100,
                 H=2, dk=128, dv=128, chunk=64, it=BF16, gmin=-5.0)
        a.update(kw)
        return L.kda_chunk_fwd_z_prologue(a["q"], a["k"], a["v"], a["beta"], a["z"], a["it"], a["A"], a["gmin"],
                                          a["S_in"], a["o"], BF16, a["S_out"], a["B"], a["T"], a["H"], a["dk"],
                                          a["dv"], a["chunk"], 1.0, None, 0, N)
    assert chunk(q=None) == ERR_NULL
    assert chunk(dk=48) == ERR_UNSUPPORTED
    assert chunk(chunk=32) == ERR_UNSUPPORTED
    assert chunk(it=7) == ERR_DTYPE
    assert chunk(o=P(2)) == ERR_ALIAS
    assert chunk(gmin=1.0) == ERR_UNSUPPORTED
    assert chunk(B=0) == OK

    def dec(**kw):
        a = dict(q=P(0), k=P(1), v=P(2), z=P(3), beta=P(4), A=P(5), S=P(6), o=P(7), N=4, H=2, dk=128, dv=128)
        a.update(kw)
        return L.kda_decode_step_prologue(a["q"], a["k"], a["v"], a["z"], a["beta"], BF16, a["A"], -5.0, a["S"],
                                          a["o"], BF16, a["N"], a["H"], a["dk"], a["dv"], 1.0, N)
    assert dec(beta=None) == ERR_NULL
    assert dec(dv=24) == ERR_UNSUPPORTED
    assert dec(o=P(6)) == ERR_ALIAS
    assert dec(N=0) == OK


def test_backward_validation(L):
    # checkpoints + scratch, dA parts and the recompute's M and AL (3 sub-chunks x 2 x 16 x 16)
    # per (b, h, slice); two value slices add their key-side parts into the outputs themselves
    mc = 3 * 2 * 16 * 16
    need = L.kda_chunk_bwd_z_workspace_bytes(2, 100, 3, 64, 32)
    assert need == (2 * 3 * (2 + 3) * 64 * 32 + 2 * 3 * 64 + 2 * 3 * mc) * 4      # one value slice at dv = 32
    two = L.kda_chunk_bwd_z_workspace_bytes(2, 100, 3, 64, 64)
    assert two == (2 * 3 * (2 + 3) * 64 * 64 + 2 * 3 * 2 * 64 + 2 * 3 * 2 * mc) * 4

    def bwd(**kw):
        a = dict(q=P(0), k=P(1), v=P(2), beta=P(3), z=P(4), A=P(5), S_in=None, do=P(6), dS_out=None, dq=P(7),
                 dk=P(8), dv=P(9), dbeta=P(10), dz=P(11), dA=P(12), dS_in=None, B=2, T=100, H=3, dk_=64, dv_=32,
                 gmin=-5.0, ws=P(13), wsb=need, it=F32)
        a.update(kw)
        return L.kda_chunk_bwd_z(a["q"], a["k"], a["v"], a["beta"], a["z"], a["it"], a["A"], a["gmin"], a["S_in"],
                                 a["do"], F32, a["dS_out"], a["dq"], a["dk"], a["dv"], a["dbeta"], a["dz"], a["dA"],
                                 a["dS_in"], a["B"], a["T"], a["H"], a["dk_"], a["dv_"], 1.0, a["ws"], a["wsb"], N)
    assert bwd(dq=None) == ERR_NULL
    assert bwd(ws=None) == ERR_NULL
    assert bwd(wsb=need - 4) == ERR_WORKSPACE
    assert bwd(gmin=-5.5) == ERR_UNSUPPORTED       # the backward needs 16 g_min >= -80
    assert bwd(dk_=48) == ERR_UNSUPPORTED
    assert bwd(dq=P(0)) == ERR_ALIAS               # gradient over an input
    assert bwd(dk=P(7)) == ERR_ALIAS               # two gradients on one buffer
    assert bwd(ws=P(11)) == ERR_ALIAS              # workspace over a gradient
    assert bwd(B=0) == OK


def test_zero_head_dims_rejected(L):
    """A head dim (or H, N) of zero is a shape error on every entry point.  The size
    checks divide by the head dims, so a zero once stopped the caller's process with
    an integer division by zero instead of returning a status."""
    for kw in ({"dk": 0}, {"dk": 0, "T": 0}):
        assert gate(L, **kw) == ERR_SHAPE, kw
    for kw in ({"dk": 0}, {"dv": 0}, {"dk": 0, "dv": 0}, {"dv": 0, "T": 0}):
        assert chunk(L, **kw) == ERR_SHAPE, kw
        assert chunk_z(L, **kw) == ERR_SHAPE, kw
    for kw in ({"dk": 0}, {"dv": 0}, {"H": 0}):
        assert decode(L, **kw) == ERR_SHAPE, kw
        assert replay(L, **kw) == ERR_SHAPE, kw
    assert chunk_seg(L, dk=0) == ERR_SHAPE
    assert L.kda_chunk_fwd_z_prologue(P(0), P(1), P(2), P(3), P(4), BF16, P(8), -5.0, P(5), P(6), BF16, P(7), 1, 100,
                                      2, 128, 0, 64, 1.0, None, 0, N) == ERR_SHAPE
    assert L.kda_decode_step_prologue(P(0), P(1), P(2), P(3), P(4), BF16, P(5), -5.0, P(6), P(7), BF16, 4, 2, 0, 128,
                                      1.0, N) == ERR_SHAPE
    assert L.kda_chunk_bwd_z(P(0), P(1), P(2), P(3), P(4), F32, P(5), -5.0, None, P(6), F32, None, P(7), P(8), P(9),
                             P(10), P(11), P(12), None, 2, 100, 3, 0, 32, 1.0, P(13), 1 << 30, N) == ERR_SHAPE


def test_token_count_limit(L):
    """T (and n_draft) is at most 2^31 - 65: the kernels round token offsets up to a
    whole chunk in 32 bits.  Just below the limit the sizes pass (the calls below
    then stop at a NULL pointer, before anything launches)."""
    big = (1 << 31) - 65
    small = dict(B=1, H=1, dk=16, dv=16)
    assert chunk(L, T=big + 1, **small) == ERR_SHAPE
    assert chunk(L, T=big, q=None, **small) == ERR_NULL
    assert chunk_z(L, T=big + 1, **small) == ERR_SHAPE
    assert gate(L, T=big + 1, B=1, H=1, dk=16) == ERR_SHAPE
    assert gate(L, T=big, B=1, H=1, dk=16, z=None) == ERR_NULL
    assert replay(L, n_draft=big + 1, Nn=1, H=1, dk=16, dv=16) == ERR_SHAPE
    assert replay(L, n_draft=big, Nn=1, H=1, dk=16, dv=16, q=None) == ERR_NULL


def test_chunk_workspace_query_and_validation(L):
    """kda_chunk_fwd_workspace_bytes sizes the workspace of the three chunked-prefill
    entry points from the sizes alone; a call with less returns KDA_ERR_WORKSPACE,
    with none KDA_ERR_NULL, and the workspace is checked for alignment and overlap."""
    q = L.kda_chunk_fwd_workspace_bytes
    assert q(4, 32768, 32, 128, 128, 64) == 0       # B*H = 128 fills the GPU in one pass
    assert q(1, 64, 8, 128, 128, 64) == 0           # a single chunk: nothing to split
    assert q(4, 4096, 64, 64, 64, 64) == 0          # B*H = 256 fills the GPU at d_v = 64
    assert q(1, 4096, 32, 64, 64, 64) > 0           # B*H = 32 at d_v = 64: eight segments
    assert q(1, 4096, 8, 128, 128, 16) == q(1, 4096, 8, 128, 128, 64)  # 256-token segments either way
    few = q(1, 4096, 8, 128, 128, 64)               # B*H = 8, 64 chunks: segment-parallel
    assert few > 0 and few % 16 == 0
    assert q(1, 1 << 20, 8, 128, 128, 64) >= few
    for bad in ((-1, 64, 8, 128, 128, 64), (1, -1, 8, 128, 128, 64), (1, 64, 0, 128, 128, 64),
                (1, 64, 8, 96, 128, 64), (1, 64, 8, 128, 128, 32)):
        assert q(*bad) == 0, bad
    kw = dict(B=1, T=4096, H=8)
    for call in (chunk, chunk_z):
        assert call(L, **kw) == ERR_NULL                               # no workspace at all
        assert call(L, ws=P(10), wsb=few - 4, **kw) == ERR_WORKSPACE   # too small
        assert call(L, ws=ctypes.c_void_p(0xb0000008), wsb=few, **kw) == ERR_ALIGN
        assert call(L, ws=P(6), wsb=few, **kw) == ERR_ALIAS            # over the output
        assert call(L, ws=P(7), wsb=few, **kw) == ERR_ALIAS            # over the final state
        assert call(L, ws=P(10), wsb=few, B=0, T=4096, H=8) == OK      # nothing to do
    # where none is needed, a NULL workspace of zero bytes is valid (the call then
    # gets past validation; without a GPU it stops at its first HIP call)
    assert chunk_z(L, ws=None, wsb=0, B=4, T=64, H=32) == ERR_HIP


def noalloc(L, q=P(0), k=P(1), v=P(2), beta=P(3), z=P(4), it=BF16, A=P(8), gmin=-5.0, S_in=P(5), o=P(6), ot=BF16,
            S_out=P(7), B=1, T=4096, H=8, dk=128, dv=128, c=64, scale=1.0):
    return L.kda_chunk_fwd_z_noalloc(q, k, v, beta, z, it, A, gmin, S_in, o, ot, S_out, B, T, H, dk, dv, c, scale, N)


def test_noalloc_validation(L):
    """The allocation-free prefill validates as kda_chunk_fwd_z, before it looks up
    its static scratch array (so every error below comes without a HIP call)."""
    assert L.kda_chunk_fwd_workspace_bytes(1, 4096, 8, 128, 128, 64) > 0  # these sizes use the scratch
    assert noalloc(L, it=9) == ERR_DTYPE
    assert noalloc(L, T=-1) == ERR_SHAPE
    assert noalloc(L, dk=48) == ERR_UNSUPPORTED
    assert noalloc(L, gmin=-5.5) == ERR_UNSUPPORTED
    for name in ("q", "k", "v", "beta", "z", "A", "o"):
        assert noalloc(L, **{name: None}) == ERR_NULL, name
    assert noalloc(L, o=P(4)) == ERR_ALIAS
    assert noalloc(L, q=ctypes.c_void_p(0x10000004)) == ERR_ALIGN
    assert noalloc(L, B=0) == OK
