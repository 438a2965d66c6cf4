"""Every kernel writes only inside its output buffers.

Each output (and each caller workspace) is carved out of a larger device buffer
whose 4 KiB on either side are filled with a sentinel byte; after the call and a
synchronisation the guards must still hold the sentinel.  Ragged token counts
(the last chunk partial) run under every launch form of the chunked prefill --
two, four and eight value-column slices per head, the fp32 vector-ALU kernel,
the segment-parallel form (explicit and chosen by the library) -- and under the
draft replay, the gate, the decode step and the backward pass.  The results are
also compared with unguarded outputs of the same call, bit for bit."""
import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
from tests._gpu import DEV, dev_inputs, say

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0xA5
ESIZE = {torch.float32: 4, torch.bfloat16: 2, torch.uint8: 1, torch.int32: 4}


class Guarded:
    """A tensor of `shape` inside a buffer with GUARD sentinel bytes before and after it."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape)) * ESIZE[dtype]
        self.buf = torch.full((GUARD + self.n + GUARD,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(*shape)

    def intact(self):
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.n:]
        return bool((head == SENTINEL).all()) and bool((tail == SENTINEL).all())


def _check(label, guards):
    torch.cuda.synchronize()
    bad = [name for name, g in guards.items() if not g.intact()]
    say(f"  {label}: guards of {sorted(guards)} {'intact' if not bad else 'OVERWRITTEN: ' + str(bad)}")
    assert not bad, f"{label}: writes outside {bad}"


def _inputs(B, H, T, dk, dv, chunk, dtype, seed):
    spec = ki.small_spec(B, H, T, dk, dv, chunk, dtype, seed=seed, s0_std=0.3, z_mean=-2.0)
    return spec, dev_inputs(ki.prefill_inputs(spec), dtype)


PREFILL_FORMS = [  # label, B, H, T, dk, dv, chunk, dtype, segments (None: the library's choice)
    ("two 64-column slices", 2, 64, 64 * 5 + 37, 128, 128, 64, "bf16", None),
    ("four 32-column slices", 1, 64, 64 * 5 + 37, 128, 128, 64, "bf16", None),
    ("eight 16-column slices", 1, 8, 64 * 5 + 37, 128, 128, 64, "bf16", None),
    ("vector-ALU kernel", 2, 3, 16 * 9 + 5, 64, 32, 16, "f32", None),
    ("segment-parallel, chosen", 1, 8, 64 * 20 + 37, 128, 128, 64, "bf16", None),
    ("segment-parallel, 3 segments", 1, 2, 64 * 7 + 37, 128, 128, 64, "bf16", 3),
]


@pytest.mark.parametrize("label,B,H,T,dk,dv,chunk,dtype,segs", PREFILL_FORMS, ids=[f[0] for f in PREFILL_FORMS])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_prefill_writes_stay_inside(label, B, H, T, dk, dv, chunk, dtype, segs, o_dtype):
    say(f"case guards prefill {label}: B={B} H={H} T={T} dk={dk} dv={dv} chunk={chunk} {dtype} o={o_dtype}")
    spec, dd = _inputs(B, H, T, dk, dv, chunk, dtype, seed=9100 + T + H)
    args = (dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"])
    g = {"o": Guarded((B, T, H, dv), o_dtype), "S_out": Guarded((B, H, dk, dv), torch.float32)}
    if segs is None:
        need = kda.chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk)
        if label.startswith("segment"):
            assert need > 0, "expected the library to pick the segment-parallel form"
        if need:
            g["workspace"] = Guarded((need,), torch.uint8)
        kda.chunk_fwd_z(*args, -5.0, chunk, S_in=dd["S0"], o=g["o"].t, S_out=g["S_out"].t,
                        workspace=g["workspace"].t if need else None)
        ref = kda.chunk_fwd_z(*args, -5.0, chunk, S_in=dd["S0"], o_dtype=o_dtype)
    else:
        need = kda.chunk_fwd_z_segmented_workspace_bytes(B, H, dk, dv, segs)
        g["workspace"] = Guarded((need,), torch.uint8)
        kda.chunk_fwd_z_segmented(*args, segs, -5.0, chunk, S_in=dd["S0"], o=g["o"].t, S_out=g["S_out"].t,
                                  workspace=g["workspace"].t)
        ref = kda.chunk_fwd_z_segmented(*args, segs, -5.0, chunk, S_in=dd["S0"], o_dtype=o_dtype)
    _check(label, g)
    assert torch.equal(g["o"].t, ref[0]) and torch.equal(g["S_out"].t, ref[1])
    if segs is None and not label.startswith("segment"):
        # the precomputed-gate entry point on the same shape
        G = kda.gate(dd["z"], dd["A"], -5.0, chunk)
        g2 = {"o": Guarded((B, T, H, dv), o_dtype), "S_out": Guarded((B, H, dk, dv), torch.float32)}
        kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], G, chunk, S_in=dd["S0"], o=g2["o"].t, S_out=g2["S_out"].t)
        _check(label + ", precomputed gate", g2)


def test_gate_writes_stay_inside():
    B, H, T = 2, 3, 64 * 3 + 11
    say(f"case guards gate B={B} H={H} T={T}")
    spec, dd = _inputs(B, H, T, 128, 128, 64, "bf16", seed=9200)
    for chunk in (1, 16, 64):
        g = {"G": Guarded((B, T, H, 128), torch.float32)}
        kda.gate(dd["z"], dd["A"], -5.0, chunk, out=g["G"].t)
        _check(f"gate chunk {chunk}", g)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 32, "f32")])
def test_decode_and_replay_writes_stay_inside(dk, dv, dtype):
    spec = ki.DecodeSpec("decode_guard", N=5, H=3, dk=dk, dv=dv, steps=6, dtype=dtype, seed=9300)
    say(f"case guards decode / replay dk={dk} dv={dv} {dtype}")
    d = ki.decode_inputs(spec)
    dd = dev_inputs(d, dtype)
    g = {"S": Guarded((5, 3, dk, dv), torch.float32), "o": Guarded((5, 3, dv), torch.float32)}
    g["S"].t.copy_(dd["S0"])
    kda.decode_step(dd["q"][0], dd["k"][0], dd["v"][0], dd["z"][0], dd["beta"][0], dd["A"], g["S"].t, o=g["o"].t)
    _check("decode step", g)
    acc = torch.tensor([0, 6, 3, 1, 5], dtype=torch.int32, device=DEV)
    g = {"o": Guarded((6, 5, 3, dv), torch.bfloat16), "S_commit": Guarded((5, 3, dk, dv), torch.float32)}
    kda.decode_replay(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["A"], dd["S0"], acc, o=g["o"].t,
                      S_commit=g["S_commit"].t)
    _check("replay", g)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 32, "f32")])
def test_backward_writes_stay_inside(dk, dv, dtype):
    B, H, T = 1, 3, 64 * 3 + 23
    say(f"case guards backward B={B} H={H} T={T} dk={dk} dv={dv} {dtype}")
    spec, dd = _inputs(B, H, T, dk, dv, 64, dtype, seed=9400)
    d_o = torch.randn(B, T, H, dv, device=DEV).to(dd["q"].dtype)
    dS = torch.randn(B, H, dk, dv, device=DEV)
    need = int(kda.lib().kda_chunk_bwd_z_workspace_bytes(B, T, H, dk, dv))
    ws = Guarded((need,), torch.uint8)
    names = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv), "dbeta": (B, T, H), "dz": (B, T, H, dk),
             "dA": (H, dk), "dS_in": (B, H, dk, dv)}
    g = {n: Guarded(s, torch.float32) for n, s in names.items()}
    f32 = {n: g[n].t for n in names}
    import ctypes
    L = kda.lib()
    code = 1 if dtype == "bf16" else 0
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = L.kda_chunk_bwd_z(p(dd["q"]), p(dd["k"]), p(dd["v"]), p(dd["beta"]), p(dd["z"]), code, p(dd["A"]), -5.0,
                           p(dd["S0"]), p(d_o), code, p(dS), p(f32["dq"]), p(f32["dk"]), p(f32["dv"]),
                           p(f32["dbeta"]), p(f32["dz"]), p(f32["dA"]), p(f32["dS_in"]), B, T, H, dk, dv, 1.0,
                           p(ws.t), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.kda_status_string(st)
    g["workspace"] = ws
    _check("backward", g)
    ref = kda.chunk_bwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], d_o, dS, -5.0, dd["S0"])
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(f32[n], ref[n]), n
