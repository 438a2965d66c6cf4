"""GPU parity of the fused-prologue entry points (kda_chunk_fwd_z_prologue,
kda_decode_step_prologue) against the fp64 oracle's prologue + recurrence, on
raw inputs: q and k un-normalised (row norms from about 4e-3 to 36, some rows
exactly zero) and beta as a logit.  Tolerance: relative L2 1e-5 for fp32
inputs and 1e-2 for bf16, separately for o and the final state."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import TOL, dev_inputs, f64_inputs, host64, rel_l2, say

pytestmark = pytest.mark.gpu


def _zero_some_rows(d, dtype, every=7):
    """Exact-zero q and k rows on every 7th token of every sequence (a zero vector stays zero)."""
    for name in ("q", "k"):
        d[name][:, ::every] = 0
    return d


def _oracle(d, dtype):
    f = f64_inputs(d, dtype)
    return oracle.forward_z_prologue(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])


CASES = [  # B, H, T, dk, dv, chunk, dtype, s0, z_mean
    (1, 2, 64 * 5 + 9, 128, 128, 64, "bf16", 0.5, 0.0),   # MFMA path, ragged last chunk, given S_in
    (2, 3, 1000, 128, 128, 64, "bf16", 0.0, -6.0),        # MFMA path, slow decay (state carried far)
    (1, 2, 100, 128, 128, 64, "f32", 0.3, 0.0),           # generic path, fp32 inputs
    (2, 2, 77, 64, 32, 16, "f32", 0.2, -4.0),             # generic path, small dims, chunk 16
    (1, 3, 130, 128, 128, 16, "bf16", 0.0, 0.0),          # generic path, bf16 inputs, chunk 16
    (1, 1, 50, 16, 128, 64, "f32", 0.1, 0.0),             # generic path, dk 16
]


@pytest.mark.parametrize("B,H,T,dk,dv,chunk,dtype,s0,zm", CASES)
def test_chunk_prologue_vs_oracle(B, H, T, dk, dv, chunk, dtype, s0, zm):
    spec = ki.small_spec(B, H, T, dk, dv, chunk, dtype, seed=5100 + T + dk, s0_std=s0, z_mean=zm, raw=True)
    say(f"case prologue prefill B={B} H={H} T={T} dk={dk} dv={dv} chunk={chunk} {dtype} s0={s0} z_mean={zm}")
    d = _zero_some_rows(ki.prefill_inputs(spec), dtype)
    dd = dev_inputs(d, dtype)
    for o_dtype in (torch.float32, torch.bfloat16):
        o, S = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, chunk,
                                        S_in=dd["S0"], o_dtype=o_dtype)
        torch.cuda.synchronize()
        o_ref, S_ref = _oracle(d, dtype)
        eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
        say(f"  o={o_dtype} rel-L2 o={eo:.3e} S={es:.3e}")
        tol = TOL[dtype] if o_dtype == torch.float32 else TOL["bf16"]
        assert eo <= tol and es <= tol


def test_chunk_prologue_in_place_and_split():
    """S_out == S_in, and two calls with the state carried equal one call."""
    spec = ki.small_spec(1, 2, 300, 128, 128, 64, "bf16", seed=5200, s0_std=0.3, raw=True)
    say("case prologue in-place + split")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, "bf16")
    o, S = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], S_in=dd["S0"])
    S_io = dd["S0"].clone()
    o2, S2 = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], S_in=S_io,
                                      S_out=S_io)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_io.data_ptr() and torch.equal(o, o2) and torch.equal(S, S2)
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o_a, S_a = kda.chunk_fwd_z_prologue(*(sl(dd[n], 0, 128) for n in ("q", "k", "v", "beta", "z")), dd["A"],
                                        S_in=dd["S0"])
    o_b, S_b = kda.chunk_fwd_z_prologue(*(sl(dd[n], 128, 300) for n in ("q", "k", "v", "beta", "z")), dd["A"],
                                        S_in=S_a)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o_a, o_b], dim=1), o) and torch.equal(S_b, S)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16), (128, 128)])
def test_decode_prologue_vs_oracle(dtype, dk, dv):
    spec = ki.DecodeSpec("decode_prologue", N=5, H=3, dk=dk, dv=dv, steps=7, dtype=dtype, s_std=0.1, seed=5300,
                         raw=True)
    say(f"case prologue decode N=5 H=3 dk={dk} dv={dv} {dtype}")
    d = ki.decode_inputs(spec)
    d["q"][2, 1] = 0
    d["k"][3, 4] = 0
    f = f64_inputs(d, dtype)
    o_ref, S_ref = oracle.decode_prologue(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"])
    dd = dev_inputs(d, dtype)
    S = dd["S0"].clone()
    outs = [kda.decode_step_prologue(dd["q"][s], dd["k"][s], dd["v"][s], dd["z"][s], dd["beta"][s], dd["A"], S)
            for s in range(spec.steps)]
    torch.cuda.synchronize()
    o = torch.stack(outs)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_prologue_matches_prefill_prologue():
    """n fused-prologue decode steps == one n-token fused-prologue prefill (fp32, GPU vs GPU)."""
    spec = ki.small_spec(3, 2, 40, 64, 64, 16, "f32", seed=5400, s0_std=0.1, raw=True)
    dd = dev_inputs(ki.prefill_inputs(spec), "f32")
    o_p, S_p = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, 16,
                                        S_in=dd["S0"])
    S = dd["S0"].clone()
    outs = [kda.decode_step_prologue(*(dd[n][:, t].contiguous() for n in ("q", "k", "v", "z", "beta")), dd["A"], S)
            for t in range(spec.T)]
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    assert rel_l2(host64(o_d), host64(o_p)) <= 1e-5 and rel_l2(host64(S), host64(S_p)) <= 1e-5


def test_prologue_32k_sampled():
    """The 32K-token workload's shape on raw inputs, in the benchmark's launch
    configuration (bf16 in and out), against the oracle on sampled heads."""
    spec = replace(ki.PREFILL_32K, name=ki.PREFILL_32K.name + "_raw", raw=True)
    say(f"case {spec.name}: generating inputs")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    o, S = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], S_in=dd["S0"],
                                    o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    for b, h in [(0, 1), (3, 30)]:
        sub = {k: np.ascontiguousarray(d[k][b:b + 1, :, h:h + 1]) for k in ("q", "k", "v", "z", "beta")}
        sub["A"] = np.ascontiguousarray(d["A"][h:h + 1])
        sub["S0"] = np.ascontiguousarray(d["S0"][b:b + 1, h:h + 1])
        o_ref, S_ref = _oracle(sub, spec.dtype)
        eo = rel_l2(host64(o[b:b + 1, :, h:h + 1]), o_ref)
        es = rel_l2(host64(S[b:b + 1, h:h + 1]), S_ref)
        say(f"  b={b} h={h} rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
