"""GPU parity in the method's degenerate and extreme cases, against the fp64
oracle on the same inputs (tolerances as everywhere: relative L2 1e-5 for fp32
inputs, 1e-2 for bf16), plus the results that are exact:

* g_min = 0: no decay at all (alpha = 1), the delta rule alone;
* g_min at the limit the entry points accept (-5, the value the pages fix);
* whole 16-token tiles at the floor of the gate (sigma saturated on every token
  of a channel, so a tile decays by exactly e^(16 g_min)), through the fused
  gate and through kda_gate followed by kda_chunk_fwd;
* decay logits far in saturation (|e^A z| ~ 100: g is exactly 0 or g_min);
* beta = 0: the state only decays and is never written;
* q = 0: every output is exactly zero; v = 0 with a zero entry state: the
  state and the outputs stay exactly zero;
* many heads (H = 1024 for the prefill, 2048 for the decode): large strides;
* head counts that select each launch shape of the matrix-core prefill: four
  32-column slices per head (B*H = 64 with the XCD-grouped workgroup order,
  B*H = 63 without it), eight 16-column slices (B*H = 16 grouped, 25 plain)
  and two 64-column slices in plain order (B*H = 130),
  for the fused gate and the precomputed gate (the segment passes' shapes are
  covered in test_gpu_segmented).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
import oracle.backward as OB
from tests._gpu import TOL, assert_states, assert_tokens, dev, dev_inputs, f64_inputs, host64, rel_l2, say

pytestmark = pytest.mark.gpu

SHAPES = [  # dk, dv, chunk, dtype: the matrix-core path and the generic one
    (128, 128, 64, "bf16"),
    (64, 32, 16, "f32"),
]


def _prefill(d, spec, g_min, dd=None):
    dd = dd or dev_inputs(d, spec.dtype)
    o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], g_min, spec.chunk,
                           S_in=dd["S0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    f = f64_inputs(d, spec.dtype)
    o_ref, S_ref = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], g_min, f["S0"])
    return o, S, o_ref, S_ref


@pytest.mark.parametrize("dk,dv,chunk,dtype", SHAPES)
@pytest.mark.parametrize("g_min", [0.0, -0.5, -5.0])
def test_gate_floor(dk, dv, chunk, dtype, g_min):
    spec = ki.small_spec(1, 3, 300, dk, dv, chunk, dtype, seed=7100 + dk, s0_std=0.3)
    say(f"case g_min={g_min} dk={dk} dv={dv} chunk={chunk} {dtype}")
    d = ki.prefill_inputs(spec)
    o, S, o_ref, S_ref = _prefill(d, spec, g_min)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("path", ["fused gate", "kda_gate then kda_chunk_fwd", "fused prologue"])
def test_whole_tiles_at_the_floor(path):
    """Key channels whose decay logit is +100 on every token (sigma = 1, g = g_min = -5
    exactly): each of their 16-token tiles decays by e^-80, whose reciprocal the
    matrix-core kernel forms; and one whole chunk with every channel there.  The fused
    prologue takes raw queries and keys of magnitudes down to 10^-3.5 (the queries are
    normalised before the decay factor, which would otherwise take them below the
    smallest normal number).  Checked per sequence and per 16-token block."""
    g_min = -5.0
    spec = ki.small_spec(1, 2, 64 * 3 + 20, 128, 128, 64, "bf16", seed=7150, s0_std=0.3,
                         raw=(path == "fused prologue"))
    say(f"case whole tiles at the floor g_min={g_min} via {path}")
    d = ki.prefill_inputs(spec)
    sat = ki.round_storage(np.full((1,), 100.0), "bf16")[0]
    d["z"][:, :, :, [0, 5, 77, 127]] = sat
    d["z"][:, 64:128] = sat
    dd = dev_inputs(d, spec.dtype)
    if path == "fused gate":
        o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], g_min, 64, S_in=dd["S0"],
                               o_dtype=torch.float32)
    elif path == "fused prologue":
        o, S = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], g_min, 64,
                                        S_in=dd["S0"], o_dtype=torch.float32)
    else:
        G = kda.gate(dd["z"], dd["A"], g_min, chunk=64)
        o, S = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], G, 64, S_in=dd["S0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    f = f64_inputs(d, spec.dtype)
    run = oracle.forward_z_prologue if path == "fused prologue" else oracle.forward_z
    o_ref, S_ref = run(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], g_min, f["S0"])
    assert_tokens("o", host64(o), o_ref, TOL["bf16"], block=16)
    assert_states("S", host64(S), S_ref, TOL["bf16"])


@pytest.mark.parametrize("dk,dv,chunk,dtype", SHAPES)
def test_saturated_gate(dk, dv, chunk, dtype):
    """Decay logits at +-100 (times e^A): sigma saturates, g is g_min or 0 exactly."""
    spec = ki.small_spec(1, 2, 200, dk, dv, chunk, dtype, seed=7200 + dk, s0_std=0.3)
    say(f"case saturated gate dk={dk} {dtype}")
    d = ki.prefill_inputs(spec)
    rng = np.random.default_rng(7201)
    sign = np.where(rng.random(d["z"].shape) < 0.5, -100.0, 100.0)
    d["z"] = ki.round_storage(sign, dtype)
    o, S, o_ref, S_ref = _prefill(d, spec, -5.0)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dk,dv,chunk,dtype", SHAPES)
def test_zero_write_strength(dk, dv, chunk, dtype):
    """beta = 0: the state only decays; the outputs read the decayed entry state."""
    spec = ki.small_spec(2, 2, 150, dk, dv, chunk, dtype, seed=7300 + dk, s0_std=0.5, z_mean=-6.0)
    say(f"case beta=0 dk={dk} {dtype}")
    d = ki.prefill_inputs(spec)
    d["beta"][:] = 0
    o, S, o_ref, S_ref = _prefill(d, spec, -5.0)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dk,dv,chunk,dtype", SHAPES)
def test_exact_zeros(dk, dv, chunk, dtype):
    """q = 0 gives exactly zero outputs; v = 0 with no entry state keeps everything zero."""
    spec = ki.small_spec(1, 2, 130, dk, dv, chunk, dtype, seed=7400 + dk, s0_std=0.3)
    say(f"case exact zeros dk={dk} {dtype}")
    d = ki.prefill_inputs(spec)
    d["q"][:] = 0
    o, S, _, S_ref = _prefill(d, spec, -5.0)
    assert float(o.abs().max()) == 0.0
    assert rel_l2(host64(S), S_ref) <= TOL[dtype]
    d = ki.prefill_inputs(ki.small_spec(1, 2, 130, dk, dv, chunk, dtype, seed=7401 + dk))
    d["v"][:] = 0
    o, S, _, _ = _prefill(d, spec, -5.0)
    assert float(o.abs().max()) == 0.0 and float(S.abs().max()) == 0.0


def test_many_heads_prefill():
    spec = ki.small_spec(1, 1024, 64 + 17, 128, 128, 64, "bf16", seed=7500, s0_std=0.1)
    say("case H=1024 T=81 prefill")
    d = ki.prefill_inputs(spec)
    o, S, o_ref, S_ref = _prefill(d, spec, -5.0)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_many_heads_decode_and_no_decay():
    spec = ki.DecodeSpec("decode_wide", N=2, H=2048, dk=128, dv=128, steps=3, dtype="bf16", s_std=0.1, seed=7600)
    d = ki.decode_inputs(spec)
    f = f64_inputs(d, "bf16")
    dd = dev_inputs(d, "bf16")
    for g_min in (-5.0, 0.0):
        say(f"case decode N=2 H=2048 g_min={g_min}")
        S = dd["S0"].clone()
        outs = [kda.decode_step(dd["q"][s], dd["k"][s], dd["v"][s], dd["z"][s], dd["beta"][s], dd["A"], S, g_min)
                for s in range(spec.steps)]
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"], g_min)
        eo, es = rel_l2(host64(torch.stack(outs)), o_ref), rel_l2(host64(S), S_ref)
        say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_no_decay_and_floor(dtype):
    """g_min = 0: the gate has no effect, so dz and dA are exactly zero and the other
    gradients match the oracle; g_min = -5 (the floor the backward accepts) as well."""
    spec = ki.small_spec(1, 2, 100, 128, 128, 64, dtype, seed=7700, s0_std=0.3)
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    rng = np.random.default_rng(7701)
    do = ki.round_storage(rng.standard_normal((1, 100, 2, 128)), dtype)
    f = f64_inputs(d, dtype)
    for g_min in (0.0, -5.0):
        say(f"case backward g_min={g_min} {dtype}")
        g = kda.chunk_bwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], dev(do, dtype), None, g_min,
                            dd["S0"])
        torch.cuda.synchronize()
        ref = OB.backward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], ki.to_f64(do, dtype), None, g_min,
                            f["S0"])
        names = ("dq", "dk", "dv", "dbeta", "dS_in") if g_min == 0.0 else ("dq", "dk", "dv", "dbeta", "dz", "dA",
                                                                           "dS_in")
        errs = {n: rel_l2(host64(g[n]), ref[n]) for n in names}
        say("  rel-L2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= TOL[dtype], (n, e)
        if g_min == 0.0:
            assert float(g["dz"].abs().max()) == 0.0 and float(g["dA"].abs().max()) == 0.0


@pytest.mark.parametrize("B,H", [(2, 32), (3, 21), (1, 16), (1, 25), (2, 65)])
def test_head_counts_select_launch_shapes(B, H):
    spec = ki.small_spec(B, H, 64 + 17, 128, 128, 64, "bf16", seed=7800 + B * H, s0_std=0.1)
    say(f"case launch shape B={B} H={H} T={spec.T} (fused gate, precomputed gate, 2 segments)")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    o, S, o_ref, S_ref = _prefill(d, spec, -5.0, dd)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  fused gate rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    G = kda.gate(dd["z"], dd["A"], -5.0, spec.chunk)
    o2, S2 = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], G, spec.chunk, S_in=dd["S0"],
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    eo, es = rel_l2(host64(o2), o_ref), rel_l2(host64(S2), S_ref)
    say(f"  precomputed gate rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # two segments of one chunk each (the last segment's pass over B*H*2 (b, h, segment)
    # units, the first segment's over B*H)
    o3, S3 = kda.chunk_fwd_z_segmented(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], 2, -5.0,
                                       spec.chunk, S_in=dd["S0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    eo, es = rel_l2(host64(o3), o_ref), rel_l2(host64(S3), S_ref)
    say(f"  two segments rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
