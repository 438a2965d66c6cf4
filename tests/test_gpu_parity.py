"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded, rounded inputs.  Tolerance: relative L2 over the whole tensor,
1e-5 for fp32 inputs and 1e-2 for bf16 inputs, separately for o and the final
state (both computed in fp64)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import DEV, TOL, dev, dev_inputs, f64_inputs, host64, rel_l2, say

pytestmark = pytest.mark.gpu


def run_gpu(dd, spec, path, o_dtype=torch.float32, S_in="given", alias=False):
    S0 = dd["S0"]
    if S_in == "zeros" and S0 is None:
        S0 = torch.zeros(spec.B, spec.H, spec.dk, spec.dv, device=DEV)
    S_out = S0 if (alias and S0 is not None) else None
    if path == "z":
        o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, spec.chunk, S_in=S0,
                               S_out=S_out, o_dtype=o_dtype)
    else:
        G = kda.gate(dd["z"], dd["A"], -5.0, spec.chunk)
        o, S = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], G, spec.chunk, S_in=S0, S_out=S_out,
                             o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, S


def oracle_ref(d, spec):
    f = f64_inputs(d, spec.dtype)
    return oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])


@pytest.mark.parametrize("path", ["z", "G"])
def test_tiny_f32(path):
    spec = ki.TINY_F32
    say(f"case {spec.name} path={path}")
    d = ki.prefill_inputs(spec)
    o, S = run_gpu(dev_inputs(d, spec.dtype), spec, path)
    o_ref, S_ref = oracle_ref(d, spec)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [1, 16, 64])
def test_gate(dtype, chunk):
    spec = ki.small_spec(2, 3, 200, 64, 16, 16, dtype, seed=77, z_scale=3.0)
    say(f"case gate dtype={dtype} chunk={chunk}")
    d = ki.prefill_inputs(spec)
    G = host64(kda.gate(dev(d["z"], dtype), dev(d["A"], "f32"), -5.0, chunk))
    G_ref = oracle.gate(ki.to_f64(d["z"], dtype), d["A"].astype(np.float64), -5.0, chunk)
    assert rel_l2(G, G_ref) <= 2e-6
    assert np.max(np.abs(G - G_ref)) <= 1e-5 * max(1.0, np.max(np.abs(G_ref)))
    assert np.all(G <= 0.0) and np.all(G >= -5.0 * chunk)


@pytest.mark.parametrize("path", ["z", "G"])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_prefill_4k(path, o_dtype):
    spec = ki.PREFILL_4K
    say(f"case {spec.name} path={path} o={o_dtype}")
    d = ki.prefill_inputs(spec)
    o, S = run_gpu(dev_inputs(d, spec.dtype), spec, path, o_dtype=o_dtype)
    o_ref, S_ref = oracle_ref(d, spec)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


EDGE = []
for T in (0, 1, 15, 16, 17, 63, 65, 127):
    EDGE.append((T, 16, 16, 16, "f32", 0.0))
    EDGE.append((T, 128, 128, 64, "bf16", 0.1))
EDGE += [(100, 32, 64, 16, "f32", 0.1), (130, 64, 32, 64, "bf16", 0.0), (77, 128, 16, 64, "f32", 0.2),
         (50, 16, 128, 16, "bf16", 0.1)]


@pytest.mark.parametrize("T,dk,dv,chunk,dtype,s0", EDGE)
def test_edge_shapes(T, dk, dv, chunk, dtype, s0):
    spec = ki.small_spec(2, 3, T, dk, dv, chunk, dtype, seed=1234 + T, s0_std=s0)
    say(f"case edge T={T} dk={dk} dv={dv} chunk={chunk} {dtype} s0={s0}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    o_ref, S_ref = oracle_ref(d, spec)
    for path in ("z", "G"):
        o, S = run_gpu(dd, spec, path, S_in="zeros" if s0 == 0.0 else "given")
        eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
        say(f"  path={path} rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]


LONG = [(128, 128, 64, "bf16"), (128, 128, 64, "f32"), (128, 128, 16, "bf16"), (64, 32, 16, "f32"),
        (32, 128, 64, "f32")]


@pytest.mark.parametrize("dk,dv,chunk,dtype", LONG)
def test_long_memory(dk, dv, chunk, dtype):
    """Slow decay (decay logits centred at -6): the entry state and the state
    carried across many chunks still shape the outputs."""
    spec = ki.small_spec(1, 3, 1500, dk, dv, chunk, dtype, seed=2200 + dk + chunk, s0_std=0.5, z_mean=-6.0)
    say(f"case long memory dk={dk} dv={dv} chunk={chunk} {dtype}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    o_ref, S_ref = oracle_ref(d, spec)
    f = f64_inputs(d, dtype)
    o_0, _ = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, None)
    gap = rel_l2(o_0, o_ref)
    say(f"  entry state dropped: rel-L2 {gap:.3e} from the true outputs")
    assert gap > 10 * TOL[dtype]
    for path in ("z", "G"):
        o, S = run_gpu(dd, spec, path)
        eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
        say(f"  path={path} rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_in_place(dtype):
    """S_out == S_in: the state is read before it is overwritten."""
    spec = ki.small_spec(1, 4, 90, 128, 128, 64, dtype, seed=5, s0_std=0.3)
    say(f"case in-place state {dtype}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    o, S = run_gpu(dd, spec, "z", alias=True)
    assert S.data_ptr() == dd["S0"].data_ptr()
    o_ref, S_ref = oracle_ref(d, spec)
    assert rel_l2(host64(o), o_ref) <= TOL[dtype] and rel_l2(host64(S), S_ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_split_carries_state(dtype):
    """run(S, L||R) = (run(run(S, L).S, R).S, concat outputs) on the GPU:
    bitwise for a chunk-aligned split, within tolerance otherwise."""
    spec = ki.small_spec(1, 2, 300, 128, 128, 64, dtype, seed=9, s0_std=0.1)
    say(f"case chunk-split {dtype}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, 64, S_in=dd["S0"])
    o_ref, S_ref = oracle_ref(d, spec)
    for cut in (128, 100):
        sl = lambda x, a, b: x[:, a:b].contiguous()
        o1, S1 = kda.chunk_fwd_z(*(sl(dd[n], 0, cut) for n in ("q", "k", "v", "beta", "z")), dd["A"], -5.0, 64,
                                 S_in=dd["S0"])
        o2, S2 = kda.chunk_fwd_z(*(sl(dd[n], cut, 300) for n in ("q", "k", "v", "beta", "z")), dd["A"], -5.0, 64,
                                 S_in=S1)
        torch.cuda.synchronize()
        oc = torch.cat([o1, o2], dim=1)
        if cut % 64 == 0:
            assert torch.equal(oc, o) and torch.equal(S2, S)
        else:
            # a different grouping of the same tokens: each result is held to the oracle
            assert rel_l2(host64(oc), o_ref) <= TOL[dtype] and rel_l2(host64(S2), S_ref) <= TOL[dtype]


def test_run_twice_bitwise():
    spec = ki.small_spec(2, 4, 333, 128, 128, 64, "bf16", seed=11, s0_std=0.1)
    say("case determinism")
    dd = dev_inputs(ki.prefill_inputs(spec), "bf16")
    o1, S1 = run_gpu(dd, spec, "z")
    o2, S2 = run_gpu(dd, spec, "z")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16), (64, 64), (128, 128)])
def test_decode_small(dtype, dk, dv):
    spec = ki.DecodeSpec("decode_small", N=5, H=3, dk=dk, dv=dv, steps=7, dtype=dtype, s_std=0.1, seed=21)
    say(f"case decode N=5 H=3 dk={dk} dv={dv} {dtype}")
    d = ki.decode_inputs(spec)
    f = f64_inputs(d, dtype)
    o_ref, S_ref = oracle.decode(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"])
    dd = dev_inputs(d, dtype)
    S = dd["S0"].clone()
    outs = []
    for s in range(spec.steps):
        outs.append(kda.decode_step(dd["q"][s], dd["k"][s], dd["v"][s], dd["z"][s], dd["beta"][s], dd["A"], S))
    torch.cuda.synchronize()
    o = torch.stack(outs)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_matches_prefill_f32():
    """n decode steps == one n-token chunked prefill (GPU vs GPU, fp32)."""
    spec = ki.small_spec(3, 2, 40, 64, 64, 16, "f32", seed=31, s0_std=0.1)
    say("case decode==prefill")
    dd = dev_inputs(ki.prefill_inputs(spec), "f32")
    o_p, S_p = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, 16, S_in=dd["S0"])
    S = dd["S0"].clone()
    outs = [kda.decode_step(*(dd[n][:, t].contiguous() for n in ("q", "k", "v", "z", "beta")), dd["A"], S)
            for t in range(spec.T)]
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    assert rel_l2(host64(o_d), host64(o_p)) <= 1e-5 and rel_l2(host64(S), host64(S_p)) <= 1e-5
