"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (fused gate, bf16 inputs and bf16 outputs), checked against
the fp64 oracle on sampled (batch, head) sequences computed one by one over
their whole length."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import TOL, dev_inputs, f64_inputs, host64, rel_l2, say

pytestmark = pytest.mark.gpu


def _prefill_sampled(spec, samples):
    say(f"case {spec.name}: generating inputs")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    say(f"case {spec.name}: GPU run")
    o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, spec.chunk,
                           S_in=dd["S0"], o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    for b, h in samples:
        say(f"  oracle b={b} h={h} T={spec.T}")
        sub = {k: np.ascontiguousarray(d[k][b:b + 1, :, h:h + 1]) for k in ("q", "k", "v", "z", "beta")}
        sub["A"] = np.ascontiguousarray(d["A"][h:h + 1])
        sub["S0"] = None if d["S0"] is None else np.ascontiguousarray(d["S0"][b:b + 1, h:h + 1])
        f = f64_inputs(sub, spec.dtype)
        o_ref, S_ref = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
        eo = rel_l2(host64(o[b:b + 1, :, h:h + 1]), o_ref)
        es = rel_l2(host64(S[b:b + 1, h:h + 1]), S_ref)
        say(f"  b={b} h={h} rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= TOL[spec.dtype] and es <= TOL[spec.dtype]
    del dd, o, S
    torch.cuda.empty_cache()


def test_prefill_32k_sampled():
    _prefill_sampled(ki.PREFILL_32K, [(0, 0), (1, 17), (3, 31)])


def test_prefill_32k_slow_decay_sampled():
    """The 32K-token workload's shape with decay logits centred at -6: the
    state is carried over many chunks before it fades."""
    spec = replace(ki.PREFILL_32K, name=ki.PREFILL_32K.name + "_slow", z_mean=-6.0)
    _prefill_sampled(spec, [(0, 3), (2, 30)])


def test_prefill_1m_sampled():
    _prefill_sampled(ki.PREFILL_1M, [(0, 5)])


def test_decode_256x32_sampled():
    spec = ki.DECODE_256
    say(f"case {spec.name}: generating inputs")
    d = ki.decode_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    S = dd["S0"].clone()
    outs = []
    say(f"case {spec.name}: GPU run, {spec.steps} steps")
    for s in range(spec.steps):
        outs.append(kda.decode_step(dd["q"][s], dd["k"][s], dd["v"][s], dd["z"][s], dd["beta"][s], dd["A"], S,
                                    o_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    o = torch.stack(outs)
    n_sel = [0, 77, 255]
    sub = {k: np.ascontiguousarray(d[k][:, n_sel]) for k in ("q", "k", "v", "z", "beta")}
    sub["A"] = d["A"]
    sub["S0"] = np.ascontiguousarray(d["S0"][n_sel])
    f = f64_inputs(sub, spec.dtype)
    say("  oracle on sequences", n_sel)
    o_ref, S_ref = oracle.decode(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"])
    eo = rel_l2(host64(o[:, n_sel]), o_ref)
    es = rel_l2(host64(S[n_sel]), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[spec.dtype] and es <= TOL[spec.dtype]
