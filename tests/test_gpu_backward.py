"""GPU parity of the backward pass (kda_chunk_bwd_z) against the fp64 oracle's
reverse-mode derivative (oracle.backward), on the same rounded inputs and the
same upstream gradients.  Tolerance: relative L2 per gradient, 1e-5 for fp32
inputs (1e-4 for the gate's derivatives dz and dA, whose chunk-form terms cancel:
see ``bwd_tol``) and 1e-2 for bf16 inputs (the bf16 path takes its checkpoints
from the bf16 matrix-core forward and runs its long products with bf16 operands
and fp32 accumulation; measured up to 5e-3)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle.backward as OB
from tests._gpu import DEV, TOL, bwd_tol, dev, dev_inputs, f64_inputs, grad_errors, host64, rel_l2, say

pytestmark = pytest.mark.gpu

GRADS = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"), ("dz", "dz"), ("dA", "dA"),
         ("dS_in", "dS_in")]


def _cot(spec, seed, with_dS):
    rng = np.random.default_rng(seed)
    do = ki.round_storage(rng.standard_normal((spec.B, spec.T, spec.H, spec.dv)), spec.dtype)
    dS = ki.round_to_f32(rng.standard_normal((spec.B, spec.H, spec.dk, spec.dv)) * 0.1) if with_dS else None
    return do, dS


def _run(spec, with_dS=True, scale=1.0, seed=7):
    d = ki.prefill_inputs(spec)
    do, dS = _cot(spec, seed, with_dS)
    dd = dev_inputs(d, spec.dtype)
    g = kda.chunk_bwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], dev(do, spec.dtype),
                        None if dS is None else dev(dS, "f32"), -5.0, dd["S0"], scale)
    torch.cuda.synchronize()
    f = f64_inputs(d, spec.dtype)
    ref = OB.backward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], ki.to_f64(do, spec.dtype),
                        None if dS is None else dS.astype(np.float64), -5.0, f["S0"], scale)
    return g, ref


CASES = [  # B, H, T, dk, dv, dtype, s0, z_mean, with_dS, scale
    (1, 2, 37, 16, 16, "f32", 0.3, 0.0, True, 1.0),
    (2, 2, 100, 64, 32, "f32", 0.0, -4.0, True, 0.5),
    (1, 2, 130, 128, 128, "f32", 0.3, -6.0, False, 1.0),
    (1, 1, 64, 32, 128, "f32", 0.2, 0.0, True, 1.0),
    (1, 2, 200, 128, 128, "bf16", 0.3, -6.0, True, 1.0),   # checkpoints from the matrix-core forward
    (2, 3, 77, 128, 64, "bf16", 0.0, 0.0, True, 1.0),
    (1, 2, 16, 16, 128, "bf16", 0.1, -4.0, False, 1.0),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,s0,zm,with_dS,scale", CASES)
def test_backward_vs_oracle(B, H, T, dk, dv, dtype, s0, zm, with_dS, scale):
    spec = ki.small_spec(B, H, T, dk, dv, 64, dtype, seed=6100 + T + dk + dv, s0_std=s0, z_mean=zm)
    say(f"case backward B={B} H={H} T={T} dk={dk} dv={dv} {dtype} s0={s0} z_mean={zm} dS_out={with_dS}")
    g, ref = _run(spec, with_dS, scale)
    errs = grad_errors(g, ref, [name for name, _ in GRADS])
    say("  rel-L2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= bwd_tol(dtype, name), (name, e)


def test_backward_empty_and_deterministic():
    spec = ki.small_spec(1, 2, 0, 64, 64, 64, "f32", seed=6200, s0_std=0.2)
    say("case backward T=0")
    g, ref = _run(spec, True)
    assert rel_l2(host64(g["dS_in"]), ref["dS_in"]) == 0.0          # dS_in = dS_out
    assert float(g["dA"].abs().max()) == 0.0
    spec = ki.small_spec(2, 2, 150, 128, 128, 64, "bf16", seed=6201, s0_std=0.2)
    say("case backward twice, bitwise")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, "bf16")
    do, dS = _cot(spec, 3, True)
    args = (dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], dev(do, "bf16"), dev(dS, "f32"), -5.0, dd["S0"])
    g1 = kda.chunk_bwd_z(*args)
    g2 = kda.chunk_bwd_z(*args)
    torch.cuda.synchronize()
    for name, _ in GRADS:
        assert torch.equal(g1[name], g2[name]), name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_one_slice_many_heads(dtype):
    """B*H = 256 at d_k = d_v = 128 runs one value slice per head (two slices are
    for fewer heads): all heads on the GPU, three sampled heads against the
    oracle.  With B = 1 a head's dA comes from that head alone."""
    B, H, T = 1, 256, 70
    spec = ki.small_spec(B, H, T, 128, 128, 64, dtype, seed=6300, s0_std=0.2, z_mean=-4.0)
    say(f"case backward one slice B={B} H={H} T={T} {dtype}")
    d = ki.prefill_inputs(spec)
    do, dS = _cot(spec, 5, True)
    dd = dev_inputs(d, dtype)
    g = kda.chunk_bwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], dev(do, dtype), dev(dS, "f32"),
                        -5.0, dd["S0"])
    torch.cuda.synchronize()
    for h in (0, 97, 255):
        sub = {k: np.ascontiguousarray(d[k][:, :, h:h + 1]) for k in ("q", "k", "v", "z", "beta")}
        sub["A"] = np.ascontiguousarray(d["A"][h:h + 1])
        sub["S0"] = np.ascontiguousarray(d["S0"][:, h:h + 1])
        f = f64_inputs(sub, dtype)
        ref = OB.backward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"],
                            ki.to_f64(np.ascontiguousarray(do[:, :, h:h + 1]), dtype),
                            np.ascontiguousarray(dS[:, h:h + 1]).astype(np.float64), -5.0, f["S0"])
        errs = {}
        for name in ("dq", "dk", "dv", "dbeta", "dz"):
            errs[name] = rel_l2(host64(g[name][:, :, h:h + 1]), ref[name])
        errs["dA"] = rel_l2(host64(g["dA"][h:h + 1]), ref["dA"])
        errs["dS_in"] = rel_l2(host64(g["dS_in"][:, h:h + 1]), ref["dS_in"])
        say(f"  h={h} rel-L2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        for name, e in errs.items():
            assert e <= bwd_tol(dtype, name), (h, name, e)


def test_backward_32k_sampled():
    """The 32K-token workload (B=4, H=32, bf16), whole batch on the GPU, against
    the oracle on one sampled (b, h) sequence over its full length (every
    gradient but dA, which sums over the batch)."""
    spec = ki.PREFILL_32K
    say(f"case backward {spec.name}: generating inputs")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    rng = np.random.default_rng(11)
    b, h = 1, 17
    do = np.zeros((spec.B, spec.T, spec.H, spec.dv), np.uint16)
    do[b, :, h] = ki.round_storage(rng.standard_normal((spec.T, spec.dv)), spec.dtype)
    other = rng.standard_normal((spec.B, spec.T, spec.H, spec.dv)).astype(np.float32)
    do_all = ki.round_storage(other, spec.dtype)
    do_all[b, :, h] = do[b, :, h]
    say("  GPU backward, whole batch")
    g = kda.chunk_bwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], dev(do_all, spec.dtype), None,
                        -5.0, dd["S0"])
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dbeta", "dz", "dA", "dS_in"):
        assert bool(torch.isfinite(g[name]).all()), name
    say(f"  oracle backward b={b} h={h} T={spec.T}")
    sub = {k: np.ascontiguousarray(d[k][b:b + 1, :, h:h + 1]) for k in ("q", "k", "v", "z", "beta")}
    sub["A"] = np.ascontiguousarray(d["A"][h:h + 1])
    sub["S0"] = np.ascontiguousarray(d["S0"][b:b + 1, h:h + 1])
    f = f64_inputs(sub, spec.dtype)
    ref = OB.backward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"],
                        ki.to_f64(np.ascontiguousarray(do_all[b:b + 1, :, h:h + 1]), spec.dtype), None, -5.0, f["S0"])
    errs = {}
    for name in ("dq", "dk", "dv", "dbeta", "dz"):
        errs[name] = rel_l2(host64(g[name][b:b + 1, :, h:h + 1]), ref[name])
    errs["dS_in"] = rel_l2(host64(g["dS_in"][b:b + 1, h:h + 1]), ref["dS_in"])
    say("  rel-L2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)
