"""GPU parity on configurations drawn at random (fixed seeds, so every run checks
the same cases): head sizes, chunk length, input and output dtypes, batch,
heads, ragged sequence lengths, gate floor, output scale, initial state and
entry point (fused gate, precomputed G, fused prologue, an explicit segment
count) for the chunked prefill, with many heads for the launch shapes that
depend on the head count, the same for decode steps, the draft replay and the
backward.  Each case is compared with the fp64 oracle (per sequence and per
16-token block for the prefill outputs), at the tolerance of the input dtype
(5e-5 on the precomputed-G path with fp32 inputs and 64-token chunks, where the fp32
rounding of G's chunk-local sums alone moves the result by up to 8e-6).  The hand-picked cases elsewhere cover the edges
one at a time; these mix them."""
import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
import oracle.backward as OB
from tests._gpu import (TOL, assert_states, assert_tokens, bwd_tol, dev, dev_inputs, f64_inputs, fwd_tol, grad_errors,
                        host64, rel_l2, say)

pytestmark = pytest.mark.gpu

DIMS = (16, 32, 64, 128)
LENGTHS = (0, 1, 15, 17, 63, 64, 65, 129, 200, 333, 512)
PATHS = ("z", "G", "prologue", "segmented")


def _prefill_cases(n=48, seed=20261):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["f32", "bf16"]))
        if i % 6 == 0:  # the matrix-core kernel's shape, regularly
            dtype, dk, dv, chunk = "bf16", 128, 128, 64
        else:
            dk, dv, chunk = int(rng.choice(DIMS)), int(rng.choice(DIMS)), int(rng.choice([16, 64]))
        path = str(rng.choice(PATHS))
        T = int(rng.choice(LENGTHS))
        if path == "segmented" and T == 0:
            T = 65
        cases.append(dict(
            B=int(rng.integers(1, 4)), H=int(rng.integers(1, 7)), T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype,
            path=path, segs=int(rng.integers(1, 7)), s0=float(rng.choice([0.0, 0.2])),
            zm=float(rng.choice([0.0, -3.0, 2.0])), g_min=float(rng.choice([-5.0, -4.5, -2.0, 0.0])),
            scale=float(rng.choice([1.0, 0.125])), o_bf16=bool(dtype == "bf16" and rng.integers(0, 2)),
            seed=7000 + i))
    return cases


def _id(c):
    return (f"{c['path']}-{c['dtype']}-B{c['B']}H{c['H']}T{c['T']}-d{c['dk']}x{c['dv']}-c{c['chunk']}"
            f"-g{c['g_min']}-s{c['segs']}")


def _wide_cases(n=8, seed=20264):
    """Many heads (B*H from 8 to 512): the launch shapes that depend on the head count
    (value-column slices of the matrix-core and tile kernels, segment counts chosen by
    the library)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["f32", "bf16"]))
        if i % 2 == 0:
            dk = dv = 128
            chunk = 64
        else:
            dk, dv, chunk = int(rng.choice(DIMS)), int(rng.choice(DIMS)), int(rng.choice([16, 64]))
        cases.append(dict(B=int(rng.choice([1, 2, 4, 8])), H=int(rng.choice([8, 16, 32, 64])),
                          T=int(rng.choice([17, 64, 100])), dk=dk, dv=dv, chunk=chunk, dtype=dtype,
                          path=str(rng.choice(["z", "G"])), segs=1, s0=0.2, zm=float(rng.choice([0.0, -3.0])),
                          g_min=-5.0, scale=1.0, o_bf16=False, seed=7300 + i))
    return cases


# a precomputed-G case with a whole fast-decaying 64-token chunk (|G| past 200), fp32
G_ROUNDING_CASE = dict(B=4, H=64, T=64, dk=128, dv=128, chunk=64, dtype="f32", path="G", segs=1, s0=0.2, zm=0.0,
                       g_min=-5.0, scale=1.0, o_bf16=False, seed=7312)


@pytest.mark.parametrize("c", _prefill_cases() + _wide_cases() + [G_ROUNDING_CASE], ids=_id)
def test_random_prefill_vs_oracle(c):
    say(f"case random prefill {c}")
    spec = ki.small_spec(c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"], c["dtype"], seed=c["seed"],
                         s0_std=c["s0"], z_mean=c["zm"], raw=(c["path"] == "prologue"))
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, c["dtype"])
    o_dtype = torch.bfloat16 if c["o_bf16"] else torch.float32
    g_min, chunk, scale = c["g_min"], c["chunk"], c["scale"]
    args = (dd["q"], dd["k"], dd["v"], dd["beta"])
    if c["path"] == "z":
        o, S = kda.chunk_fwd_z(*args, dd["z"], dd["A"], g_min, chunk, S_in=dd["S0"], o_dtype=o_dtype, scale=scale)
    elif c["path"] == "G":
        G = kda.gate(dd["z"], dd["A"], g_min, chunk)
        o, S = kda.chunk_fwd(*args, G, chunk, S_in=dd["S0"], o_dtype=o_dtype, scale=scale)
    elif c["path"] == "prologue":
        o, S = kda.chunk_fwd_z_prologue(*args, dd["z"], dd["A"], g_min, chunk, S_in=dd["S0"], o_dtype=o_dtype,
                                        scale=scale)
    else:
        o, S = kda.chunk_fwd_z_segmented(*args, dd["z"], dd["A"], c["segs"], g_min, chunk, S_in=dd["S0"],
                                         o_dtype=o_dtype, scale=scale)
    torch.cuda.synchronize()
    assert o.dtype == o_dtype
    f = f64_inputs(d, c["dtype"])
    run = oracle.forward_z_prologue if c["path"] == "prologue" else oracle.forward_z
    o_ref, S_ref = run(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], g_min, f["S0"], scale)
    tol = fwd_tol(c["dtype"], c["path"], chunk)
    assert_tokens("o", host64(o), o_ref, tol, block=16)
    assert_states("S", host64(S), S_ref, tol)


def _decode_cases(n=16, seed=20262):
    rng = np.random.default_rng(seed)
    return [dict(N=int(rng.integers(1, 9)), H=int(rng.integers(1, 5)), dk=int(rng.choice(DIMS)),
                 dv=int(rng.choice(DIMS)), dtype=str(rng.choice(["f32", "bf16"])), prologue=bool(rng.integers(0, 2)),
                 g_min=float(rng.choice([-5.0, -2.0, 0.0])), scale=float(rng.choice([1.0, 0.125])), seed=7100 + i)
            for i in range(n)]


@pytest.mark.parametrize("c", _decode_cases(),
                         ids=lambda c: f"{c['dtype']}-N{c['N']}H{c['H']}-d{c['dk']}x{c['dv']}-p{int(c['prologue'])}")
def test_random_decode_vs_oracle(c):
    say(f"case random decode {c}")
    spec = ki.DecodeSpec("decode_random", N=c["N"], H=c["H"], dk=c["dk"], dv=c["dv"], steps=5, dtype=c["dtype"],
                         s_std=0.1, seed=c["seed"], raw=c["prologue"])
    d = ki.decode_inputs(spec)
    f = f64_inputs(d, c["dtype"])
    run = oracle.decode_prologue if c["prologue"] else oracle.decode
    o_ref, S_ref = run(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"], c["g_min"], c["scale"])
    dd = dev_inputs(d, c["dtype"])
    S = dd["S0"].clone()
    step = kda.decode_step_prologue if c["prologue"] else kda.decode_step
    outs = [step(dd["q"][s], dd["k"][s], dd["v"][s], dd["z"][s], dd["beta"][s], dd["A"], S, c["g_min"],
                 o_dtype=torch.float32, scale=c["scale"]) for s in range(spec.steps)]
    torch.cuda.synchronize()
    o = torch.stack(outs)
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL[c["dtype"]] and es <= TOL[c["dtype"]]


def _backward_cases(n=16, seed=20263):
    rng = np.random.default_rng(seed)
    return [dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                 T=int(rng.choice([1, 15, 16, 17, 64, 65, 100, 150])), dk=int(rng.choice(DIMS)),
                 dv=int(rng.choice(DIMS)), dtype=str(rng.choice(["f32", "bf16"])), s0=float(rng.choice([0.0, 0.2])),
                 zm=float(rng.choice([0.0, -4.0, 2.0])), with_dS=bool(rng.integers(0, 2)),
                 scale=float(rng.choice([1.0, 0.125])), g_min=float(rng.choice([-5.0, -2.0, 0.0])), seed=7200 + i)
            for i in range(n)]


@pytest.mark.parametrize("c", _backward_cases(),
                         ids=lambda c: f"{c['dtype']}-B{c['B']}H{c['H']}T{c['T']}-d{c['dk']}x{c['dv']}-g{c['g_min']}")
def test_random_backward_vs_oracle(c):
    say(f"case random backward {c}")
    spec = ki.small_spec(c["B"], c["H"], c["T"], c["dk"], c["dv"], 64, c["dtype"], seed=c["seed"], s0_std=c["s0"],
                         z_mean=c["zm"])
    d = ki.prefill_inputs(spec)
    rng = np.random.default_rng([c["seed"], 1])
    do = ki.round_storage(rng.standard_normal((spec.B, spec.T, spec.H, spec.dv)), spec.dtype)
    dS = ki.round_to_f32(rng.standard_normal((spec.B, spec.H, spec.dk, spec.dv)) * 0.1) if c["with_dS"] else None
    dd = dev_inputs(d, spec.dtype)
    g = kda.chunk_bwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], dev(do, spec.dtype),
                        None if dS is None else dev(dS, "f32"), c["g_min"], dd["S0"], c["scale"])
    torch.cuda.synchronize()
    f = f64_inputs(d, spec.dtype)
    ref = OB.backward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], ki.to_f64(do, spec.dtype),
                        None if dS is None else dS.astype(np.float64), c["g_min"], f["S0"], c["scale"])
    errs = grad_errors(g, ref, ("dq", "dk", "dv", "dbeta", "dz", "dA", "dS_in"))
    say("  rel-L2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= bwd_tol(c["dtype"], n), (n, e)


def _replay_cases(n=8, seed=20265):
    rng = np.random.default_rng(seed)
    return [dict(n_draft=int(rng.integers(1, 20)), N=int(rng.integers(1, 9)), H=int(rng.integers(1, 4)),
                 dk=int(rng.choice(DIMS)), dv=int(rng.choice(DIMS)), dtype=str(rng.choice(["f32", "bf16"])),
                 g_min=float(rng.choice([-5.0, -2.0, 0.0])), scale=float(rng.choice([1.0, 0.125])), seed=7400 + i)
            for i in range(n)]


@pytest.mark.parametrize("c", _replay_cases(),
                         ids=lambda c: f"{c['dtype']}-n{c['n_draft']}-N{c['N']}H{c['H']}-d{c['dk']}x{c['dv']}")
def test_random_replay_vs_oracle(c):
    say(f"case random replay {c}")
    spec = ki.DecodeSpec("replay_random", N=c["N"], H=c["H"], dk=c["dk"], dv=c["dv"], steps=c["n_draft"],
                         dtype=c["dtype"], s_std=0.1, seed=c["seed"])
    d = ki.decode_inputs(spec)
    acc = np.random.default_rng([c["seed"], 2]).integers(0, c["n_draft"] + 1, size=c["N"]).astype(np.int32)
    f = f64_inputs(d, c["dtype"])
    o_ref, S_ref = oracle.replay(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"], acc, c["g_min"],
                                 c["scale"])
    dd = dev_inputs(d, c["dtype"])
    snap = dd["S0"].clone()
    o, S = kda.decode_replay(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["A"], dd["S0"],
                             torch.from_numpy(acc).to(dd["A"].device), c["g_min"], o_dtype=torch.float32,
                             scale=c["scale"])
    torch.cuda.synchronize()
    assert torch.equal(dd["S0"], snap)  # the snapshot is read only
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  accepted {acc.tolist()} rel-L2 o={eo:.3e} S_commit={es:.3e}")
    assert eo <= TOL[c["dtype"]] and es <= TOL[c["dtype"]]
