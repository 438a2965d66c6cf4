"""GPU parity of the speculative-decoding replay (kda_decode_replay) against the
fp64 oracle ("Kimi K3: architecture, derivations and a pinned-source audit",
section 10.3), and its equivalence with stepping kda_decode_step."""
import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import DEV, TOL, dev_inputs, f64_inputs, host64, rel_l2, say

pytestmark = pytest.mark.gpu


def _case(n_draft, N, H, dk, dv, dtype, seed, s_std=0.1):
    spec = ki.DecodeSpec("replay", N=N, H=H, dk=dk, dv=dv, steps=n_draft, dtype=dtype, s_std=s_std, seed=seed)
    return spec, ki.decode_inputs(spec)


def _accepted(N, n_draft, seed):
    rng = np.random.default_rng(seed)
    acc = rng.integers(0, n_draft + 1, size=N)
    acc[0] = 0
    if N > 1:
        acc[1] = n_draft
    return acc.astype(np.int32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16), (128, 128)])
def test_replay_small(dtype, dk, dv):
    n_draft, N, H = 7, 6, 3
    spec, d = _case(n_draft, N, H, dk, dv, dtype, seed=41 + dk + dv)
    acc = _accepted(N, n_draft, 5)
    say(f"case replay n_draft={n_draft} N={N} H={H} dk={dk} dv={dv} {dtype} accepted={acc.tolist()}")
    f = f64_inputs(d, dtype)
    o_ref, S_ref = oracle.replay(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"], acc)
    dd = dev_inputs(d, dtype)
    snap = dd["S0"]
    snap_before = snap.clone()
    o, S = kda.decode_replay(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["A"], snap,
                             torch.from_numpy(acc).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(snap, snap_before)                       # the snapshot is only read
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S_commit={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    assert torch.equal(S[0], snap[0])                           # nothing accepted: the snapshot itself


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("g_min,n_draft", [(-5.0, 5), (-6.0, 19)])
def test_replay_equals_decode_steps(dtype, g_min, n_draft):
    """Replaying every draft gives, bit for bit, what n_draft kda_decode_step calls give
    (19 drafts span three staging groups)."""
    N, H, dk, dv = 4, 2, 128, 128
    spec, d = _case(n_draft, N, H, dk, dv, dtype, seed=77)
    say(f"case replay==decode {dtype} g_min={g_min} n_draft={n_draft}")
    dd = dev_inputs(d, dtype)
    acc = torch.full((N,), n_draft, dtype=torch.int32, device=DEV)
    o, S = kda.decode_replay(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["A"], dd["S0"], acc, g_min=g_min)
    S_dec = dd["S0"].clone()
    outs = [kda.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["z"][t], dd["beta"][t], dd["A"], S_dec,
                            g_min=g_min) for t in range(n_draft)]
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(outs), o)
    assert torch.equal(S_dec, S)


def test_replay_nothing_drafted():
    N, H, dk, dv = 3, 2, 64, 64
    spec, d = _case(1, N, H, dk, dv, "f32", seed=3)
    say("case replay n_draft=0")
    dd = dev_inputs(d, "f32")
    empty = lambda t: t[:0].contiguous()
    acc = torch.zeros(N, dtype=torch.int32, device=DEV)
    o, S = kda.decode_replay(*(empty(dd[n]) for n in ("q", "k", "v", "z", "beta")), dd["A"], dd["S0"], acc)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and torch.equal(S, dd["S0"])


def test_replay_decode_workload_sampled():
    """The decode workload's shape (N = 256, H = 32, d = 128), eight drafts, random
    accepted prefixes; the oracle runs on a sample of sequences."""
    base = ki.DECODE_256
    n_draft = 8
    spec, d = _case(n_draft, base.N, base.H, base.dk, base.dv, "bf16", seed=base.seed + 7, s_std=base.s_std)
    acc = _accepted(base.N, n_draft, 11)
    say(f"case replay N={base.N} H={base.H} n_draft={n_draft} bf16")
    dd = dev_inputs(d, "bf16")
    o, S = kda.decode_replay(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["A"], dd["S0"],
                             torch.from_numpy(acc).to(DEV))
    torch.cuda.synchronize()
    sel = [0, 1, 77, 255]
    f = f64_inputs(d, "bf16")
    cut = lambda a: a[:, sel] if a.ndim >= 3 else a
    o_ref, S_ref = oracle.replay(cut(f["q"]), cut(f["k"]), cut(f["v"]), cut(f["z"]), f["beta"][:, sel], f["A"],
                                 f["S0"][sel], acc[sel])
    eo = rel_l2(host64(o)[:, sel], o_ref)
    es = rel_l2(host64(S)[sel], S_ref)
    say(f"  sampled rel-L2 o={eo:.3e} S_commit={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_three_groups_vs_oracle(dtype):
    """19 drafts (three staging groups), accepted prefixes inside every group, against
    the oracle."""
    n_draft, N, H, dk, dv = 19, 8, 2, 64, 64
    spec, d = _case(n_draft, N, H, dk, dv, dtype, seed=91)
    acc = np.array([0, 19, 3, 8, 9, 15, 16, 12], dtype=np.int32)
    say(f"case replay n_draft={n_draft} {dtype} accepted={acc.tolist()}")
    f = f64_inputs(d, dtype)
    o_ref, S_ref = oracle.replay(f["q"], f["k"], f["v"], f["z"], f["beta"], f["A"], f["S0"], acc)
    dd = dev_inputs(d, dtype)
    o, S = kda.decode_replay(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["A"], dd["S0"],
                             torch.from_numpy(acc).to(DEV))
    torch.cuda.synchronize()
    eo, es = rel_l2(host64(o), o_ref), rel_l2(host64(S), S_ref)
    say(f"  rel-L2 o={eo:.3e} S_commit={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    for i in range(N):
        assert rel_l2(host64(S[i]), S_ref[i]) <= TOL[dtype], i
