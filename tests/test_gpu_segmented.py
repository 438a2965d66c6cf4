"""GPU parity of the segment-parallel prefill (kda_chunk_fwd_z_segmented, and the
form kda_chunk_fwd_z and kda_chunk_fwd choose themselves for few, long sequences)
against the fp64 oracle, and against the one-pass GPU prefill on the same
inputs.  Tolerance: relative L2 1e-2 (bf16 inputs), separately for o and the
final state; the segmented form regroups the arithmetic, so it is compared to
the one-pass kernel at the same tolerance, not bit for bit (segments == 1 is
the one-pass kernel itself and is compared exactly)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import (DEV, TOL, assert_states, assert_tokens, dev_inputs, f64_inputs, fwd_tol, host64, rel_l2,
                        say, sub_inputs)

pytestmark = pytest.mark.gpu


def _spec(B, H, T, seed, z_scale=1.0, s0_std=0.0, z_mean=0.0):
    return ki.small_spec(B, H, T, 128, 128, 64, "bf16", seed=seed, z_scale=z_scale, s0_std=s0_std, z_mean=z_mean)


def _plain(dd, S0, o_dtype=torch.bfloat16):
    o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, 64, S_in=S0,
                           o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, S


def _seg(dd, S0, segments, o_dtype=torch.bfloat16, **kw):
    o, S = kda.chunk_fwd_z_segmented(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], segments, -5.0, 64,
                                     S_in=S0, o_dtype=o_dtype, **kw)
    torch.cuda.synchronize()
    return o, S


CASES = [  # B, H, T, segments, z_mean, s0_std
    (1, 2, 1024, 4, 0.0, 0.0),          # four equal segments, fast decay
    (1, 2, 1024, 4, -6.0, 0.0),         # the same with slow decay: segment boundaries carry state
    (1, 2, 1000, 3, -6.0, 0.5),         # ragged last chunk and last segment, given entry state
    (2, 3, 64 * 9 + 17, 7, -4.0, 0.5),  # seven segments over ten chunks (two chunks, last one short)
    (1, 1, 512, 8, -8.0, 1.0),          # one chunk per segment, slowest decay: transitions matter most
    (1, 2, 200, 100, -6.0, 0.5),        # more segments than chunks: one chunk each
    (1, 8, 64 * 16, 8, -6.0, 0.3),      # 64 (b, h, segment) units: four 32-column slices, XCD-grouped order
    (3, 5, 64 * 10 - 9, 5, -6.0, 0.3),  # 75 units: four 32-column slices, plain order; ragged end
]


@pytest.mark.parametrize("B,H,T,segs,zm,s0", CASES)
def test_segmented_vs_oracle(B, H, T, segs, zm, s0):
    spec = _spec(B, H, T, seed=4100 + T + segs, z_mean=zm, s0_std=s0)
    say(f"case segmented B={B} H={H} T={T} segments={segs} z_mean={zm} s0_std={s0}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    o, S = _seg(dd, dd["S0"], segs, o_dtype=torch.float32)
    f = f64_inputs(d, spec.dtype)
    o_ref, S_ref = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
    assert_tokens("segmented vs oracle, o", host64(o), o_ref, TOL["bf16"])
    assert_states("segmented vs oracle, S", host64(S), S_ref, TOL["bf16"])
    o1, S1 = _plain(dd, dd["S0"], o_dtype=torch.float32)
    assert_tokens("segmented vs one-pass kernel, o", host64(o), host64(o1), TOL["bf16"])
    assert_states("segmented vs one-pass kernel, S", host64(S), host64(S1), TOL["bf16"])
    if zm < 0:
        # the case is sensitive to the state carried into the last segment: the
        # oracle run over that segment alone, from the zero state, is far off
        nch = (T + 63) // 64
        t_last = ((nch - 1) // ((nch + segs - 1) // segs)) * ((nch + segs - 1) // segs) * 64
        cut = {n: np.ascontiguousarray(f[n][:, t_last:]) for n in ("q", "k", "v", "beta", "z")}
        o_cut, _ = oracle.forward_z(cut["q"], cut["k"], cut["v"], cut["beta"], cut["z"], f["A"], -5.0, None)
        gap = rel_l2(o_cut, o_ref[:, t_last:])
        say(f"  last segment from zero state: rel-L2 {gap:.3e} from the true outputs")
        assert gap > 10 * TOL["bf16"]


def test_one_segment_is_the_one_pass_kernel():
    spec = _spec(1, 2, 777, seed=4200, s0_std=0.5)
    say("case segments=1 T=777")
    dd = dev_inputs(ki.prefill_inputs(spec), spec.dtype)
    o, S = _seg(dd, dd["S0"], 1)
    o1, S1 = _plain(dd, dd["S0"])
    assert torch.equal(o, o1) and torch.equal(S, S1)


def test_in_place_state_and_no_state():
    spec = _spec(1, 2, 640, seed=4300, s0_std=0.5)
    say("case segments=5 in-place S and S_out=None")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    o_ref, S_ref = _seg(dd, dd["S0"], 5)
    S_io = dd["S0"].clone()
    o, S = _seg(dd, S_io, 5, S_out=S_io)
    assert S.data_ptr() == S_io.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    o2, S2 = _seg(dd, dd["S0"], 5, want_state=False)
    assert S2 is None and torch.equal(o2, o_ref)


def test_workspace_reuse_and_dirty_workspace():
    spec = _spec(2, 2, 900, seed=4400, s0_std=0.5)
    say("case segments=4 caller workspace, filled with garbage between calls")
    dd = dev_inputs(ki.prefill_inputs(spec), spec.dtype)
    need = kda.chunk_fwd_z_segmented_workspace_bytes(2, 2, 128, 128, 4)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws.fill_(0x7f)  # large finite fp32 values everywhere
    o1, S1 = _seg(dd, dd["S0"], 4, workspace=ws)
    ws.fill_(0x3c)
    o2, S2 = _seg(dd, dd["S0"], 4, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    with pytest.raises(kda.KDAError, match="WORKSPACE"):
        _seg(dd, dd["S0"], 4, workspace=ws[: need - 16])


def test_prefill_1m_slow_decay_segmented():
    """The million-token, 8-head prefill with slow decay (z centred at -6) in 64
    segments: against the one-pass kernel on every head and every 64-token
    block, and against the oracle on two heads."""
    spec = replace(ki.PREFILL_1M, name=ki.PREFILL_1M.name + "_slow", z_mean=-6.0)
    segs = 64
    say(f"case {spec.name}: segments={segs}, generating inputs")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, spec.dtype)
    say("  GPU runs (segmented, one-pass)")
    o, S = _seg(dd, dd["S0"], segs)
    o1, S1 = _plain(dd, dd["S0"])
    del dd
    for h in range(spec.H):
        assert_tokens(f"h={h} segmented vs one-pass kernel, o", host64(o[:, :, h:h + 1]), host64(o1[:, :, h:h + 1]),
                      TOL["bf16"], offset=(0, h))
    assert_states("segmented vs one-pass kernel, S", host64(S), host64(S1), TOL["bf16"])
    h0 = 2
    say(f"  oracle b=0 h=[{h0},{h0 + 2}) T={spec.T}")
    f = f64_inputs(sub_inputs(d, 0, 1, h0, h0 + 2), spec.dtype)
    o_ref, S_ref = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
    del f
    assert_tokens("segmented vs oracle, o", host64(o[:, :, h0:h0 + 2]), o_ref, TOL["bf16"], offset=(0, h0))
    assert_states("segmented vs oracle, S", host64(S[:, h0:h0 + 2]), S_ref, TOL["bf16"], offset=(0, h0))
    del o, S, o1, S1
    torch.cuda.empty_cache()


# The tile kernel (every shape but bf16 d = 128 chunk 64) runs the same three passes;
# the transitions have d_k columns whatever d_v is.  Tolerance of the input dtype.
GEN_CASES = [  # B, H, T, dk, dv, chunk, dtype, segments, z_mean, s0_std
    (1, 2, 1000, 128, 128, 64, "f32", 4, -6.0, 0.5),   # ragged last chunk and segment, slow decay
    (1, 3, 777, 64, 32, 16, "bf16", 5, -6.0, 0.3),     # d_k > d_v, chunk 16
    (2, 2, 640, 32, 128, 64, "f32", 3, -4.0, 0.2),     # d_k < d_v
    (1, 1, 300, 16, 16, 16, "f32", 8, -8.0, 1.0),      # smallest dims, slowest decay, many segments
    (1, 2, 1024, 128, 128, 16, "bf16", 6, -6.0, 0.0),  # bf16, chunk 16
]


@pytest.mark.parametrize("B,H,T,dk,dv,chunk,dtype,segs,zm,s0", GEN_CASES)
def test_segmented_tile_kernel_vs_oracle(B, H, T, dk, dv, chunk, dtype, segs, zm, s0):
    assert not kda.chunk_uses_mfma(torch.bfloat16 if dtype == "bf16" else torch.float32, dk, dv, chunk)
    spec = ki.small_spec(B, H, T, dk, dv, chunk, dtype, seed=4300 + T + dk + segs, z_mean=zm, s0_std=s0)
    say(f"case segmented tile kernel B={B} H={H} T={T} dk={dk} dv={dv} chunk={chunk} {dtype} segments={segs}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    o, S = kda.chunk_fwd_z_segmented(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], segs, -5.0, chunk,
                                     S_in=dd["S0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    f = f64_inputs(d, dtype)
    o_ref, S_ref = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
    assert_tokens("segmented vs oracle, o", host64(o), o_ref, TOL[dtype], block=16)
    assert_states("segmented vs oracle, S", host64(S), S_ref, TOL[dtype])


def test_tile_kernel_picks_segments_itself():
    """fp32, d = 128, 8 heads of 4096 tokens: kda_chunk_fwd_z cuts each sequence into
    16 segments itself (its workspace query says so) and matches the oracle."""
    B, H, T = 1, 8, 4096
    assert kda.chunk_fwd_workspace_bytes(B, T, H, 128, 128, 64) > 0
    spec = ki.small_spec(B, H, T, 128, 128, 64, "f32", seed=4400, z_mean=-6.0, s0_std=0.3)
    say("case fp32 d=128 B=1 H=8 T=4096 through kda_chunk_fwd_z (automatic segments)")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, "f32")
    o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, 64, S_in=dd["S0"])
    torch.cuda.synchronize()
    f = f64_inputs(d, "f32")
    o_ref, S_ref = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
    assert_tokens("automatic segments vs oracle, o", host64(o), o_ref, TOL["f32"])
    assert_states("automatic segments vs oracle, S", host64(S), S_ref, TOL["f32"])


@pytest.mark.parametrize("entry", ["precomputed G", "fused prologue"])
@pytest.mark.parametrize("dtype,dk,dv,chunk", [("bf16", 128, 128, 64), ("f32", 128, 128, 64), ("bf16", 64, 32, 16)])
def test_other_entry_points_pick_segments_themselves(entry, dtype, dk, dv, chunk):
    """kda_gate then kda_chunk_fwd, and kda_chunk_fwd_z_prologue on raw inputs, on four
    sequences of 2085 tokens: each runs the segment-parallel form itself (eight segments;
    the matrix-core kernel for the first shape, the tile kernel for the others), with slow
    decay and a given entry state so that the segment boundaries carry state, and matches
    the oracle per sequence and block."""
    B, H, T = 1, 4, 2085
    assert kda.chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk) > 0
    prologue = entry == "fused prologue"
    spec = ki.small_spec(B, H, T, dk, dv, chunk, dtype, seed=4500 + dk + chunk + prologue, z_mean=-6.0, s0_std=0.3,
                         raw=prologue)
    say(f"case {entry}, automatic segments: B={B} H={H} T={T} dk={dk} dv={dv} chunk={chunk} {dtype}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    if prologue:
        o, S = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, chunk,
                                        S_in=dd["S0"], o_dtype=torch.float32)
    else:
        G = kda.gate(dd["z"], dd["A"], -5.0, chunk)
        o, S = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], G, chunk, S_in=dd["S0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    f = f64_inputs(d, dtype)
    run = oracle.forward_z_prologue if prologue else oracle.forward_z
    o_ref, S_ref = run(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
    tol = fwd_tol(dtype, "prologue" if prologue else "G", chunk)
    assert_tokens(f"automatic segments ({entry}) vs oracle, o", host64(o), o_ref, tol, block=16)
    assert_states(f"automatic segments ({entry}) vs oracle, S", host64(S), S_ref, tol)
