"""GPU parity of the fp32 matrix-core prefill (every shape outside the bf16
d = 128, chunk 64 kernel) at head counts large enough that the library picks
its 32- and 64-value-column slices (the smaller tests run 16-column slices):
B*H >= 64 gives 32-column slices of dv >= 64, B*H >= 128 gives 64-column slices
of dv = 128.  Ragged T, every entry path (fused gate, precomputed G, fused
prologue), per-sequence and per-block relative L2 against the fp64 oracle, at
the tolerance of the input dtype (fp32 inputs: fp32 products throughout; bf16
inputs: bf16 products with fp32 accumulation)."""
import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import TOL, assert_states, assert_tokens, dev_inputs, f64_inputs, host64, say

pytestmark = pytest.mark.gpu

CASES = [  # B, H, T, dk, dv, chunk, dtype, path, s0
    (4, 32, 83, 128, 128, 64, "f32", "z", 0.3),      # 64-column slices
    (2, 64, 61, 128, 128, 16, "bf16", "G", 0.0),     # 64-column slices, chunk 16, precomputed G
    (4, 32, 100, 64, 64, 64, "bf16", "prologue", 0.2),  # 32-column slices, fused prologue
    (8, 32, 45, 64, 32, 16, "f32", "z", 0.0),        # 32-column slices of dv = 32
    (2, 64, 77, 32, 128, 64, "bf16", "G", 0.1),      # 64-column slices, dk 32
]


@pytest.mark.parametrize("B,H,T,dk,dv,chunk,dtype,path,s0", CASES)
def test_wide_grid_vs_oracle(B, H, T, dk, dv, chunk, dtype, path, s0):
    assert not kda.chunk_uses_mfma(torch.bfloat16 if dtype == "bf16" else torch.float32, dk, dv, chunk)
    spec = ki.small_spec(B, H, T, dk, dv, chunk, dtype, seed=6200 + T + dk + dv, s0_std=s0,
                         raw=(path == "prologue"))
    say(f"case wide grid B={B} H={H} T={T} dk={dk} dv={dv} chunk={chunk} {dtype} path={path} s0={s0}")
    d = ki.prefill_inputs(spec)
    dd = dev_inputs(d, dtype)
    if path == "z":
        o, S = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, chunk, S_in=dd["S0"])
    elif path == "G":
        G = kda.gate(dd["z"], dd["A"], -5.0, chunk)
        o, S = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], G, chunk, S_in=dd["S0"])
    else:
        o, S = kda.chunk_fwd_z_prologue(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, chunk,
                                        S_in=dd["S0"])
    torch.cuda.synchronize()
    f = f64_inputs(d, dtype)
    run = oracle.forward_z_prologue if path == "prologue" else oracle.forward_z
    o_ref, S_ref = run(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
    assert o.dtype == torch.float32
    assert_tokens("o", host64(o), o_ref, TOL[dtype], block=16)
    assert_states("S", host64(S), S_ref, TOL[dtype])
