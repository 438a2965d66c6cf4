"""The allocation-free prefill (kda_chunk_fwd_z_noalloc) through the C ABI,
against kda_chunk_fwd_z with a caller workspace on the same inputs: two calls in
a row on one device, the second on a smaller input, each bit for bit equal to
the workspace entry point (both run the same kernels, the static array only
replacing the workspace) and within the bf16 tolerance of the fp64 oracle on
every sequence and 64-token block.  A third call whose sizes need no scratch
memory checks the plain one-pass route of the same entry point."""
import ctypes

import pytest
import torch

import gated_delta_rule_11_amd as kda
import kda_inputs as ki
import oracle
from tests._gpu import TOL, assert_states, assert_tokens, dev_inputs, f64_inputs, host64, say

pytestmark = pytest.mark.gpu


def _noalloc(dd, spec, o, S_out):
    L = kda.lib()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = L.kda_chunk_fwd_z_noalloc(p(dd["q"]), p(dd["k"]), p(dd["v"]), p(dd["beta"]), p(dd["z"]), 1, p(dd["A"]),
                                   -5.0, p(dd["S0"]), p(o), 0, p(S_out), spec.B, spec.T, spec.H, spec.dk, spec.dv,
                                   spec.chunk, 1.0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.kda_status_string(st).decode()


@pytest.mark.parametrize("first", [True, False])
def test_noalloc_matches_workspace_entry_point(first):
    cases = [(1, 8, 4096, 0.3, -3.0), (1, 4, 64 * 30 + 19, 0.5, -6.0), (2, 64, 64 * 3 + 5, 0.2, 0.0)]
    if not first:
        cases = cases[::-1]  # the scratch array keeps the last call's contents: both orders
    for B, H, T, s0, zm in cases:
        spec = ki.small_spec(B, H, T, 128, 128, 64, "bf16", seed=9900 + T, s0_std=s0, z_mean=zm)
        need = kda.chunk_fwd_workspace_bytes(B, T, H, 128, 128, 64)
        say(f"case noalloc B={B} H={H} T={T} (workspace need {need} bytes)")
        d = ki.prefill_inputs(spec)
        dd = dev_inputs(d, spec.dtype)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0") if need else None
        o_ref, S_ref = kda.chunk_fwd_z(dd["q"], dd["k"], dd["v"], dd["beta"], dd["z"], dd["A"], -5.0, 64,
                                       S_in=dd["S0"], o_dtype=torch.float32, workspace=ws)
        o = torch.full_like(o_ref, float("nan"))
        S = torch.full_like(S_ref, float("nan"))
        _noalloc(dd, spec, o, S)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        f = f64_inputs(d, spec.dtype)
        o64, S64 = oracle.forward_z(f["q"], f["k"], f["v"], f["beta"], f["z"], f["A"], -5.0, f["S0"])
        assert_tokens("noalloc o vs oracle", host64(o), o64, TOL["bf16"])
        assert_states("noalloc S vs oracle", host64(S), S64, TOL["bf16"])
