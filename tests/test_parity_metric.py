"""The parity metric of the GPU tests, on the CPU: a single wrong 64-token
block in a million-token sequence, or one wrong sequence among many, fails
``assert_tokens`` although the whole-tensor relative L2 stays under the
tolerance."""
import numpy as np
import pytest

from tests._gpu import assert_states, assert_tokens, token_report


def _noisy(ref, rel, rng):
    return ref + rel * rng.standard_normal(ref.shape) * np.sqrt(np.mean(ref * ref))


def test_one_wrong_block_in_a_million_tokens_fails():
    rng = np.random.default_rng(0)
    T = 1 << 20
    ref = rng.standard_normal((1, T, 1, 8))
    x = _noisy(ref, 4e-3, rng)
    assert_tokens("baseline", x, ref, 1e-2)
    bad = x.copy()
    t0 = 64 * 12345
    bad[:, t0:t0 + 64] = 0.0  # one chunk entirely wrong (its outputs lost)
    r = token_report(bad, ref)
    assert r["whole"] < 1e-2            # the whole-tensor metric does not see it ...
    assert r["block_at"] == (0, t0, 0)  # ... the per-block one does, at the right place
    with pytest.raises(AssertionError, match="block"):
        assert_tokens("one wrong block", bad, ref, 1e-2)


def test_ragged_tail_is_checked_with_the_last_block():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((2, 64 * 5 + 7, 3, 4))
    x = ref.copy()
    x[1, -3:, 2] += 1.0  # only the last 3 tokens of one sequence
    r = token_report(x, ref)
    assert r["blocks"] == 2 * 5 * 3
    assert r["block_at"] == (1, 64 * 4, 2) and r["block_max"] > 0.1  # the last block spans 71 tokens
    with pytest.raises(AssertionError):
        assert_tokens("tail", x, ref, 1e-2)
    short = rng.standard_normal((1, 40, 1, 4))  # shorter than one block: one block
    assert token_report(short, short)["blocks"] == 1


def test_one_wrong_sequence_fails():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((4, 512, 32, 4))
    x = _noisy(ref, 1e-3, rng)
    x[3, :, 17] = _noisy(ref[3, :, 17], 5e-2, rng)
    r = token_report(x, ref)
    assert r["whole"] < 1e-2 and r["pair_at"] == (3, 17)
    with pytest.raises(AssertionError):
        assert_tokens("one wrong sequence", x, ref, 1e-2)


def test_state_per_sequence_and_exact_zero():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((2, 64, 4, 4))
    x = ref.copy()
    x[1, 63] *= 1.2
    with pytest.raises(AssertionError):
        assert_states("one wrong state", x, ref, 1e-2)
    z = np.zeros((1, 64, 1, 4))
    assert token_report(z, z)["block_max"] == 0.0
    nz = z.copy()
    nz[0, 5, 0, 1] = 1e-30  # any nonzero output where the reference is exactly zero
    assert token_report(nz, z)["block_max"] == np.inf


def test_small_sequences_are_measured_against_the_typical_magnitude():
    """A sequence whose outputs are 100 times smaller than the rest, off by rounding at
    the rest's magnitude, passes; the same sequence off by more than the tolerance times
    the typical magnitude, or set to zero, fails."""
    rng = np.random.default_rng(4)
    ref = rng.standard_normal((1, 256, 4, 8))
    ref[0, :, 2] *= 1e-2
    x = _noisy(ref, 1e-3, rng)  # noise at 1e-3 of the tensor's RMS everywhere
    r = token_report(x, ref)
    assert r["pair_max"] < 2e-3 and r["block_max"] < 3e-3  # the small head: 1e-1 of its own norm
    wrong = x.copy()
    wrong[0, :, 2] += 3e-2 * np.sqrt(np.mean(ref * ref))
    with pytest.raises(AssertionError):
        assert_tokens("small sequence off", wrong, ref, 1e-2)
    lost = x.copy()
    lost[0, 64:128, 1] = 0.0  # a block of a typical head lost
    r = token_report(lost, ref)
    assert r["block_at"] == (0, 64, 1) and r["block_max"] > 0.5
    with pytest.raises(AssertionError, match="rel-L2"):
        assert_tokens("lost", lost, ref, 1e-2)


def test_non_finite_output_fails():
    ref = np.ones((1, 64, 1, 4))
    x = ref.copy()
    x[0, 3, 0, 0] = np.nan
    with pytest.raises(AssertionError, match="non-finite"):
        token_report(x, ref)


def test_fp32_rounding_of_G_alone_moves_the_fp64_result():
    """What the fp32 bar of the precomputed-G path with 64-token chunks (``fwd_tol``: 5e-5)
    has to admit, measured without any kernel: the fp64 recurrence driven by the per-token
    decays that G's chunk-local sums imply once rounded to fp32 (summed in fp32, in token
    order), against the same recurrence on the exact decays.  A whole fast-decaying chunk
    takes |G| past 200, where fp32 numbers are 1.5e-5 apart.  With 16-token chunks the same
    rounding is far below the 1e-5 bar."""
    import kda_inputs as ki
    import oracle
    from tests._gpu import f64_inputs, fwd_tol, state_report

    def moved(chunk):
        spec = ki.small_spec(4, 64, 64, 128, 128, chunk, "f32", seed=7312, s0_std=0.2)
        f = f64_inputs(ki.prefill_inputs(spec), "f32")
        g = oracle.gate(f["z"], f["A"], -5.0, 1)
        g32 = g.astype(np.float32)
        G32 = np.empty_like(g32)
        for t in range(spec.T):
            G32[:, t] = g32[:, t] if t % chunk == 0 else (G32[:, t - 1] + g32[:, t]).astype(np.float32)
        g_impl = G32.astype(np.float64)
        g_impl[:, 1:] -= np.where((np.arange(1, spec.T) % chunk == 0)[None, :, None, None], 0.0,
                                  G32[:, :-1].astype(np.float64))
        _, S_ref = oracle.recurrence(f["q"], f["k"], f["v"], f["beta"], g, f["S0"])
        _, S_g32 = oracle.recurrence(f["q"], f["k"], f["v"], f["beta"], g_impl, f["S0"])
        return state_report(S_g32, S_ref)["pair_max"], float(np.abs(G32).max())

    m64, gmax = moved(64)
    m16, _ = moved(16)
    print(f"chunk 64: max |G| {gmax:.1f}, worst (b, h) state moved by {m64:.2e}; chunk 16: {m16:.2e}")
    assert gmax > 200.0
    assert 3e-6 < m64 < fwd_tol("f32", "G", 64) / 4  # near the input dtype's 1e-5, well inside 5e-5
    assert m16 < fwd_tol("f32", "G", 16) / 4
