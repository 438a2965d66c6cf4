"""Helpers for the GPU parity tests: storage arrays -> device tensors, the
relative-L2 metric, and oracle runs on the same rounded inputs.

Parity is judged per sequence and per 64-token block, not only over a whole
tensor: at a million tokens one 64-token block is 1/16384 of the output, so a
block that came out entirely wrong would barely move a whole-tensor relative
L2.  ``assert_tokens`` therefore checks the relative L2 of every (b, h)
sequence and of every 64-token block of it, and ``assert_states`` that of
every (b, h) state, each against the same tolerance.

A sequence or block whose outputs are smaller than the tensor's typical
magnitude is measured against that typical magnitude instead of its own (its
error norm over the norm it would have at the tensor's RMS per element): an
output that is a short sum of products can be far smaller than the terms that
form it (one token's output is beta (q . k) v), and rounding of those terms,
at the level the dtype allows, is then a large fraction of it.  A wrong block
still fails: its error is of the order of the typical magnitude."""
from __future__ import annotations

import sys

import numpy as np
import torch

import kda_inputs as ki

DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 1e-2}
BLOCK = 64


def grad_errors(g: dict, ref: dict, names) -> dict:
    """Relative L2 of each gradient against the fp64 reference.  A gradient whose reference
    is exactly zero (a structural zero: dz and dA with one token and a zero initial state,
    where the state that the decay acts on is zero) cannot come out exactly zero from
    rounded arithmetic; it is measured by its largest magnitude over the largest magnitude
    among the call's non-zero reference gradients."""
    refs = {n: np.asarray(ref[n], np.float64) for n in names}
    gots = {n: host64(g[n]) for n in names}
    scale = max([float(np.abs(r).max()) for r in refs.values() if r.size and np.any(r)] or [0.0])
    out = {}
    for n in names:
        r, x = refs[n], gots[n]
        if r.size and not np.any(r) and scale > 0.0:
            assert np.all(np.isfinite(x)), f"non-finite values in {n}"
            out[n] = float(np.abs(x).max()) / scale
        else:
            out[n] = rel_l2(x, r)
    return out


def bwd_tol(dtype: str, name: str) -> float:
    """Relative-L2 bar of one gradient of the backward.  The gate's derivatives (dz and
    its sum over tokens, dA) are formed in the chunk form from per-token terms of dG that
    cancel (the key terms scaled by e^G and by e^-G); with fp32 arithmetic the terms'
    rounding is amplified by that cancellation (measured up to 5.5e-6 for dz and 2.3e-5
    for dA on a saturated-gate case whose fp64 gradients move by 1.5e-7 under fp32-sized
    input perturbations), so their fp32 bar is 1e-4.  Every other gradient keeps the
    input dtype's bar."""
    if dtype == "f32" and name in ("dz", "dA"):
        return 1e-4
    return TOL[dtype]


def fwd_tol(dtype: str, path: str, chunk: int) -> float:
    """Relative-L2 bar of a prefill.  On the precomputed-G path (``kda_gate``, then
    ``kda_chunk_fwd``) with fp32 inputs and 64-token chunks it is 5e-5: G holds
    chunk-local sums of the per-token log-decay, up to 64 |g_min| = 320 in magnitude,
    where consecutive fp32 numbers are 3.05e-5 apart, and every decay factor comes from
    a difference of two such sums, so the rounding of G alone (no kernel involved) moves
    the fp64 result by up to 8e-6 per (b, h) state in seeded cases
    (``tests/test_parity_metric.py``).  With 16-token chunks (|G| <= 80) and on the
    paths that form decays from per-token factors, the input dtype's bar holds."""
    if dtype == "f32" and path == "G" and chunk > 16:
        return 5e-5
    return TOL[dtype]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage numpy array (uint16 bf16 bits or float32) -> contiguous device tensor."""
    if arr is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(DEV)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.array_equal(x, ref) else float("inf")
    return float(np.linalg.norm(x - ref) / nr)


def _ratio(d2: np.ndarray, r2: np.ndarray) -> np.ndarray:
    """sqrt(d2 / r2) elementwise; 0 where both are 0, inf where only r2 is."""
    out = np.zeros(np.broadcast(d2, r2).shape)
    nz = r2 > 0
    out[nz] = np.sqrt(d2[nz] / r2[nz])
    out[(~nz) & (d2 > 0)] = np.inf
    return out


def token_report(x: np.ndarray, ref: np.ndarray, block: int = BLOCK) -> dict:
    """x, ref [B, T, H, d]: relative L2 over the whole tensor, per (b, h)
    sequence and per (b, h, block of ``block`` tokens; the last block also takes
    the remainder of T, so it holds ``block`` to 2 ``block`` - 1 tokens), each of
    the latter two with its reference energy floored at the tensor's mean energy
    per element times its element count; the largest absolute error and where
    it is."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape and x.ndim == 4, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    B, T, H, _ = x.shape
    diff = x - ref
    d2 = np.einsum("bthc,bthc->bth", diff, diff)
    r2 = np.einsum("bthc,bthc->bth", ref, ref)
    # blocks of `block` tokens; a shorter remainder joins the last full block (a
    # handful of tokens is too few for a relative norm: single outputs can be small
    # where the terms that form them are not)
    nb = max(1, T // block)
    starts = np.arange(nb) * block
    d2b = np.add.reduceat(d2, starts, axis=1) if T else np.zeros((B, 1, H))  # [B, nb, H]
    r2b = np.add.reduceat(r2, starts, axis=1) if T else np.zeros((B, 1, H))
    # the floor: the energy the sequence or block would have at the tensor's mean energy
    # per element (0 when the whole reference is zero: then only exact zeros pass)
    e_mean = float(r2.sum()) / max(1, x.size)
    n_blk = np.diff(np.append(starts, T)) if T else np.zeros(1)  # tokens per block
    fl_b = e_mean * x.shape[3] * n_blk[None, :, None]
    blk = _ratio(d2b, np.maximum(r2b, fl_b))
    pair = _ratio(d2b.sum(axis=1), np.maximum(r2b.sum(axis=1), e_mean * x.shape[3] * T))  # [B, H]
    whole = float(_ratio(np.array(d2b.sum()), np.array(r2b.sum())))
    ab = np.abs(diff)
    iw = np.unravel_index(int(np.argmax(ab)), ab.shape) if ab.size else (0, 0, 0, 0)
    ib = np.unravel_index(int(np.argmax(blk)), blk.shape) if blk.size else (0, 0, 0)
    ip = np.unravel_index(int(np.argmax(pair)), pair.shape) if pair.size else (0, 0)
    return {"whole": whole, "pair_max": float(pair.max()) if pair.size else 0.0, "pair_at": tuple(map(int, ip)),
            "block_max": float(blk.max()) if blk.size else 0.0,
            "block_at": (int(ib[0]), int(ib[1]) * block, int(ib[2])),
            "max_abs": float(ab.max()) if ab.size else 0.0, "max_abs_at": tuple(map(int, iw)),
            "blocks": int(blk.size)}


def state_report(x: np.ndarray, ref: np.ndarray) -> dict:
    """x, ref [B, H, dk, dv]: relative L2 over the whole tensor and per (b, h)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape and x.ndim == 4, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU state"
    diff = x - ref
    d2 = np.einsum("bhij,bhij->bh", diff, diff)
    r2 = np.einsum("bhij,bhij->bh", ref, ref)
    pair = _ratio(d2, r2)
    ip = np.unravel_index(int(np.argmax(pair)), pair.shape) if pair.size else (0, 0)
    ab = np.abs(diff)
    return {"whole": float(_ratio(np.array(d2.sum()), np.array(r2.sum()))),
            "pair_max": float(pair.max()) if pair.size else 0.0, "pair_at": tuple(map(int, ip)),
            "max_abs": float(ab.max()) if ab.size else 0.0}


# Sequences shorter than one 16-token tile are judged over the whole tensor only: the
# relative L2 of one token's outputs is that of a single dot product of rounded operands
# (beta (q . k) v), which has no relative bound at any resolution where q . k cancels.
MIN_UNIT_TOKENS = 16


def assert_tokens(label: str, x: np.ndarray, ref: np.ndarray, tol: float, block: int = BLOCK,
                  offset: tuple = (0, 0)) -> dict:
    """Relative L2 <= tol over the whole tensor and, for sequences of at least
    MIN_UNIT_TOKENS tokens, over every (b, h) sequence and every ``block``-token
    block of it.  ``offset`` = (b0, h0) of x within the full tensor, for the
    printed coordinates."""
    r = token_report(x, ref, block)
    b0, h0 = offset
    pb, ph = r["pair_at"]
    bb, bt, bh = r["block_at"]
    mb, mt, mh, mc = r["max_abs_at"]
    say(f"  {label}: rel-L2 whole {r['whole']:.3e}; worst (b,h) {r['pair_max']:.3e} at ({pb + b0},{ph + h0}); "
        f"worst of {r['blocks']} {block}-token blocks {r['block_max']:.3e} at (b={bb + b0}, t={bt}, h={bh + h0}); "
        f"max-abs {r['max_abs']:.3e} at (b={mb + b0}, t={mt}, h={mh + h0}, c={mc})")
    assert r["whole"] <= tol, f"{label}: whole-tensor rel-L2 {r['whole']:.3e} > {tol}"
    if x.shape[1] >= MIN_UNIT_TOKENS:
        assert r["pair_max"] <= tol, f"{label}: sequence rel-L2 {r['pair_max']:.3e} > {tol}"
        assert r["block_max"] <= tol, f"{label}: {block}-token block rel-L2 {r['block_max']:.3e} > {tol}"
    return r


def assert_states(label: str, x: np.ndarray, ref: np.ndarray, tol: float, offset: tuple = (0, 0)) -> dict:
    """Relative L2 <= tol for every (b, h) state."""
    r = state_report(x, ref)
    b0, h0 = offset
    pb, ph = r["pair_at"]
    say(f"  {label}: rel-L2 whole {r['whole']:.3e}; worst (b,h) {r['pair_max']:.3e} at ({pb + b0},{ph + h0}); "
        f"max-abs {r['max_abs']:.3e}")
    assert r["pair_max"] <= tol, f"{label}: state rel-L2 {r['pair_max']:.3e} > {tol}"
    return r


def f64_inputs(d: dict, dtype: str) -> dict:
    out = {k: ki.to_f64(d[k], dtype) for k in ("q", "k", "v", "z", "beta")}
    out["A"] = d["A"].astype(np.float64)
    out["S0"] = None if d.get("S0") is None else d["S0"].astype(np.float64)
    return out


def sub_inputs(d: dict, b0: int, b1: int, h0: int, h1: int) -> dict:
    """Storage arrays of batch entries [b0, b1) and heads [h0, h1) of a prefill workload."""
    sub = {k: np.ascontiguousarray(d[k][b0:b1, :, h0:h1]) for k in ("q", "k", "v", "z", "beta")}
    sub["A"] = np.ascontiguousarray(d["A"][h0:h1])
    sub["S0"] = None if d.get("S0") is None else np.ascontiguousarray(d["S0"][b0:b1, h0:h1])
    return sub


def dev_inputs(d: dict, dtype: str) -> dict:
    out = {k: dev(d[k], dtype) for k in ("q", "k", "v", "z", "beta")}
    out["A"] = dev(d["A"], "f32")
    out["S0"] = dev(d["S0"], "f32") if d.get("S0") is not None else None
    return out
