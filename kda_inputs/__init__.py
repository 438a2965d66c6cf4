"""Seeded synthetic inputs for the KDA forward pass.

This module is shared by the fp64 oracle side and the GPU side: it only draws
random numbers, shapes them like the workloads described on the pages, and
rounds them to the storage dtype.  It holds none of the method's arithmetic
(no gate, no decay, no recurrence).

Distributions (Kimi K3 pages: "Kimi K3: the paper and proofs side by side",
section 2.1.1 Equations 2-6, for the regularised L2 normalisation of q and k;
the workloads themselves are synthetic):

* q, k ~ N(0, 1) per channel, then L2-normalised per (b, t, h) in fp64 as
  x / sqrt(|x|^2 + 1e-6) (the divisor is stripped from the page; this is the
  reading taken), then rounded to the storage dtype.
* v ~ N(0, 1), z ~ N(0, 1) * z_scale + z_mean, beta = sigmoid(N(0, 1)).
  z_mean = 0 (the workloads) puts the gate logit near 0, so most key
  channels lose about half their remaining log-range per token and the state
  forgets within one chunk; a negative z_mean (long-memory test cases) makes
  the decay slow, so the state carried across chunks and segments matters.
* raw = True (inputs of the fused-prologue entry points): q and k are NOT
  normalised: each token row is N(0, 1) times a magnitude 10^U(-3.5, 0.5)
  drawn per row (norms from about 4e-3 to 36, so the 1e-6 regulariser
  matters at the small end), and beta is a logit, N(0, 2^2), with no sigmoid.
* A ~ N(0, 0.5^2) per (head, key channel), stored fp32.
* S0 ~ N(0, s0_std^2) per (b, h) state, stored fp32 (absent when s0_std == 0).

Rounding: fp64 -> fp32 round-to-nearest-even, then (for bf16 storage)
fp32 -> bf16 round-to-nearest-even.  bf16 values are held in numpy as uint16
bit patterns.  Both sides consume exactly these rounded values.

Generation is blocked: each (tensor, b, h, block of TBLK tokens) draws from its
own ``numpy.random.Generator`` seeded with ``[seed, tag, b, h, block]``, so any
(b, h) sub-sequence can be regenerated alone and blocks can be drawn in
parallel threads with identical results.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence

import numpy as np

TBLK = 4096          # tokens per generation block
L2_EPS = 1e-6        # regulariser of the q/k L2 normalisation

_TAG = {"q": 11, "k": 12, "v": 13, "z": 14, "beta": 15, "A": 16, "S0": 17}


# ----------------------------------------------------------------------------
# dtype helpers
# ----------------------------------------------------------------------------
def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = round_to_f32(x64)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def storage_np_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2norm_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def _raw_rows(rng, x: np.ndarray) -> np.ndarray:
    """Un-normalised rows: x times a per-row magnitude 10^U(-3.5, 0.5)."""
    mag = 10.0 ** rng.uniform(-3.5, 0.5, x.shape[:-1] + (1,))
    return x * mag


def _beta_draw(rng, shape, raw: bool) -> np.ndarray:
    x = rng.standard_normal(shape)
    return 2.0 * x if raw else _sigmoid(x)


# ----------------------------------------------------------------------------
# workload specs
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str            # storage dtype of q, k, v, z, beta: "f32" | "bf16"
    z_scale: float = 1.0
    s0_std: float = 0.0   # 0 -> no incoming state (zeros)
    z_mean: float = 0.0   # offset of the decay logits z (negative: slow decay, long memory)
    raw: bool = False     # q, k un-normalised and beta a logit (fused-prologue inputs)
    seed: int = 1000


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: str
    s_std: float = 0.1
    seed: int = 1004
    raw: bool = False     # q, k un-normalised and beta a logit (fused-prologue inputs)


# The five workloads: a tiny fp32 case, a 4K-token prefill, the 32K-token
# throughput prefill, a 1M-token single-sequence prefill with z scaled by 3,
# and 64 decode steps over 256 sequences.
TINY_F32 = PrefillSpec("tiny_f32_T64_d16", B=1, H=2, T=64, dk=16, dv=16, chunk=16, dtype="f32", seed=1000)
PREFILL_4K = PrefillSpec("prefill_bf16_B1_H8_T4096", B=1, H=8, T=4096, dk=128, dv=128, chunk=64, dtype="bf16", seed=1001)
PREFILL_32K = PrefillSpec("prefill_bf16_B4_H32_T32768", B=4, H=32, T=32768, dk=128, dv=128, chunk=64, dtype="bf16",
                          s0_std=0.01, seed=1002)
PREFILL_1M = PrefillSpec("prefill_bf16_B1_H8_T1048576_z3", B=1, H=8, T=1 << 20, dk=128, dv=128, chunk=64, dtype="bf16",
                         z_scale=3.0, seed=1003)
DECODE_256 = DecodeSpec("decode_bf16_N256_H32_64steps", N=256, H=32, dk=128, dv=128, steps=64, dtype="bf16",
                        s_std=0.1, seed=1004)

WORKLOADS = {s.name: s for s in (TINY_F32, PREFILL_4K, PREFILL_32K, PREFILL_1M, DECODE_256)}


def _threads() -> int:
    n = os.cpu_count() or 4
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# prefill inputs
# ----------------------------------------------------------------------------
def _draw_block(spec: PrefillSpec, b: int, h: int, blk: int, t0: int, t1: int) -> Dict[str, np.ndarray]:
    n = t1 - t0
    out = {}
    for name, width in (("q", spec.dk), ("k", spec.dk), ("v", spec.dv), ("z", spec.dk)):
        rng = np.random.default_rng([spec.seed, _TAG[name], b, h, blk])
        x = rng.standard_normal((n, width))
        if name in ("q", "k"):
            x = _raw_rows(rng, x) if spec.raw else _l2norm_rows(x)
        elif name == "z":
            x = x * spec.z_scale
            if spec.z_mean:
                x = x + spec.z_mean
        out[name] = round_storage(x, spec.dtype)
    rng = np.random.default_rng([spec.seed, _TAG["beta"], b, h, blk])
    out["beta"] = round_storage(_beta_draw(rng, n, spec.raw), spec.dtype)
    return out


def gen_A(spec) -> np.ndarray:
    rng = np.random.default_rng([spec.seed, _TAG["A"]])
    return round_to_f32(0.5 * rng.standard_normal((spec.H, spec.dk)))


def gen_S0(spec: PrefillSpec, b_sel: Sequence[int], h_sel: Sequence[int]) -> Optional[np.ndarray]:
    if spec.s0_std == 0.0:
        return None
    S0 = np.empty((len(b_sel), len(h_sel), spec.dk, spec.dv), dtype=np.float32)
    for bi, b in enumerate(b_sel):
        for hi, h in enumerate(h_sel):
            rng = np.random.default_rng([spec.seed, _TAG["S0"], b, h])
            S0[bi, hi] = round_to_f32(spec.s0_std * rng.standard_normal((spec.dk, spec.dv)))
    return S0


def prefill_inputs(spec: PrefillSpec, b_sel: Optional[Sequence[int]] = None,
                   h_sel: Optional[Sequence[int]] = None, T: Optional[int] = None,
                   threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Storage arrays for the (b, h) selection of a prefill workload.

    Returns q, k, z [B', T, H', dk]; v [B', T, H', dv]; beta [B', T, H'] in the
    storage dtype (uint16 bf16 bits or float32); A [H', dk] float32; S0
    [B', H', dk, dv] float32 or None.  ``T`` truncates the sequence (a prefix
    of the full workload's tokens: blocks are drawn identically).
    """
    b_sel = list(range(spec.B)) if b_sel is None else list(b_sel)
    h_sel = list(range(spec.H)) if h_sel is None else list(h_sel)
    T = spec.T if T is None else int(T)
    Bp, Hp = len(b_sel), len(h_sel)
    sdt = storage_np_dtype(spec.dtype)
    out = {
        "q": np.empty((Bp, T, Hp, spec.dk), sdt),
        "k": np.empty((Bp, T, Hp, spec.dk), sdt),
        "v": np.empty((Bp, T, Hp, spec.dv), sdt),
        "z": np.empty((Bp, T, Hp, spec.dk), sdt),
        "beta": np.empty((Bp, T, Hp), sdt),
    }
    jobs = []
    for bi, b in enumerate(b_sel):
        for hi, h in enumerate(h_sel):
            for blk in range((T + TBLK - 1) // TBLK):
                jobs.append((bi, b, hi, h, blk))

    def run(job):
        bi, b, hi, h, blk = job
        t0 = blk * TBLK
        t1 = min(T, t0 + TBLK)
        d = _draw_block(spec, b, h, blk, t0, t0 + TBLK)
        for name in ("q", "k", "v", "z"):
            out[name][bi, t0:t1, hi, :] = d[name][: t1 - t0]
        out["beta"][bi, t0:t1, hi] = d["beta"][: t1 - t0]

    nthr = threads or _threads()
    if nthr > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    A = gen_A(spec)
    out["A"] = np.ascontiguousarray(A[h_sel])
    out["S0"] = gen_S0(spec, b_sel, h_sel)
    return out


def small_spec(B, H, T, dk, dv, chunk, dtype, seed, z_scale=1.0, s0_std=0.0, name="custom",
               z_mean=0.0, raw=False) -> PrefillSpec:
    return PrefillSpec(name, B=B, H=H, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype, z_scale=z_scale,
                       s0_std=s0_std, seed=seed, z_mean=z_mean, raw=raw)


# ----------------------------------------------------------------------------
# decode inputs
# ----------------------------------------------------------------------------
def decode_step_inputs(spec: DecodeSpec, step: int, n_sel: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Per-step tokens: q, k, v, z [N', H, d], beta [N', H] in the storage dtype."""
    out = {}
    for name, width in (("q", spec.dk), ("k", spec.dk), ("v", spec.dv), ("z", spec.dk)):
        rng = np.random.default_rng([spec.seed, _TAG[name], step])
        x = rng.standard_normal((spec.N, spec.H, width))
        if name in ("q", "k"):
            x = _raw_rows(rng, x) if spec.raw else _l2norm_rows(x)
        out[name] = round_storage(x, spec.dtype)
    rng = np.random.default_rng([spec.seed, _TAG["beta"], step])
    out["beta"] = round_storage(_beta_draw(rng, (spec.N, spec.H), spec.raw), spec.dtype)
    if n_sel is not None:
        n_sel = list(n_sel)
        out = {k: np.ascontiguousarray(v[n_sel]) for k, v in out.items()}
    return out


def decode_inputs(spec: DecodeSpec, n_sel: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All steps stacked: q, k, v, z [steps, N', H, d]; beta [steps, N', H];
    A [H, dk]; S0 [N', H, dk, dv] float32."""
    nthr = threads or _threads()
    with ThreadPoolExecutor(nthr) as ex:
        per = list(ex.map(lambda s: decode_step_inputs(spec, s, n_sel), range(spec.steps)))
    out = {k: np.stack([p[k] for p in per]) for k in per[0]}
    out["A"] = gen_A(spec)
    n_list = list(range(spec.N)) if n_sel is None else list(n_sel)
    S0 = np.empty((len(n_list), spec.H, spec.dk, spec.dv), dtype=np.float32)

    def fill(i_n):
        i, n = i_n
        rng = np.random.default_rng([spec.seed, _TAG["S0"], n])
        S0[i] = round_to_f32(spec.s_std * rng.standard_normal((spec.H, spec.dk, spec.dv)))

    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill, list(enumerate(n_list))))
    out["S0"] = S0
    return out
