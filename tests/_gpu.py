"""Helpers for the GPU parity tests: storage arrays -> device tensors, the
relative-L2 metric, and oracle runs on the same rounded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import kda_inputs as ki

DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 1e-2}


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


def f64_inputs(d: dict, dtype: str) -> dict:
    out = {k: ki.to_f64(d[k], dtype) for k in ("q", "k", "v", "z", "beta")}
    out["A"] = d["A"].astype(np.float64)
    out["S0"] = None if d.get("S0") is None else d["S0"].astype(np.float64)
    return out


def dev_inputs(d: dict, dtype: str) -> dict:
    out = {k: dev(d[k], dtype) for k in ("q", "k", "v", "z", "beta")}
    out["A"] = dev(d["A"], "f32")
    out["S0"] = dev(d["S0"], "f32") if d.get("S0") is not None else None
    return out
