"""Python binding of libkda.so -- the MI355X (gfx950) Kimi Delta Attention
forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/kda.h).  PyTorch supplies device memory and
the current stream.  There is no CPU fallback: the functions raise when the
library is not built or when a tensor is not on a GPU.

Entry points (same names as the C ABI):
  gate(z, A, g_min, chunk)                        -> G           (kda_gate)
  chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk) -> bytes     (kda_chunk_fwd_workspace_bytes)
  chunk_fwd(q, k, v, beta, G, chunk, ...)         -> (o, S_out)  (kda_chunk_fwd)
  chunk_fwd_z(q, k, v, beta, z, A, g_min, chunk)  -> (o, S_out)  (kda_chunk_fwd_z)
  decode_step(q, k, v, z, beta, A, S, g_min)      -> o           (kda_decode_step; S updated in place)
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

__all__ = ["gate", "chunk_fwd", "chunk_fwd_z", "chunk_fwd_workspace_bytes", "decode_step", "chunk_uses_mfma", "lib",
           "KDAError", "LIB_PATH", "G_MIN"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
G_MIN = -5.0
KDA_F32, KDA_BF16 = 0, 1

_lib = None


class KDAError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libkda.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KDAError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.kda_status_string.argtypes = [I]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_version.argtypes = []
    L.kda_version.restype = I
    L.kda_chunk_uses_mfma.argtypes = [I, I, I, I]
    L.kda_chunk_uses_mfma.restype = I
    L.kda_gate.argtypes = [P, I, P, F, I, I, I, I, I, P, P]
    L.kda_gate.restype = I
    Z = ctypes.c_size_t
    L.kda_chunk_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.kda_chunk_fwd_workspace_bytes.restype = Z
    L.kda_chunk_fwd.argtypes = [P, P, P, P, I, P, P, P, I, P, I, I, I, I, I, I, F, P, Z, P]
    L.kda_chunk_fwd.restype = I
    L.kda_chunk_fwd_z.argtypes = [P, P, P, P, P, I, P, F, P, P, I, P, I, I, I, I, I, I, F, P, Z, P]
    L.kda_chunk_fwd_z.restype = I
    L.kda_decode_step.argtypes = [P, P, P, P, P, I, P, F, P, P, I, I, I, I, I, F, P]
    L.kda_decode_step.restype = I
    L.kda_decode_replay.argtypes = [P, P, P, P, P, I, P, F, P, P, P, I, P, I, I, I, I, I, F, P]
    L.kda_decode_replay.restype = I
    L.kda_chunk_fwd_z_noalloc.argtypes = [P, P, P, P, P, I, P, F, P, P, I, P, I, I, I, I, I, I, F, P]
    L.kda_chunk_fwd_z_noalloc.restype = I
    L.kda_chunk_fwd_z_prologue.argtypes = L.kda_chunk_fwd_z.argtypes
    L.kda_chunk_fwd_z_prologue.restype = I
    L.kda_decode_step_prologue.argtypes = L.kda_decode_step.argtypes
    L.kda_decode_step_prologue.restype = I
    L.kda_chunk_bwd_z_workspace_bytes.argtypes = [I, I, I, I, I]
    L.kda_chunk_bwd_z_workspace_bytes.restype = ctypes.c_size_t
    L.kda_chunk_bwd_z.argtypes = [P, P, P, P, P, I, P, F, P, P, I, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P,
                                  ctypes.c_size_t, P]
    L.kda_chunk_bwd_z.restype = I
    L.kda_chunk_fwd_z_segmented_workspace_bytes.argtypes = [I, I, I, I, I]
    L.kda_chunk_fwd_z_segmented_workspace_bytes.restype = ctypes.c_size_t
    L.kda_chunk_fwd_z_segmented.argtypes = [P, P, P, P, P, I, P, F, P, P, I, P, I, I, I, I, I, I, F, I, P,
                                            ctypes.c_size_t, P]
    L.kda_chunk_fwd_z_segmented.restype = I
    _lib = L
    return L


def chunk_uses_mfma(dtype: torch.dtype, dk: int, dv: int, chunk: int) -> bool:
    """True when the chunked prefill runs the MFMA kernel for these arguments."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return bool(lib().kda_chunk_uses_mfma(code, dk, dv, chunk))


def _check(status: int, what: str):
    if status != 0:
        msg = lib().kda_status_string(status).decode()
        raise KDAError(f"{what}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise KDAError("libkda runs on the GPU only: tensor is on the CPU")
        if not t.is_contiguous():
            raise KDAError("tensors must be contiguous")


_F32 = (torch.float32,)
_IO = (torch.float32, torch.bfloat16)


def _shapes(what: str, *specs):
    """The C ABI takes raw pointers and trusts the sizes it is given, so every
    tensor's shape and dtype are checked here, before any pointer is passed:
    specs are (name, tensor or None, expected shape, allowed dtypes)."""
    dev = None
    for name, t, shape, dtypes in specs:
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise KDAError(f"{what}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype not in dtypes:
            raise KDAError(f"{what}: {name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise KDAError(f"{what}: {name} is on {t.device}, the other tensors on {dev}")


def _on_tensor_device(fn):
    """Run a call with the device of its first tensor argument current: the library
    launches on the current device, on that device's current stream."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        t = next((a for a in args if isinstance(a, torch.Tensor)), None)
        if t is None or not t.is_cuda:
            return fn(*args, **kwargs)
        with torch.cuda.device(t.device):
            return fn(*args, **kwargs)
    return wrapper


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@_on_tensor_device
def gate(z: torch.Tensor, A: torch.Tensor, g_min: float = G_MIN, chunk: int = 1,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """G [B,T,H,dk] fp32: chunk-local sums of g = g_min*sigmoid(exp(A) z)."""
    B, T, H, dk = z.shape
    if out is None:
        out = torch.empty((B, T, H, dk), dtype=torch.float32, device=z.device)
    _shapes("kda_gate", ("z", z, (B, T, H, dk), _IO), ("A", A, (H, dk), _F32), ("out", out, (B, T, H, dk), _F32))
    _dev(z, A, out)
    _check(lib().kda_gate(_p(z), _dtype_code(z), _p(A), float(g_min), B, T, H, dk, int(chunk), _p(out),
                          _stream(stream)), "kda_gate")
    return out


def _chunk_shapes(what, q, k, v, beta, z=None, A=None, G=None, S_in=None, o=None, S_out=None):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = (q.dtype,) if q.dtype in _IO else _IO
    _shapes(what, ("q", q, (B, T, H, dk), _IO), ("k", k, (B, T, H, dk), io), ("v", v, (B, T, H, dv), io),
            ("beta", beta, (B, T, H), io), ("z", z, (B, T, H, dk), io), ("A", A, (H, dk), _F32),
            ("G", G, (B, T, H, dk), _F32), ("S_in", S_in, (B, H, dk, dv), _F32), ("o", o, (B, T, H, dv), _IO),
            ("S_out", S_out, (B, H, dk, dv), _F32))


def chunk_fwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, chunk: int) -> int:
    """Device bytes kda_chunk_fwd / kda_chunk_fwd_z / kda_chunk_fwd_z_prologue need
    as workspace for these sizes (0: none)."""
    return int(lib().kda_chunk_fwd_workspace_bytes(int(B), int(T), int(H), int(dk), int(dv), int(chunk)))


def _workspace(workspace, q, v, chunk):
    """(pointer, bytes) of the caller's workspace, or of a new one of the queried
    size (None, 0 when the call needs none)."""
    B, T, H, dk = q.shape
    if workspace is None:
        need = chunk_fwd_workspace_bytes(B, T, H, dk, v.shape[-1], chunk)
        if need == 0:
            return None, 0, None
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(workspace)
    return _p(workspace), workspace.numel() * workspace.element_size(), workspace


def _outs(q, v, o, S_out, o_dtype, want_state):
    B, T, H, _ = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or torch.float32, device=q.device)
    if S_out is None and want_state:
        S_out = torch.empty((B, H, q.shape[-1], dv), dtype=torch.float32, device=q.device)
    return o, S_out


@_on_tensor_device
def chunk_fwd(q, k, v, beta, G, chunk: int = 64, S_in=None, o=None, S_out=None, o_dtype=None,
              scale: float = 1.0, want_state: bool = True, workspace=None,
              stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill from the chunk-local sums G of kda_gate (same chunk).
    ``workspace``: a device tensor of at least ``chunk_fwd_workspace_bytes``
    bytes, or None (one is allocated when the call needs it).
    Returns (o [B,T,H,dv], S_out [B,H,dk,dv] or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o, S_out = _outs(q, v, o, S_out, o_dtype, want_state)
    _chunk_shapes("kda_chunk_fwd", q, k, v, beta, G=G, S_in=S_in, o=o, S_out=S_out)
    _dev(q, k, v, beta, G, S_in, o, S_out)
    wp, wb, _keep = _workspace(workspace, q, v, chunk)
    _check(lib().kda_chunk_fwd(_p(q), _p(k), _p(v), _p(beta), _dtype_code(q), _p(G), _p(S_in), _p(o),
                               _dtype_code(o), _p(S_out), B, T, H, dk, dv, int(chunk), float(scale), wp, wb,
                               _stream(stream)), "kda_chunk_fwd")
    return o, S_out


@_on_tensor_device
def chunk_fwd_z(q, k, v, beta, z, A, g_min: float = G_MIN, chunk: int = 64, S_in=None, o=None, S_out=None,
                o_dtype=None, scale: float = 1.0, want_state: bool = True, workspace=None,
                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill with the gate fused (decay logits z, A, g_min).
    ``workspace``: as ``chunk_fwd``.
    Returns (o [B,T,H,dv], S_out [B,H,dk,dv] or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o, S_out = _outs(q, v, o, S_out, o_dtype, want_state)
    _chunk_shapes("kda_chunk_fwd_z", q, k, v, beta, z=z, A=A, S_in=S_in, o=o, S_out=S_out)
    _dev(q, k, v, beta, z, A, S_in, o, S_out)
    wp, wb, _keep = _workspace(workspace, q, v, chunk)
    _check(lib().kda_chunk_fwd_z(_p(q), _p(k), _p(v), _p(beta), _p(z), _dtype_code(q), _p(A), float(g_min),
                                 _p(S_in), _p(o), _dtype_code(o), _p(S_out), B, T, H, dk, dv, int(chunk),
                                 float(scale), wp, wb, _stream(stream)), "kda_chunk_fwd_z")
    return o, S_out


@_on_tensor_device
def chunk_fwd_z_noalloc(q, k, v, beta, z, A, g_min: float = G_MIN, chunk: int = 64, S_in=None, o=None, S_out=None,
                        o_dtype=None, scale: float = 1.0, want_state: bool = True,
                        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd_z`` whose scratch memory is the library's static device array
    (kda_chunk_fwd_z_noalloc): no workspace is allocated for the call.  Calls that
    overlap in time on one device share that array and must not be issued."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o, S_out = _outs(q, v, o, S_out, o_dtype, want_state)
    _chunk_shapes("kda_chunk_fwd_z_noalloc", q, k, v, beta, z=z, A=A, S_in=S_in, o=o, S_out=S_out)
    _dev(q, k, v, beta, z, A, S_in, o, S_out)
    _check(lib().kda_chunk_fwd_z_noalloc(_p(q), _p(k), _p(v), _p(beta), _p(z), _dtype_code(q), _p(A), float(g_min),
                                         _p(S_in), _p(o), _dtype_code(o), _p(S_out), B, T, H, dk, dv, int(chunk),
                                         float(scale), _stream(stream)), "kda_chunk_fwd_z_noalloc")
    return o, S_out


@_on_tensor_device
def chunk_fwd_z_prologue(q_raw, k_raw, v, beta_logit, z, A, g_min: float = G_MIN, chunk: int = 64, S_in=None,
                         o=None, S_out=None, o_dtype=None, scale: float = 1.0, want_state: bool = True,
                         workspace=None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd_z`` with the prologue fused: q, k un-normalised, beta as a logit."""
    B, T, H, dk = q_raw.shape
    dv = v.shape[-1]
    o, S_out = _outs(q_raw, v, o, S_out, o_dtype, want_state)
    _chunk_shapes("kda_chunk_fwd_z_prologue", q_raw, k_raw, v, beta_logit, z=z, A=A, S_in=S_in, o=o, S_out=S_out)
    _dev(q_raw, k_raw, v, beta_logit, z, A, S_in, o, S_out)
    wp, wb, _keep = _workspace(workspace, q_raw, v, chunk)
    _check(lib().kda_chunk_fwd_z_prologue(_p(q_raw), _p(k_raw), _p(v), _p(beta_logit), _p(z), _dtype_code(q_raw),
                                          _p(A), float(g_min), _p(S_in), _p(o), _dtype_code(o), _p(S_out), B, T, H,
                                          dk, dv, int(chunk), float(scale), wp, wb, _stream(stream)),
           "kda_chunk_fwd_z_prologue")
    return o, S_out


@_on_tensor_device
def decode_step_prologue(q_raw, k_raw, v, z, beta_logit, A, S, g_min: float = G_MIN, o=None, o_dtype=None,
                         scale: float = 1.0, stream=None) -> torch.Tensor:
    """``decode_step`` with the prologue fused: q, k un-normalised, beta as a logit."""
    N, H, dk = q_raw.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype or torch.float32, device=q_raw.device)
    _decode_shapes("kda_decode_step_prologue", q_raw, k_raw, v, z, beta_logit, A, S, o)
    _dev(q_raw, k_raw, v, z, beta_logit, A, S, o)
    _check(lib().kda_decode_step_prologue(_p(q_raw), _p(k_raw), _p(v), _p(z), _p(beta_logit), _dtype_code(q_raw),
                                          _p(A), float(g_min), _p(S), _p(o), _dtype_code(o), N, H, dk, dv,
                                          float(scale), _stream(stream)), "kda_decode_step_prologue")
    return o


@_on_tensor_device
def chunk_bwd_z(q, k, v, beta, z, A, d_o, dS_out=None, g_min: float = G_MIN, S_in=None, scale: float = 1.0,
                want_dS_in: bool = True, workspace=None, stream=None) -> dict:
    """Backward of ``chunk_fwd_z``: gradients (fp32) of a loss given dL/do (``d_o``)
    and optionally dL/dS_out.  Returns a dict with dq, dk, dv, dbeta, dz, dA and
    dS_in (None unless ``want_dS_in``)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    f32 = torch.float32
    out = {"dq": torch.empty((B, T, H, dk), dtype=f32, device=dev),
           "dk": torch.empty((B, T, H, dk), dtype=f32, device=dev),
           "dv": torch.empty((B, T, H, dv), dtype=f32, device=dev),
           "dbeta": torch.empty((B, T, H), dtype=f32, device=dev),
           "dz": torch.empty((B, T, H, dk), dtype=f32, device=dev),
           "dA": torch.empty((H, dk), dtype=f32, device=dev),
           "dS_in": torch.empty((B, H, dk, dv), dtype=f32, device=dev) if want_dS_in else None}
    need = int(lib().kda_chunk_bwd_z_workspace_bytes(B, T, H, dk, dv))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _chunk_shapes("kda_chunk_bwd_z", q, k, v, beta, z=z, A=A, S_in=S_in)
    _shapes("kda_chunk_bwd_z", ("q", q, q.shape, _IO), ("d_o", d_o, (B, T, H, dv), _IO),
            ("dS_out", dS_out, (B, H, dk, dv), _F32))
    _dev(q, k, v, beta, z, A, d_o, dS_out, S_in, workspace, *[t for t in out.values() if t is not None])
    _check(lib().kda_chunk_bwd_z(_p(q), _p(k), _p(v), _p(beta), _p(z), _dtype_code(q), _p(A), float(g_min), _p(S_in),
                                 _p(d_o), _dtype_code(d_o), _p(dS_out), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]),
                                 _p(out["dbeta"]), _p(out["dz"]), _p(out["dA"]), _p(out["dS_in"]), B, T, H, dk, dv,
                                 float(scale), _p(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "kda_chunk_bwd_z")
    return out


def chunk_fwd_z_segmented_workspace_bytes(B: int, H: int, dk: int, dv: int, segments: int) -> int:
    """Device bytes the segment-parallel prefill needs for ``segments`` segments."""
    return int(lib().kda_chunk_fwd_z_segmented_workspace_bytes(B, H, dk, dv, int(segments)))


@_on_tensor_device
def chunk_fwd_z_segmented(q, k, v, beta, z, A, segments: int, g_min: float = G_MIN, chunk: int = 64, S_in=None,
                          o=None, S_out=None, o_dtype=None, scale: float = 1.0, want_state: bool = True,
                          workspace=None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd_z`` with the sequence cut into ``segments`` chunk-aligned
    segments run in parallel (for small B*H and long T).  ``workspace`` is a
    device tensor of at least ``chunk_fwd_z_segmented_workspace_bytes`` bytes;
    one is allocated when it is None.  Returns (o, S_out or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o, S_out = _outs(q, v, o, S_out, o_dtype, want_state)
    need = chunk_fwd_z_segmented_workspace_bytes(B, H, dk, dv, segments)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _chunk_shapes("kda_chunk_fwd_z_segmented", q, k, v, beta, z=z, A=A, S_in=S_in, o=o, S_out=S_out)
    _dev(q, k, v, beta, z, A, S_in, o, S_out, workspace)
    _check(lib().kda_chunk_fwd_z_segmented(_p(q), _p(k), _p(v), _p(beta), _p(z), _dtype_code(q), _p(A),
                                           float(g_min), _p(S_in), _p(o), _dtype_code(o), _p(S_out), B, T, H, dk,
                                           dv, int(chunk), float(scale), int(segments), _p(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)),
           "kda_chunk_fwd_z_segmented")
    return o, S_out


def _decode_shapes(what, q, k, v, z, beta, A, S, o):
    N, H, dk = q.shape
    dv = v.shape[-1]
    io = (q.dtype,) if q.dtype in _IO else _IO
    _shapes(what, ("q", q, (N, H, dk), _IO), ("k", k, (N, H, dk), io), ("v", v, (N, H, dv), io),
            ("z", z, (N, H, dk), io), ("beta", beta, (N, H), io), ("A", A, (H, dk), _F32),
            ("S", S, (N, H, dk, dv), _F32), ("o", o, (N, H, dv), _IO))


@_on_tensor_device
def decode_step(q, k, v, z, beta, A, S, g_min: float = G_MIN, o=None, o_dtype=None, scale: float = 1.0,
                stream=None) -> torch.Tensor:
    """One token per sequence; S [N,H,dk,dv] fp32 is updated in place.
    Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype or torch.float32, device=q.device)
    _decode_shapes("kda_decode_step", q, k, v, z, beta, A, S, o)
    _dev(q, k, v, z, beta, A, S, o)
    _check(lib().kda_decode_step(_p(q), _p(k), _p(v), _p(z), _p(beta), _dtype_code(q), _p(A), float(g_min),
                                 _p(S), _p(o), _dtype_code(o), N, H, dk, dv, float(scale), _stream(stream)),
           "kda_decode_step")
    return o


@_on_tensor_device
def decode_replay(q, k, v, z, beta, A, S_snapshot, accepted, g_min: float = G_MIN, o=None, o_dtype=None,
                  S_commit=None, scale: float = 1.0, stream=None):
    """Speculative-decoding replay: the drafted tokens q, k, z [n_draft,N,H,dk],
    v [n_draft,N,H,dv], beta [n_draft,N,H] run from S_snapshot [N,H,dk,dv] fp32
    (left unchanged); accepted [N] int32 holds each sequence's accepted prefix
    length.  Returns (o [n_draft,N,H,dv] for every drafted token, S_commit
    [N,H,dk,dv], the state after the accepted prefix)."""
    n_draft, N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((n_draft, N, H, dv), dtype=o_dtype or torch.float32, device=q.device)
    if S_commit is None:
        S_commit = torch.empty_like(S_snapshot)
    io = (q.dtype,) if q.dtype in _IO else _IO
    _shapes("kda_decode_replay", ("q", q, (n_draft, N, H, dk), _IO), ("k", k, (n_draft, N, H, dk), io),
            ("v", v, (n_draft, N, H, dv), io), ("z", z, (n_draft, N, H, dk), io), ("beta", beta, (n_draft, N, H), io),
            ("A", A, (H, dk), _F32), ("S_snapshot", S_snapshot, (N, H, dk, dv), _F32),
            ("accepted", accepted, (N,), (torch.int32,)), ("o", o, (n_draft, N, H, dv), _IO),
            ("S_commit", S_commit, (N, H, dk, dv), _F32))
    _dev(q, k, v, z, beta, A, S_snapshot, accepted, o, S_commit)
    _check(lib().kda_decode_replay(_p(q), _p(k), _p(v), _p(z), _p(beta), _dtype_code(q), _p(A), float(g_min),
                                   _p(S_snapshot), _p(accepted), _p(o), _dtype_code(o), _p(S_commit), n_draft, N,
                                   H, dk, dv, float(scale), _stream(stream)),
           "kda_decode_replay")
    return o, S_commit
