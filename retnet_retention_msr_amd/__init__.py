"""Multi-Scale Retention on MI355X: a thin torch binding of libretention.so.

The functions here only marshal arguments: they check tensors, allocate
outputs and workspace with torch, and call the C ABI (include/retention.h) on
the current HIP stream. Every step of the computation runs in the library's
HIP kernels; there is no other code path. The operator follows "RetNet -
Retentive Network - A Successor to Transformer for LLMs" (Key Equations:
parallel, recurrent and chunkwise recurrent forms; Key components, 2.
Multi-Scale Retention) and the jisaku.com RetNet glossary entry.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence, Union

import torch

from . import _lib

__all__ = [
    "GroupNorm",
    "parallel",
    "chunkwise",
    "chunk_states",
    "chunk_output",
    "recurrent_step",
    "chunkwise_workspace_bytes",
    "chunkwise_backward",
    "chunkwise_backward_workspace_bytes",
    "RetentionError",
]


class RetentionError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {_lib.status_string(code)} ({code})")
        self.code = code


@dataclass
class GroupNorm:
    """Per-head GroupNorm epilogue: eps and optional fp32 [H*dv] weight/bias on the device."""

    eps: float = 1e-5
    weight: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None


GammaLike = Union[torch.Tensor, Sequence[float]]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.RET_F32
    if t.dtype == torch.bfloat16:
        return _lib.RET_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _gamma_array(gamma: GammaLike, H: int):
    g = torch.as_tensor(gamma, dtype=torch.float32).detach().to("cpu").contiguous()
    if g.numel() != H:
        raise ValueError(f"gamma has {g.numel()} entries, expected H={H}")
    arr = (ctypes.c_float * H)(*g.tolist())
    return arr


def _gn_struct(gn: Optional[GroupNorm], H: int, dv: int, device, gate=None, like=None):
    """The retention_gn_t for ``gn``; ``gate`` (optional) must match ``like`` (the output)."""
    if gn is None:
        if gate is not None:
            raise ValueError("a gate needs the GroupNorm epilogue (gn)")
        return None, ()
    keep = []
    ptrs = []
    for t in (gn.weight, gn.bias):
        if t is None:
            ptrs.append(None)
            continue
        if t.device != device or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != H * dv:
            raise ValueError("GroupNorm weight/bias must be contiguous float32 [H*dv] on the input's device")
        keep.append(t)
        ptrs.append(t.data_ptr())
    gate_ptr = None
    if gate is not None:
        if (not gate.is_cuda or gate.device != like.device or gate.dtype != like.dtype or not gate.is_contiguous()
                or gate.numel() != like.numel()):
            raise ValueError("gate must be a contiguous device tensor with the output's dtype and shape")
        if gate.data_ptr() == like.data_ptr():
            raise ValueError("gate must not alias the output")
        keep.append(gate)
        gate_ptr = gate.data_ptr()
    s = _lib.GnStruct(float(gn.eps), ptrs[0], ptrs[1], gate_ptr)
    return ctypes.byref(s), (s, keep)


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B,H,N,dk] and v [B,H,N,dv]")
    B, H, N, dk = q.shape
    return B, H, N, dk, v.shape[3], _dtype_code(q)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def parallel(q, k, v, gamma: GammaLike, gn: Optional[GroupNorm] = None, out=None, gate=None):
    """Parallel form O = (Q K^T * D) V per head (optionally GroupNorm-ed).

    ``gate`` (optional, needs ``gn``): a tensor like the output; the result
    becomes GroupNorm(O) * swish(gate).
    """
    lib = _lib.load()
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    rc = lib.retention_parallel(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, out.data_ptr(), B, H, N, dk, dv, dt,
                                gn_p, _stream(q))
    if rc != 0:
        raise RetentionError("retention_parallel", rc)
    return out


def chunkwise_workspace_bytes(B, H, N, dk, dv, chunk, dtype=torch.bfloat16) -> int:
    code = _lib.RET_BF16 if dtype == torch.bfloat16 else _lib.RET_F32
    return int(_lib.load().retention_chunkwise_workspace_bytes(B, H, N, dk, dv, int(chunk), code))


def chunkwise(q, k, v, gamma: GammaLike, chunk: int, state_in=None, state_out: Union[bool, torch.Tensor] = False,
              gn: Optional[GroupNorm] = None, out=None, workspace=None, gate=None):
    """Chunkwise recurrent form. Returns (o, state_out or None).

    ``state_out``: False (not produced), True (allocate), or an fp32
    [B,H,dk,dv] tensor to fill (it may be ``state_in`` itself). ``gate``
    (optional, needs ``gn``): a tensor like the output; the result becomes
    GroupNorm(O) * swish(gate).
    """
    lib = _lib.load()
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        if isinstance(s, torch.Tensor):
            if s.dtype != torch.float32 or not s.is_contiguous() or tuple(s.shape) != (B, H, dk, dv):
                raise ValueError(f"{name} must be contiguous float32 [B,H,dk,dv]")
    if state_out is True:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    nbytes = int(lib.retention_chunkwise_workspace_bytes(B, H, N, dk, dv, int(chunk), dt))
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    rc = lib.retention_chunkwise(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), g, out.data_ptr(), B, H, N, dk, dv, int(chunk), dt,
        state_in.data_ptr() if state_in is not None else None,
        state_out.data_ptr() if state_out is not None else None,
        gn_p, ws_ptr, ws_bytes, _stream(q))
    if rc != 0:
        raise RetentionError("retention_chunkwise", rc)
    return out, state_out


def chunk_states(k, v, gamma: GammaLike, chunk: int, workspace, state_in=None, state_out=None):
    """First stage of the chunkwise form: the state carried into every chunk, kept in ``workspace``.

    ``workspace`` is a device uint8 tensor of at least chunkwise_workspace_bytes(...)
    bytes; ``state_out`` (optional fp32 [B,H,dk,dv]) receives the final state.
    """
    lib = _lib.load()
    B, H, N, dk, dv, dt = _check_qkv(k, k, v)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, dk, dv)):
            raise ValueError(f"{name} must be contiguous float32 [B,H,dk,dv]")
    g = _gamma_array(gamma, H)
    rc = lib.retention_chunk_states(
        k.data_ptr(), v.data_ptr(), g, B, H, N, dk, dv, int(chunk), dt,
        state_in.data_ptr() if state_in is not None else None,
        state_out.data_ptr() if state_out is not None else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(k))
    if rc != 0:
        raise RetentionError("retention_chunk_states", rc)
    return state_out


def chunk_output(q, k, v, gamma: GammaLike, chunk: int, workspace, has_state_in: bool = False,
                 gn: Optional[GroupNorm] = None, out=None, gate=None):
    """Second stage of the chunkwise form: O from q, k, v and the chunk states in ``workspace``.

    ``gate`` as in ``chunkwise``.
    """
    lib = _lib.load()
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    rc = lib.retention_chunk_output(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), g, out.data_ptr(), B, H, N, dk, dv, int(chunk), dt,
        1 if has_state_in else 0, gn_p, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(q))
    if rc != 0:
        raise RetentionError("retention_chunk_output", rc)
    return out


def recurrent_step(q, k, v, gamma: GammaLike, state, gn: Optional[GroupNorm] = None, out=None, gate=None):
    """One decode step: state <- gamma*state + k^T v (in place), returns o = q.state.

    q, k are [B,H,dk] (or [B,H,1,dk]); v is [B,H,dv] (or [B,H,1,dv]).
    ``gate`` (optional, needs ``gn``): B*H*dv values of the output's dtype;
    the result becomes GroupNorm(o) * swish(gate).
    """
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("state", state)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if state.dtype != torch.float32 or state.dim() != 4:
        raise ValueError("state must be float32 [B,H,dk,dv]")
    B, H, dk, dv = state.shape
    if q.numel() != B * H * dk or k.numel() != B * H * dk or v.numel() != B * H * dv:
        raise ValueError("q, k must hold B*H*dk and v B*H*dv elements")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    rc = lib.retention_recurrent_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, state.data_ptr(),
                                      out.data_ptr(), B, H, dk, dv, dt, gn_p, _stream(q))
    if rc != 0:
        raise RetentionError("retention_recurrent_step", rc)
    return out


def chunkwise_backward_workspace_bytes(B, H, N, dk, dv, chunk, dtype=torch.bfloat16) -> int:
    code = _lib.RET_BF16 if dtype == torch.bfloat16 else _lib.RET_F32
    return int(_lib.load().retention_chunkwise_backward_workspace_bytes(B, H, N, dk, dv, int(chunk), code))


def chunkwise_backward(q, k, v, grad_o, gamma: GammaLike, chunk: int, state_in=None, grad_state_out=None,
                       grad_state_in: Union[bool, torch.Tensor] = False, workspace=None, grads=None):
    """Gradients of the chunkwise form (no GroupNorm or gate) for dL/dO = grad_o.

    Returns (grad_q, grad_k, grad_v, grad_state_in or None). ``grad_state_out``
    is dL/dS_N (fp32 [B,H,dk,dv], None = 0); ``grad_state_in``: False (not
    produced), True (allocate) or an fp32 [B,H,dk,dv] tensor to fill.
    ``grads``: optional preallocated (grad_q, grad_k, grad_v).
    """
    lib = _lib.load()
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    if not grad_o.is_cuda or not grad_o.is_contiguous() or grad_o.dtype != q.dtype or grad_o.shape != v.shape:
        raise ValueError("grad_o must be a contiguous device tensor shaped and typed like v")
    for name, t in (("state_in", state_in), ("grad_state_out", grad_state_out), ("grad_state_in", grad_state_in)):
        if isinstance(t, torch.Tensor):
            if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, dk, dv):
                raise ValueError(f"{name} must be contiguous float32 [B,H,dk,dv]")
    if grad_state_in is True:
        grad_state_in = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif grad_state_in is False:
        grad_state_in = None
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    gq, gk, gv = grads
    nbytes = int(lib.retention_chunkwise_backward_workspace_bytes(B, H, N, dk, dv, int(chunk), dt))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    g = _gamma_array(gamma, H)
    rc = lib.retention_chunkwise_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), grad_o.data_ptr(), g, gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
        B, H, N, dk, dv, int(chunk), dt,
        state_in.data_ptr() if state_in is not None else None,
        grad_state_out.data_ptr() if grad_state_out is not None else None,
        grad_state_in.data_ptr() if grad_state_in is not None else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    if rc != 0:
        raise RetentionError("retention_chunkwise_backward", rc)
    return gq, gk, gv, grad_state_in

