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
    "chunkwise_noalloc",
    "chunk_states",
    "chunk_output",
    "recurrent_step",
    "xpos_rotate",
    "xpos_theta",
    "chunkwise_workspace_bytes",
    "chunk_stages_workspace_bytes",
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


def _require(t, name, shape, dtype, device):
    """Raise ValueError unless ``t`` is a contiguous tensor of exactly this shape
    and dtype on ``device``. Every pointer handed to the C ABI passes through
    here (or _check_qkv) first: the library cannot tell a host pointer or a
    short buffer from a valid one."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (the inputs' device), not {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _require_workspace(ws, name, nbytes, device):
    """A device byte buffer of at least ``nbytes`` bytes (contiguous)."""
    if not isinstance(ws, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if ws.device != device:
        raise ValueError(f"{name} must be on {device} (the inputs' device), not {ws.device}")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = ws.numel() * ws.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, {nbytes} are needed")
    return ws


def _no_overlap(out, name, *inputs):
    """``out`` must not share memory with any of ``inputs``."""
    lo = out.data_ptr()
    hi = lo + out.numel() * out.element_size()
    for t in inputs:
        if t is None:
            continue
        a = t.data_ptr()
        b = a + t.numel() * t.element_size()
        if lo < b and a < hi:
            raise ValueError(f"{name} must not overlap an input")


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B,H,N,dk] and v [B,H,N,dv]")
    B, H, N, dk = q.shape
    return B, H, N, dk, v.shape[3], _dtype_code(q)


def _output(out, q, shape):
    """The output tensor: allocated like q when None, else checked and kept apart from the inputs."""
    if out is None:
        return torch.empty(shape, dtype=q.dtype, device=q.device)
    return _require(out, "out", shape, q.dtype, q.device)


def _state(t, name, B, H, dk, dv, device):
    return None if t is None else _require(t, name, (B, H, dk, dv), torch.float32, device)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def parallel(q, k, v, gamma: GammaLike, gn: Optional[GroupNorm] = None, out=None, gate=None):
    """Parallel form O = (Q K^T * D) V per head (optionally GroupNorm-ed).

    ``gate`` (optional, needs ``gn``): a tensor like the output; the result
    becomes GroupNorm(O) * swish(gate).
    """
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    out = _output(out, q, (B, H, N, dv))
    _no_overlap(out, "out", q, k, v)
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    lib = _lib.load()
    rc = lib.retention_parallel(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, out.data_ptr(), B, H, N, dk, dv, dt,
                                gn_p, _stream(q))
    if rc != 0:
        raise RetentionError("retention_parallel", rc)
    return out


def chunkwise_workspace_bytes(B, H, N, dk, dv, chunk, dtype=torch.bfloat16) -> int:
    code = _lib.RET_BF16 if dtype == torch.bfloat16 else _lib.RET_F32
    return int(_lib.load().retention_chunkwise_workspace_bytes(B, H, N, dk, dv, int(chunk), code))


def chunk_stages_workspace_bytes(B, H, N, dk, dv, chunk, dtype=torch.bfloat16) -> int:
    """Workspace bytes of chunk_states / chunk_output (the state of every chunk)."""
    code = _lib.RET_BF16 if dtype == torch.bfloat16 else _lib.RET_F32
    return int(_lib.load().retention_chunk_stages_workspace_bytes(B, H, N, dk, dv, int(chunk), code))


def chunkwise(q, k, v, gamma: GammaLike, chunk: int, state_in=None, state_out: Union[bool, torch.Tensor] = False,
              gn: Optional[GroupNorm] = None, out=None, workspace=None, gate=None):
    """Chunkwise recurrent form. Returns (o, state_out or None).

    ``state_out``: False (not produced), True (allocate), or an fp32
    [B,H,dk,dv] tensor to fill (it may be ``state_in`` itself). ``gate``
    (optional, needs ``gn``): a tensor like the output; the result becomes
    GroupNorm(O) * swish(gate).
    """
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    out = _output(out, q, (B, H, N, dv))
    _no_overlap(out, "out", q, k, v)
    state_in = _state(state_in, "state_in", B, H, dk, dv, q.device)
    if state_out is True:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif state_out is False or state_out is None:
        state_out = None
    else:
        _state(state_out, "state_out", B, H, dk, dv, q.device)
    lib = _lib.load()
    nbytes = int(lib.retention_chunkwise_workspace_bytes(B, H, N, dk, dv, int(chunk), dt))
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif workspace is not None:
        _require_workspace(workspace, "workspace", nbytes, q.device)
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


def chunkwise_noalloc(q, k, v, gamma: GammaLike, chunk: int, out, state_in=None, state_out=None,
                      gn: Optional[GroupNorm] = None, gate=None):
    """retention_chunkwise_noalloc: the chunkwise form with the library's own
    device scratch as workspace, for callers that cannot allocate (nothing is
    allocated here either: ``out`` and ``state_out``, if wanted, are the
    caller's). Returns ``out``. Raises RetentionError (RET_ERR_UNSUPPORTED)
    when the sizes need more workspace than the scratch holds
    (NOALLOC_MAX_WORKSPACE_BYTES). Calls that overlap in time on one GPU race
    on the shared scratch.
    """
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    _require(out, "out", (B, H, N, dv), q.dtype, q.device)
    _no_overlap(out, "out", q, k, v)
    state_in = _state(state_in, "state_in", B, H, dk, dv, q.device)
    state_out = _state(state_out, "state_out", B, H, dk, dv, q.device)
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    lib = _lib.load()
    rc = lib.retention_chunkwise_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), g, out.data_ptr(), B, H, N, dk, dv, int(chunk), dt,
        state_in.data_ptr() if state_in is not None else None,
        state_out.data_ptr() if state_out is not None else None, gn_p, _stream(q))
    if rc != 0:
        raise RetentionError("retention_chunkwise_noalloc", rc)
    return out


def chunk_states(k, v, gamma: GammaLike, chunk: int, workspace, state_in=None, state_out=None):
    """First stage of the chunkwise form: the state carried into every chunk, kept in ``workspace``.

    ``workspace`` is a device uint8 tensor of at least chunk_stages_workspace_bytes(...)
    bytes; ``state_out`` (optional fp32 [B,H,dk,dv]) receives the final state.
    """
    B, H, N, dk, dv, dt = _check_qkv(k, k, v)
    state_in = _state(state_in, "state_in", B, H, dk, dv, k.device)
    state_out = _state(state_out, "state_out", B, H, dk, dv, k.device)
    lib = _lib.load()
    _require_workspace(workspace, "workspace",
                       int(lib.retention_chunk_stages_workspace_bytes(B, H, N, dk, dv, int(chunk), dt)), k.device)
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
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    out = _output(out, q, (B, H, N, dv))
    _no_overlap(out, "out", q, k, v, workspace)
    lib = _lib.load()
    _require_workspace(workspace, "workspace",
                       int(lib.retention_chunk_stages_workspace_bytes(B, H, N, dk, dv, int(chunk), dt)), q.device)
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
    for name, t in (("q", q), ("k", k), ("v", v), ("state", state)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.device != state.device:
            raise ValueError(f"{name} must be on the state's device {state.device}")
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
    elif not isinstance(out, torch.Tensor) or out.numel() != B * H * dv:
        raise ValueError(f"out must hold B*H*dv = {B * H * dv} elements")
    else:
        _require(out, "out", tuple(out.shape), q.dtype, q.device)
    _no_overlap(out, "out", q, k, v, state)
    lib = _lib.load()
    g = _gamma_array(gamma, H)
    gn_p, _keep = _gn_struct(gn, H, dv, q.device, gate, out)
    rc = lib.retention_recurrent_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, state.data_ptr(),
                                      out.data_ptr(), B, H, dk, dv, dt, gn_p, _stream(q))
    if rc != 0:
        raise RetentionError("retention_recurrent_step", rc)
    return out


def xpos_theta(d: int, base: float = 10000.0) -> torch.Tensor:
    """Angles per position for the d/2 feature pairs: theta_i = base^(-2i/d),
    i = 0 .. d/2 - 1 (float32, CPU). The pages give no schedule for the xPos
    rotation; this geometric one (fast turns on the first pairs, slow on the
    last) is a default reading, and any other may be passed to xpos_rotate."""
    if d <= 0 or d % 2:
        raise ValueError("d must be a positive even number")
    i = torch.arange(d // 2, dtype=torch.float64)
    return (float(base) ** (-2.0 * i / d)).to(torch.float32)


def xpos_rotate(q, k=None, theta=None, pos0: int = 0, out_q=None, out_k=None):
    """xPos rotation of q (and k): pair i of the features at position
    pos0 + n is multiplied, as a complex number, by exp(1j (pos0 + n) theta_i).

    q, k are [B, H, N, d] device tensors of one dtype (bf16 or fp32); theta is
    d/2 angles (default ``xpos_theta(d)``). out_q / out_k may be q / k (in
    place); by default new tensors are returned. Returns (q_rot, k_rot), k_rot
    None when k is None. A decode step passes its token's position as pos0.
    """
    if not isinstance(q, torch.Tensor) or not q.is_cuda or q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B,H,N,d] device tensor")
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    if k is not None:
        _require(k, "k", (B, H, N, d), q.dtype, q.device)
    if theta is None:
        theta = xpos_theta(d)
    th = torch.as_tensor(theta, dtype=torch.float32).detach().to("cpu").contiguous()
    if th.numel() != d // 2:
        raise ValueError(f"theta has {th.numel()} entries, expected d/2 = {d // 2}")
    arr = (ctypes.c_float * (d // 2))(*th.tolist())
    if out_q is None:
        out_q = torch.empty_like(q)
    else:
        _require(out_q, "out_q", (B, H, N, d), q.dtype, q.device)
    if k is None:
        if out_k is not None:
            raise ValueError("out_k needs k")
    elif out_k is None:
        out_k = torch.empty_like(k)
    else:
        _require(out_k, "out_k", (B, H, N, d), q.dtype, q.device)
    # Outputs are their own inputs or apart from every other buffer.
    if out_q.data_ptr() != q.data_ptr():
        _no_overlap(out_q, "out_q", q, k)
    if k is not None:
        if out_k.data_ptr() != k.data_ptr():
            _no_overlap(out_k, "out_k", q, k)
        _no_overlap(out_k, "out_k", out_q)
    lib = _lib.load()
    rc = lib.retention_xpos_rotate(q.data_ptr(), None if k is None else k.data_ptr(), out_q.data_ptr(),
                                   None if k is None else out_k.data_ptr(), arr, B, H, N, d, int(pos0), dt,
                                   _stream(q))
    if rc != 0:
        raise RetentionError("retention_xpos_rotate", rc)
    return out_q, out_k


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
    B, H, N, dk, dv, dt = _check_qkv(q, k, v)
    _require(grad_o, "grad_o", tuple(v.shape), q.dtype, q.device)
    state_in = _state(state_in, "state_in", B, H, dk, dv, q.device)
    grad_state_out = _state(grad_state_out, "grad_state_out", B, H, dk, dv, q.device)
    if grad_state_in is True:
        grad_state_in = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif grad_state_in is False or grad_state_in is None:
        grad_state_in = None
    else:
        _state(grad_state_in, "grad_state_in", B, H, dk, dv, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    if len(grads) != 3:
        raise ValueError("grads must be (grad_q, grad_k, grad_v)")
    gq, gk, gv = grads
    for name, t, shape in (("grad_q", gq, q.shape), ("grad_k", gk, k.shape), ("grad_v", gv, v.shape)):
        _require(t, name, tuple(shape), q.dtype, q.device)
        _no_overlap(t, name, q, k, v, grad_o, state_in, grad_state_out)
    lib = _lib.load()
    nbytes = int(lib.retention_chunkwise_backward_workspace_bytes(B, H, N, dk, dv, int(chunk), dt))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _require_workspace(workspace, "workspace", nbytes, q.device)
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

