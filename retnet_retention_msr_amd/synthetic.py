"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and casts them; it holds none of the
retention arithmetic, so both the HIP path and the CPU oracle can be fed the
same tensors from it.

Recipe: values are drawn in float32 on the CPU from ``torch.Generator`` with
a fixed seed, scaled, then cast to the requested dtype (bfloat16 casts round
to nearest even). Q and K are Gaussian with variance 1/sqrt(dk), so q.k has
unit variance; V is standard Gaussian. The decay of head h is the
multi-scale schedule gamma_h = 1 - 2^(-5-h) (0-based h), stored as float32;
it is exact in float32 for h <= 18.
"""

from __future__ import annotations

import torch


def head_gammas(H: int) -> torch.Tensor:
    """Per-head decays 1 - 2^(-5-h), h = 0..H-1, as a float32 CPU tensor."""
    return torch.tensor([1.0 - 2.0 ** (-5 - h) for h in range(H)], dtype=torch.float32)


def _randn(shape, gen, std=1.0):
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


def make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=0, qk_var=None, v_std=1.0):
    """Q, K [B,H,N,dk] and V [B,H,N,dv] on the CPU in ``dtype``.

    ``qk_var`` is the variance of Q and K (default 1/sqrt(dk)).
    """
    gen = torch.Generator().manual_seed(int(seed))
    var = (1.0 / dk ** 0.5) if qk_var is None else float(qk_var)
    std = var ** 0.5
    q = _randn((B, H, N, dk), gen, std).to(dtype)
    k = _randn((B, H, N, dk), gen, std).to(dtype)
    v = _randn((B, H, N, dv), gen, v_std).to(dtype)
    return q, k, v


def make_state(B, H, dk, dv, seed=0, std=1.0):
    """A float32 state [B,H,dk,dv] on the CPU."""
    gen = torch.Generator().manual_seed(int(seed))
    return _randn((B, H, dk, dv), gen, std)


def make_gn_affine(H, dv, seed=0):
    """GroupNorm weight and bias, float32 [H*dv] each, on the CPU."""
    gen = torch.Generator().manual_seed(int(seed))
    w = 1.0 + 0.25 * _randn((H * dv,), gen)
    b = 0.1 * _randn((H * dv,), gen)
    return w, b


def make_gate(shape, dtype=torch.bfloat16, seed=0, std=2.0):
    """Gate pre-activations of the given shape (like the output), N(0, std^2), on the CPU."""
    gen = torch.Generator().manual_seed(int(seed))
    return _randn(tuple(shape), gen, std).to(dtype)
