"""Plain fp64 CPU oracle for Multi-Scale Retention (test infrastructure only).

This module is the checker, not the product. Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the HIP library and imports nothing from it.

Sources (the pages this follows; cited by tag below):
  [KR]  "RetNet - Retentive Network - A Successor to Transformer for LLMs"
        (irregular6612.github.io blog): Methods; Key components (1. Retention,
        2. Multi-Scale Retention); Key Equations (recurrent, parallel and
        chunkwise recurrent forms).
  [JP]  jisaku.com glossary entry on RetNet: the retention definition with the
        causal decay mask, and the three computation modes.
  [EN]  "What Is RetNet ? could it challenge the dominance of the Transformer ?"
        (medium.com, Publicis Sapient): "How is this dual representation
        achieved?" (the matrix D and the GroupNorm that follows it).
  [SP]  "RetNet入門" (Spiral.AI blog digest, news.ainew.jp): Multi-Scale
        Retention (MSR) (the normalised head outputs multiplied elementwise by
        a gated branch); the parallel representation (a conjugate in the
        retention product) and the remark on LEX Transformer (the
        intermediate expression of the derivation is xPos itself).

Conventions (readings where the pages are silent):
  * positions n, m and the head index h are 0-based;
  * shapes: q, k are [B, H, N, dk]; v is [B, H, N, dv]; a state is
    [B, H, dk, dv]; gamma is [H];
  * a recurrent step updates the state first and then reads it out, so token
    n sees itself with weight gamma^0 = 1;
  * the chunkwise form uses xi_j = gamma^(j+1) on the cross-chunk read-out and
    zeta_j = gamma^(L-1-j) inside the state update, for local row j of a chunk
    of length L; these are the only factors that make it equal the recurrence.

Every function widens its inputs to float64 and runs in float64. Nothing here
is blocked, fused or reordered beyond what the cited definition states.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    """Exact widening of a numpy array or CPU torch tensor to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _zero_state(q, v):
    B, H, _, dk = q.shape
    dv = v.shape[-1]
    return np.zeros((B, H, dk, dv), dtype=np.float64)


def decay_mask(N, gamma):
    """The N x N causal decay matrix of one head.

    [KR] Key Equations, parallel form; [JP] retention definition:
    D[n, m] = gamma^(n - m) for n >= m and 0 for n < m. With gamma = 0 the
    diagonal stays 1 (0^0 = 1), so the gamma -> 0 limit is well defined.
    """
    n = np.arange(N)[:, None]
    m = np.arange(N)[None, :]
    diff = n - m
    g = float(gamma)
    out = np.where(diff >= 0, np.power(g, np.maximum(diff, 0).astype(np.float64)), 0.0)
    return out


def parallel(q, k, v, gamma, state_in=None):
    """Parallel form, O = (Q K^T * D) V per head.

    [KR] Key Equations, parallel form; [JP] retention definition and the
    parallel mode. Multi-Scale Retention runs this independently per head h
    with that head's own gamma_h ([KR] Key components, 2. Multi-Scale
    Retention).

    When ``state_in`` S0 is given the output also carries the contribution of
    the history summarised by S0: the recurrence unrolled from S_{-1} = S0
    adds gamma^(n+1) q_n S0 to row n. The parallel form on the pages has no
    state; this term only exists so the three forms can be compared with a
    starting state.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _f64(gamma)
    B, H, N, _ = q.shape
    out = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    S0 = None if state_in is None else _f64(state_in)
    for h in range(H):
        D = decay_mask(N, g[h])
        for b in range(B):
            scores = (q[b, h] @ k[b, h].T) * D
            out[b, h] = scores @ v[b, h]
            if S0 is not None:
                xi = np.power(g[h], np.arange(1, N + 1, dtype=np.float64))
                out[b, h] += xi[:, None] * (q[b, h] @ S0[b, h])
    return out


def parallel_rows(q, k, v, gamma, rows, state_in=None):
    """Selected output rows of the parallel form, one row at a time.

    Row n of [KR] Key Equations, parallel form, written as the sum it is:
    o_n = sum_{m <= n} gamma^(n-m) (q_n . k_m) v_m  (+ gamma^(n+1) q_n S0).
    Used to sample outputs at sizes where the full N x N product is too big.
    Returns an array [B, H, len(rows), dv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _f64(gamma)
    B, H, N, _ = q.shape
    rows = [int(r) for r in rows]
    out = np.empty((B, H, len(rows), v.shape[-1]), dtype=np.float64)
    S0 = None if state_in is None else _f64(state_in)
    for i, n in enumerate(rows):
        for h in range(H):
            w = np.power(g[h], np.arange(n, -1, -1, dtype=np.float64))  # gamma^(n-m), m=0..n
            for b in range(B):
                s = (k[b, h, : n + 1] @ q[b, h, n]) * w
                out[b, h, i] = s @ v[b, h, : n + 1]
                if S0 is not None:
                    out[b, h, i] += (g[h] ** (n + 1)) * (q[b, h, n] @ S0[b, h])
    return out


def recurrent_step(q, k, v, gamma, state):
    """One token of the recurrent form.

    [KR] Methods and Key Equations, recurrent form; [JP] recurrent mode:
    S_n = gamma * S_{n-1} + k_n^T v_n (a dk x dv outer product), then
    o_n = q_n S_n. Shapes: q, k [B, H, dk]; v [B, H, dv]; state [B, H, dk, dv].
    Returns (o [B, H, dv], new state).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _f64(gamma)
    S = _f64(state)
    S_new = g[None, :, None, None] * S + k[..., :, None] * v[..., None, :]
    o = np.einsum("bhk,bhkv->bhv", q, S_new)
    return o, S_new


def recurrent(q, k, v, gamma, state_in=None):
    """Recurrent form over a whole sequence, token by token.

    [KR] Key Equations, recurrent form, iterated from S_{-1} = state_in
    (zeros when absent). Returns (o [B, H, N, dv], S_{N-1}).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N = q.shape[2]
    S = _zero_state(q, v) if state_in is None else _f64(state_in).copy()
    out = np.empty(q.shape[:3] + (v.shape[-1],), dtype=np.float64)
    for n in range(N):
        out[:, :, n], S = recurrent_step(q[:, :, n], k[:, :, n], v[:, :, n], gamma, S)
    return out, S


def chunkwise(q, k, v, gamma, chunk, state_in=None):
    """Chunkwise recurrent form: parallel inside a chunk, recurrent across.

    [KR] Key Equations, chunkwise recurrent form (inner parallel term plus the
    cross-chunk term (Q_[i] * xi) R_{i-1}) and Key components, 1. Retention
    (the chunk-state carry); [JP] chunkwise mode.

    For chunk i with rows [i*C, i*C + L) and local row j:
      O_[i] = (Q_[i] K_[i]^T * D_L) V_[i] + diag(xi) Q_[i] R_{i-1},
      R_i   = gamma^L R_{i-1} + K_[i]^T diag(zeta) V_[i],
    with xi_j = gamma^(j+1), zeta_j = gamma^(L-1-j), R_{-1} = state_in (or 0).
    The carry printed on the page lacks the in-chunk factor zeta; taken
    literally it would break the equality with the recurrence that the same
    page asserts, so zeta is included.
    Returns (o [B, H, N, dv], R_last).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _f64(gamma)
    B, H, N, _ = q.shape
    C = int(chunk)
    if C < 1:
        raise ValueError("chunk must be >= 1")
    R = _zero_state(q, v) if state_in is None else _f64(state_in).copy()
    out = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    for start in range(0, N, C):
        L = min(C, N - start)
        sl = slice(start, start + L)
        j = np.arange(L, dtype=np.float64)
        for h in range(H):
            D = decay_mask(L, g[h])
            xi = np.power(g[h], j + 1.0)
            zeta = np.power(g[h], (L - 1.0) - j)
            carry = g[h] ** L
            for b in range(B):
                Qi, Ki, Vi = q[b, h, sl], k[b, h, sl], v[b, h, sl]
                inner = ((Qi @ Ki.T) * D) @ Vi
                cross = xi[:, None] * (Qi @ R[b, h])
                out[b, h, sl] = inner + cross
                R[b, h] = carry * R[b, h] + Ki.T @ (zeta[:, None] * Vi)
    return out, R


def state_after(k, v, gamma, state_in=None):
    """State after all N tokens, the recurrence unrolled in closed form.

    Unrolling [KR] Key Equations, recurrent form, from S_{-1} = S0 gives
    S_{N-1} = gamma^N S0 + sum_m gamma^(N-1-m) k_m^T v_m.
    """
    k, v = _f64(k), _f64(v)
    g = _f64(gamma)
    B, H, N, dk = k.shape
    S = np.empty((B, H, dk, v.shape[-1]), dtype=np.float64)
    for h in range(H):
        w = np.power(g[h], np.arange(N - 1, -1, -1, dtype=np.float64))
        for b in range(B):
            S[b, h] = k[b, h].T @ (w[:, None] * v[b, h])
            if state_in is not None:
                S[b, h] += (g[h] ** N) * _f64(state_in)[b, h]
    return S


def backward(q, k, v, gamma, d_o, state_in=None, d_state_out=None):
    """Gradients of retention with respect to q, k, v and the starting state.

    The forward map is the parallel form with a starting state S0 ([KR] Key
    Equations, parallel form; the state term as in ``parallel``) together
    with the state it leaves behind (``state_after``):
        O   = (Q K^T * D) V + diag(xi) Q S0,         xi_n   = gamma^(n+1)
        S_N = K^T diag(zeta) V + gamma^N S0,          zeta_m = gamma^(N-1-m)
    The pages name training as the purpose of the parallel and chunkwise forms
    but print no gradients; these are the derivatives of the two maps above,
    given d_o = dL/dO and d_state_out = dL/dS_N (None = 0). With A = Q K^T * D
    and dA = (d_o V^T) * D:
        dV  = A^T d_o + diag(zeta) K dS_N
        dQ  = dA K + diag(xi) d_o S0^T
        dK  = dA^T Q + diag(zeta) V dS_N^T
        dS0 = Q^T diag(xi) d_o + gamma^N dS_N
    Returns (dq, dk, dv, d_state_in); d_state_in is None when state_in is None
    and d_state_out is None.
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    g = _f64(gamma)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S0 = None if state_in is None else _f64(state_in)
    dSN = None if d_state_out is None else _f64(d_state_out)
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    want_ds0 = S0 is not None or dSN is not None
    dS0 = np.zeros((B, H, dk, dv)) if want_ds0 else None
    for h in range(H):
        D = decay_mask(N, g[h])
        xi = np.power(g[h], np.arange(1, N + 1, dtype=np.float64))
        zeta = np.power(g[h], np.arange(N - 1, -1, -1, dtype=np.float64))
        for b in range(B):
            Q, K, V, G = q[b, h], k[b, h], v[b, h], d_o[b, h]
            A = (Q @ K.T) * D
            dA = (G @ V.T) * D
            dv_[b, h] = A.T @ G
            dq[b, h] = dA @ K
            dk_[b, h] = dA.T @ Q
            if S0 is not None:
                dq[b, h] += xi[:, None] * (G @ S0[b, h].T)
            if dSN is not None:
                dv_[b, h] += zeta[:, None] * (K @ dSN[b, h])
                dk_[b, h] += zeta[:, None] * (V @ dSN[b, h].T)
            if want_ds0:
                dS0[b, h] = Q.T @ (xi[:, None] * G)
                if dSN is not None:
                    dS0[b, h] += (g[h] ** N) * dSN[b, h]
    return dq, dk_, dv_, dS0


def backward_rows(q, k, v, gamma, d_o, rows, state_in=None, d_state_out=None):
    """Rows of the gradients of ``backward``, each row on its own (for sampled
    checks on long sequences). Same maps and result as ``backward``, written
    per token: for a row n of dQ and a row m of dK and dV,
        dQ_n = sum_{m<=n} gamma^(n-m) (dO_n . v_m) k_m + gamma^(n+1) dO_n S0^T
        dK_m = sum_{n>=m} gamma^(n-m) (dO_n . v_m) q_n + gamma^(N-1-m) v_m dS_N^T
        dV_m = sum_{n>=m} gamma^(n-m) (q_n . k_m) dO_n + gamma^(N-1-m) k_m dS_N
    Returns (dq, dk, dv) of shape [B, H, len(rows), d].
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    g = _f64(gamma)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    rows = [int(r) for r in rows]
    S0 = None if state_in is None else _f64(state_in)
    dSN = None if d_state_out is None else _f64(d_state_out)
    R = len(rows)
    dq, dk_, dv_ = np.zeros((B, H, R, dk)), np.zeros((B, H, R, dk)), np.zeros((B, H, R, dv))
    for h in range(H):
        for b in range(B):
            Q, K, V, G = q[b, h], k[b, h], v[b, h], d_o[b, h]
            for i, n in enumerate(rows):
                m = np.arange(n + 1)
                w = np.power(g[h], (n - m).astype(np.float64)) * (V[: n + 1] @ G[n])
                dq[b, h, i] = w @ K[: n + 1]
                if S0 is not None:
                    dq[b, h, i] += g[h] ** (n + 1) * (S0[b, h] @ G[n])
                later = np.arange(n, N)
                decay = np.power(g[h], (later - n).astype(np.float64))
                dk_[b, h, i] = (decay * (G[n:] @ V[n])) @ Q[n:]
                dv_[b, h, i] = (decay * (Q[n:] @ K[n])) @ G[n:]
                if dSN is not None:
                    z = g[h] ** (N - 1 - n)
                    dk_[b, h, i] += z * (dSN[b, h] @ V[n])
                    dv_[b, h, i] += z * (K[n] @ dSN[b, h])
    return dq, dk_, dv_


def group_norm(o, eps=1e-5, weight=None, bias=None):
    """Per-head GroupNorm applied to retention outputs.

    [KR] Methods (block: MSR, then GroupNorm) and Key components, 4. block;
    [EN] "How is this dual representation achieved?" (a GroupNorm after the
    retention product). One group per head: for each (b, h, n) the mean and
    the biased variance are taken over that head's dv outputs, then
    y = (o - mean) / sqrt(var + eps) * weight[h] + bias[h]. ``weight`` and
    ``bias`` are [H, dv] (or flat [H*dv]); absent means identity.
    """
    o = _f64(o)
    H, dv = o.shape[1], o.shape[-1]
    mu = o.mean(axis=-1, keepdims=True)
    var = ((o - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (o - mu) / np.sqrt(var + float(eps))
    if weight is not None:
        y = y * _f64(weight).reshape(1, H, 1, dv)
    if bias is not None:
        y = y + _f64(bias).reshape(1, H, 1, dv)
    return y


def group_norm_rows(o_rows, eps=1e-5, weight=None, bias=None):
    """GroupNorm of sampled rows [B, H, R, dv]; same definition as group_norm."""
    return group_norm(o_rows, eps, weight, bias)


def swish(x):
    """swish(x) = x * sigmoid(x) = x / (1 + exp(-x)), elementwise.

    [KR] Key components, 4. block names a swish gate after the GroupNorm; the
    pages do not define swish, and this is its usual definition (also called
    SiLU). Written so that no exp overflows: for x < 0 it uses
    x * e^x / (1 + e^x).
    """
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, x / (1.0 + e), x * e / (1.0 + e))


def gated_group_norm(o, gate, eps=1e-5, weight=None, bias=None):
    """The gated epilogue: swish(gate) * GroupNorm(o), elementwise.

    [KR] Key components, 4. block (GroupNorm with swish gating); [SP]
    Multi-Scale Retention (MSR) (the normalised head outputs times the gated
    branch, before the output projection, which is not part of this). ``gate``
    is the gate branch's pre-activation for these outputs, in o's layout
    [B, H, N, dv] (head h's dv channels of it).
    """
    return swish(gate) * group_norm(o, eps, weight, bias)


def xpos_rotate(x, theta, pos0=0):
    """The rotation of the xPos relative position encoding, applied to Q or K.

    [KR] Methods (block structure: xPos applied to Q and K), Key components,
    3. xPos (a complex rotation that injects relative position into Q and K),
    and the glossary at its end (xPos couples the rotation with a decay);
    [SP] the parallel representation (a conjugate in the retention product)
    and the remark on LEX Transformer. The pages give no formula; the reading
    here: the d features of a token form d/2 complex numbers
    z_i = x[2i] + 1j * x[2i+1], and the token at position n = pos0 + (its
    index along the sequence) has z_i multiplied by exp(1j * n * theta_i).
    Rotating Q and K alike and taking the real dot product gives
    Re(sum_i zq_i * conj(zk_i) * exp(1j * (n - m) * theta_i)): the conjugate
    form, a function of n - m only. The decay half of xPos is the retention's
    own gamma^(n - m) (the matrix D), so no decay is applied here.

    x is [..., N, d] with d even, theta is [d/2]; returns float64 of x's shape.
    """
    x = _f64(x)
    theta = _f64(theta)
    d = x.shape[-1]
    if d % 2 or theta.shape != (d // 2,):
        raise ValueError("x must have an even last axis d and theta d/2 entries")
    N = x.shape[-2]
    n = float(pos0) + np.arange(N, dtype=np.float64)
    angle = n[:, None] * theta[None, :]  # [N, d/2]
    c, s = np.cos(angle), np.sin(angle)
    re, im = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = re * c - im * s
    y[..., 1::2] = re * s + im * c
    return y
