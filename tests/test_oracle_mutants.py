"""Plant plausible mistakes in copies of the oracle and check a pin catches each.

The mutants live here, on the CPU; the oracle itself is untouched. Each
mutant is one slip a reader could make when writing the forms from the pages
(a dropped decay term, an off-by-one exponent, a transposed mask or operand,
read-out before update). The pins are the brute-force double loop and the
hand-worked fixture.
"""

import numpy as np
import pytest

from oracle import retention_oracle as orc
from tests.test_oracle import _brute_parallel, _brute_state_one_based, _inputs


def _chunkwise_mutant(q, k, v, gamma, chunk, kind):
    B, H, N, _ = q.shape
    R = np.zeros((B, H, q.shape[-1], v.shape[-1]))
    out = np.empty((B, H, N, v.shape[-1]))
    for start in range(0, N, chunk):
        L = min(chunk, N - start)
        sl = slice(start, start + L)
        j = np.arange(L, dtype=np.float64)
        for h in range(H):
            g = gamma[h]
            D = orc.decay_mask(L, g)
            xi = g ** (j + 1.0)
            zeta = g ** (L - 1.0 - j)
            carry = g ** L
            if kind == "no_zeta":  # the carry exactly as printed, without in-chunk decay
                zeta = np.ones(L)
            elif kind == "xi_off_by_one":
                xi = g ** j
            elif kind == "mask_transposed":
                D = D.T
            elif kind == "carry_off_by_one":
                carry = g ** (L - 1)
            for b in range(B):
                Qi, Ki, Vi = q[b, h, sl], k[b, h, sl], v[b, h, sl]
                out[b, h, sl] = ((Qi @ Ki.T) * D) @ Vi + xi[:, None] * (Qi @ R[b, h])
                R[b, h] = carry * R[b, h] + Ki.T @ (zeta[:, None] * Vi)
    return out, R


def _recurrent_readout_first(q, k, v, gamma):
    B, H, N, dk = q.shape
    S = np.zeros((B, H, dk, v.shape[-1]))
    out = np.empty((B, H, N, v.shape[-1]))
    for n in range(N):
        out[:, :, n] = np.einsum("bhk,bhkv->bhv", q[:, :, n], S)
        S = gamma[None, :, None, None] * S + k[:, :, n, :, None] * v[:, :, n, None, :]
    return out, S


@pytest.mark.parametrize("kind", ["no_zeta", "xi_off_by_one", "mask_transposed", "carry_off_by_one"])
def test_chunkwise_mutants_are_caught(kind):
    q, k, v = _inputs(1, 2, 11, 3, 2, seed=7)
    g = np.array([0.9, 0.6])
    ref_o = _brute_parallel(q, k, v, g)
    ref_S = _brute_state_one_based(k, v, g)
    o, S = _chunkwise_mutant(q, k, v, g, 4, kind)
    caught = np.max(np.abs(o - ref_o)) > 1e-6 or np.max(np.abs(S - ref_S)) > 1e-6
    assert caught, kind
    # The unmutated copy of the same code passes, so the harness itself is sound.
    o0, S0 = _chunkwise_mutant(q, k, v, g, 4, "none")
    assert np.max(np.abs(o0 - ref_o)) < 1e-10 and np.max(np.abs(S0 - ref_S)) < 1e-10


def test_readout_before_update_is_caught():
    q, k, v = _inputs(1, 1, 6, 2, 2, seed=9)
    g = np.array([0.5])
    o, _ = _recurrent_readout_first(q, k, v, g)
    assert np.max(np.abs(o - _brute_parallel(q, k, v, g))) > 1e-6


def test_transposed_operand_is_caught():
    """Swapping K and V roles (dk != dv) cannot even run; swapping Q and K changes the result."""
    q, k, v = _inputs(1, 1, 8, 3, 3, seed=11)
    g = np.array([0.8])
    ref = _brute_parallel(q, k, v, g)
    swapped = orc.parallel(k, q, v, g)
    assert np.max(np.abs(swapped - ref)) > 1e-6


@pytest.mark.parametrize("kind", ["sign_flipped", "sigmoid_only", "gate_before_norm"])
def test_gate_mutants_are_caught(kind):
    """Slips in the gated epilogue: exp(+x) for exp(-x), sigmoid without the
    factor x, and the gate applied before the GroupNorm instead of after.
    The pin is the tanh form of the sigmoid times the library GroupNorm."""
    rng = np.random.default_rng(90)
    o = rng.standard_normal((1, 2, 4, 8)) * 2.0 + 0.3
    gate = rng.standard_normal((1, 2, 4, 8)) * 2.0
    pin = gate * 0.5 * (1.0 + np.tanh(0.5 * gate)) * orc.group_norm(o)
    if kind == "sign_flipped":
        y = gate / (1.0 + np.exp(gate)) * orc.group_norm(o)
    elif kind == "sigmoid_only":
        y = 1.0 / (1.0 + np.exp(-gate)) * orc.group_norm(o)
    else:
        y = orc.group_norm(orc.swish(gate) * o)
    assert np.max(np.abs(y - pin)) > 1e-6, kind
    np.testing.assert_allclose(orc.gated_group_norm(o, gate), pin, rtol=0, atol=1e-13)


def _backward_mutant(q, k, v, g, G, U, kind):
    """dQ, dK, dV with one planted slip (single head, no starting state)."""
    Q, K, V, G, U = q[0, 0], k[0, 0], v[0, 0], G[0, 0], U[0, 0]
    N = Q.shape[0]
    D = orc.decay_mask(N, g)
    zeta = g ** np.arange(N - 1, -1, -1, dtype=np.float64)
    if kind == "zeta_reversed":
        zeta = zeta[::-1]
    A = (Q @ K.T) * D
    dA = (G @ V.T) * (np.tril(np.ones((N, N))) if kind == "mask_without_decay" else D)
    dq = dA @ K
    dk = (dA @ Q if kind == "dA_not_transposed" else dA.T @ Q) + zeta[:, None] * (V @ U.T)
    dv = A.T @ G + zeta[:, None] * (K @ U)
    return dq, dk, dv


@pytest.mark.parametrize("kind", ["mask_without_decay", "dA_not_transposed", "zeta_reversed"])
def test_backward_mutants_are_caught(kind):
    """The pin: autograd through the token recurrence (as in test_oracle)."""
    import torch

    q, k, v = _inputs(1, 1, 7, 3, 3, seed=13)
    rng = np.random.default_rng(14)
    G, U = rng.standard_normal((1, 1, 7, 3)), rng.standard_normal((1, 1, 3, 3))
    g = 0.8
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    S = torch.zeros(1, 1, 3, 3, dtype=torch.float64)
    outs = []
    for n in range(7):
        S = g * S + tk[:, :, n, :, None] * tv[:, :, n, None, :]
        outs.append(torch.einsum("bhk,bhkv->bhv", tq[:, :, n], S))
    ((torch.stack(outs, 2) * torch.from_numpy(G)).sum() + (S * torch.from_numpy(U)).sum()).backward()
    ref = [t.grad.numpy()[0, 0] for t in (tq, tk, tv)]
    got = _backward_mutant(q, k, v, g, G, U, kind)
    assert max(np.max(np.abs(a - b)) for a, b in zip(got, ref)) > 1e-6, kind
    ok = _backward_mutant(q, k, v, g, G, U, "none")
    assert max(np.max(np.abs(a - b)) for a, b in zip(ok, ref)) < 1e-10
